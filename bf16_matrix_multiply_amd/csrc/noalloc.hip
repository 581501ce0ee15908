// The split-K multiply-accumulate for callers that cannot allocate device
// memory (code under graph capture, tight serving loops, harnesses that forbid
// hipMalloc): the partial sums live in a file-scope device array instead of a
// caller workspace. Arithmetic, kernels and validation are those of
// bmm_mma_tile_splitk (add reduction of the cp.async.bulk.tensor page,
// "Stores, reductions, and completion", applied to the K splits).
//
// Every GPU the library runs on holds its own copy of the array, from the
// first call on that device until the process ends. Calls on one device share
// it: calls that overlap in time on one device (two streams, two threads)
// race on the partial sums. Nothing in it must start at zero: each split
// writes every element of its partial sum before the reduce reads it.
#include <mutex>
#include <string>

#include "launch.h"
#include "validate.h"

namespace {

constexpr int64_t kScratchBytes = BMM_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// Device-side storage. In host code this name is only a stand-in for the
// symbol: its device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the array's copy on the device that runs `stream`
// (the current device for the null stream), looked up once per device with
// that device current, and kept.
hipError_t scratch_for_stream(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const int current = dev;
  if (stream) {
    hipDevice_t sd = -1;
    e = hipStreamGetDevice(stream, &sd);
    if (e != hipSuccess) return e;
    dev = int(sd);
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != current && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != current) {
      const hipError_t r = hipSetDevice(current);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int bmm_mma_tile_splitk_noalloc(float* D, const uint32_t* A, const uint32_t* B, const float* C,
                                float c_scalar, int64_t batch, int64_t M_rep, int64_t N_rep,
                                int64_t K_rep, bmm_dtype dtype, int32_t atom_k, int32_t splits,
                                void* stream) {
  const int64_t need =
      bmm_mma_splitk_workspace_bytes(batch, M_rep, N_rep, K_rep, atom_k, splits);
  // Invalid extents, atom K or split count: the regular validation rejects
  // them (naming the field) before any launch; an empty problem is a no-op.
  if (need < 0)
    return bmm_mma_tile_splitk(D, A, B, C, c_scalar, batch, M_rep, N_rep, K_rep, dtype, atom_k,
                               splits, nullptr, 0, stream);
  if (need > kScratchBytes) {
    bmm::set_last_error("mma_tile_splitk_noalloc: " + std::to_string(splits) +
                        " partial sums need " + std::to_string(need) +
                        " bytes of scratch; the static scratch holds " +
                        std::to_string(kScratchBytes) +
                        " (use fewer splits, or bmm_mma_tile_splitk with a workspace)");
    return BMM_ERANGE;
  }
  void* ws = nullptr;
  const hipError_t e = scratch_for_stream(static_cast<hipStream_t>(stream), &ws);
  if (e != hipSuccess) {
    bmm::set_last_error(std::string("mma_tile_splitk_noalloc: scratch address: ") +
                        hipGetErrorString(e));
    return BMM_EHIP;
  }
  return bmm_mma_tile_splitk(D, A, B, C, c_scalar, batch, M_rep, N_rep, K_rep, dtype, atom_k,
                             splits, static_cast<float*>(ws), kScratchBytes, stream);
}

}  // extern "C"
