// Split-K reduction: the add reduction of the cp.async.bulk.tensor page
// ("Stores, reductions, and completion") applied to the partial sums of the
// tiled kernel's K splits. The destination starts at its intended value (C,
// or the scalar) and each split's partial sum is added to it in K order, one
// rounding per add, so the result does not depend on how the splits were
// scheduled. Fused into one pass: each output is read from C and from every
// partial once and written once (HBM bound: (splits + 2) x 4 bytes per
// output with a C tensor).
#include "common.h"
#include "launch.h"

namespace bmm {
namespace {

constexpr int kReduceThreads = 256;

template <bool kHasC>
__global__ __launch_bounds__(kReduceThreads) void splitk_reduce_kernel(
    float* D, const float* C, float c, const float* __restrict__ parts,
    int splits, int64_t part_floats, int64_t n4) {
  const int64_t stride = int64_t(gridDim.x) * kReduceThreads;
  for (int64_t i = int64_t(blockIdx.x) * kReduceThreads + threadIdx.x; i < n4; i += stride) {
    f32x4 acc = kHasC ? load16f(C + 4 * i) : f32x4{c, c, c, c};
    for (int s = 0; s < splits; ++s) {
      const f32x4 v = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4*>(parts + s * part_floats + 4 * i));
      acc += v;
    }
    store16f(D + 4 * i, acc);
  }
}

}  // namespace

hipError_t launch_splitk_reduce(float* D, const float* C, float c, const float* parts,
                                int splits, int64_t part_floats, int64_t n4, hipStream_t s) {
  // enough workgroups to fill the chip several times over; grid-stride beyond
  int64_t blocks = (n4 + kReduceThreads - 1) / kReduceThreads;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) return hipSuccess;
  if (C)
    hipLaunchKernelGGL(splitk_reduce_kernel<true>, dim3(unsigned(blocks)), dim3(kReduceThreads),
                       0, s, D, C, c, parts, splits, part_floats, n4);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<false>, dim3(unsigned(blocks)), dim3(kReduceThreads),
                       0, s, D, C, c, parts, splits, part_floats, n4);
  return hipGetLastError();
}

}  // namespace bmm
