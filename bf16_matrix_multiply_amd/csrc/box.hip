// Box copy through an LDS image: the role of the TMA tile-mode box load of the
// cp.async.bulk.tensor page ("Operands and descriptor fields", "Example: two
// explicit 8x16 boxes"), done the CDNA4 way. One workgroup stages one repeat:
// its lanes read the box from global memory with consecutive lanes on
// consecutive innermost elements (coalesced), substitute zero outside the
// tensor, and write the LDS image in the requested XOR-swizzled layout; after a
// barrier they read the image back through the same swizzle and store it
// compact and unswizzled.
#include "common.h"
#include "launch.h"

namespace bmm {
namespace {

constexpr int kBoxThreads = 256;

// Swizzle of an LDS byte offset: mode s in 1..3 XORs the 16-byte chunk bits
// [4, 4+s) with the 128-byte row bits [7, 7+s); mode 0 is the identity. Each
// offset stays inside its own 128-byte row, and the map is an involution.
__device__ __forceinline__ uint32_t swizzle_offset(uint32_t off, int mode) {
  const uint32_t mask = (1u << mode) - 1u;
  return off ^ (((off >> 7) & mask) << 4);
}

struct BoxParams {
  int32_t rank, eb, swizzle, pad;
  int64_t dims[5], strides[5], coords[5], step[5];
  int32_t box[5];
  int32_t box_elems;
};

template <typename T>
__device__ __forceinline__ void copy_in(const char* src, char* lds, const BoxParams& p,
                                        int64_t t) {
  for (int32_t e = threadIdx.x; e < p.box_elems; e += kBoxThreads) {
    int32_t rem = e;
    bool inside = true;
    int64_t off = 0;
    for (int d = p.rank - 1; d >= 0; --d) {
      const int32_t j = rem % p.box[d];
      rem /= p.box[d];
      const int64_t g = p.coords[d] + t * p.step[d] + j;
      inside = inside && g >= 0 && g < p.dims[d];
      off += g * p.strides[d];
    }
    const T v = inside ? *reinterpret_cast<const T*>(src + off) : T(0);
    *reinterpret_cast<T*>(lds + swizzle_offset(uint32_t(e) * sizeof(T), p.swizzle)) = v;
  }
}

template <typename T>
__device__ __forceinline__ void copy_out(char* dst, const char* lds, const BoxParams& p,
                                         int64_t t) {
  T* out = reinterpret_cast<T*>(dst) + t * p.box_elems;
  for (int32_t e = threadIdx.x; e < p.box_elems; e += kBoxThreads)
    out[e] = *reinterpret_cast<const T*>(lds + swizzle_offset(uint32_t(e) * sizeof(T), p.swizzle));
}

__global__ __launch_bounds__(kBoxThreads) void box_kernel(char* __restrict__ dst,
                                                          const char* __restrict__ src,
                                                          BoxParams p) {
  extern __shared__ __attribute__((aligned(128))) char lds[];
  const int64_t t = blockIdx.x;
  switch (p.eb) {
    case 1: copy_in<uint8_t>(src, lds, p, t); break;
    case 2: copy_in<uint16_t>(src, lds, p, t); break;
    case 4: copy_in<uint32_t>(src, lds, p, t); break;
    default: copy_in<uint64_t>(src, lds, p, t); break;
  }
  __syncthreads();
  switch (p.eb) {
    case 1: copy_out<uint8_t>(dst, lds, p, t); break;
    case 2: copy_out<uint16_t>(dst, lds, p, t); break;
    case 4: copy_out<uint32_t>(dst, lds, p, t); break;
    default: copy_out<uint64_t>(dst, lds, p, t); break;
  }
}

}  // namespace

hipError_t launch_box(void* dst, const void* src, const bmm_box_desc& d, hipStream_t s) {
  BoxParams p{};
  p.rank = d.rank;
  p.eb = d.elem_bytes;
  p.swizzle = d.swizzle;
  int64_t elems = 1;
  for (int i = 0; i < d.rank; ++i) {
    p.dims[i] = d.dims[i];
    p.strides[i] = d.strides[i];
    p.coords[i] = d.coords[i];
    p.step[i] = d.coord_step[i];
    p.box[i] = d.box[i];
    elems *= d.box[i];
  }
  p.box_elems = int32_t(elems);
  // The swizzle keeps every offset inside its 128-byte row: round the image up.
  const size_t lds_bytes = size_t((elems * d.elem_bytes + 127) / 128 * 128);
  hipLaunchKernelGGL(box_kernel, dim3(unsigned(d.n_repeat)), dim3(kBoxThreads), lds_bytes, s,
                     static_cast<char*>(dst), static_cast<const char*>(src), p);
  return hipGetLastError();
}

}  // namespace bmm
