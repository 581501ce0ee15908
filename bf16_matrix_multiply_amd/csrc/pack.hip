// Row-major halves -> packed b32 atoms (the operand layouts of the mma.sync
// page, "Operand coordinates and ownership", built from row-major matrices as
// in the page's worked example).
//
// Eight consecutive K values of one row are, in memory, exactly the four
// packed words of half an atom row (even K in the low half of each word on
// this little-endian machine), so packing is a permutation of 16-byte chunks:
// output chunk (row block rb, c) with c = (kr, i, h) comes from source row
// R*rb + i, K offset 16*kr + 8*h. Stores are fully contiguous; each 32-byte
// piece of a source row is read by two adjacent lanes, and the K atoms of one
// row are read by the same block in successive chunk groups.
#include "common.h"
#include "launch.h"

namespace bmm {
namespace {

constexpr int kPackThreads = 256;
constexpr int kPackUnroll = 4;

template <int R>
__global__ __launch_bounds__(kPackThreads) void pack_kernel(uint32_t* __restrict__ dst,
                                                            const uint16_t* __restrict__ src,
                                                            int64_t rb0, int32_t chunks_per_rb,
                                                            int64_t ld) {
  constexpr int kLog2R = R == 16 ? 4 : 3;
  const int64_t rb = rb0 + blockIdx.y;
  const uint16_t* srow = src + rb * R * ld;
  uint32_t* drb = dst + rb * int64_t(chunks_per_rb) * 4;
  const int32_t c0 = blockIdx.x * (kPackThreads * kPackUnroll) + threadIdx.x;
  u32x4 v[kPackUnroll];
#pragma unroll
  for (int u = 0; u < kPackUnroll; ++u) {
    const int32_t c = c0 + u * kPackThreads;
    if (c < chunks_per_rb) {
      const int32_t h = c & 1, i = (c >> 1) & (R - 1), kr = c >> (kLog2R + 1);
      v[u] = load16_nt(reinterpret_cast<const uint32_t*>(srow + i * ld + 16 * kr + 8 * h));
    }
  }
#pragma unroll
  for (int u = 0; u < kPackUnroll; ++u) {
    const int32_t c = c0 + u * kPackThreads;
    if (c < chunks_per_rb)
      __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4*>(drb + int64_t(c) * 4));
  }
}

}  // namespace

hipError_t launch_pack(uint32_t* dst, const uint16_t* src, int64_t batch, int64_t rows,
                       int64_t K, int64_t ld, int R, hipStream_t s) {
  const int64_t n_rb = batch * (rows / R);
  const int32_t chunks = int32_t(2 * R * (K / 16));  // 16-byte chunks per row block
  const int per_block = kPackThreads * kPackUnroll;
  const unsigned gx = unsigned((chunks + per_block - 1) / per_block);
  for (int64_t rb0 = 0; rb0 < n_rb; rb0 += 65535) {
    const unsigned gy = unsigned(n_rb - rb0 < 65535 ? n_rb - rb0 : 65535);
    if (R == 16)
      hipLaunchKernelGGL(pack_kernel<16>, dim3(gx, gy), dim3(kPackThreads), 0, s, dst, src,
                         rb0, chunks, ld);
    else
      hipLaunchKernelGGL(pack_kernel<8>, dim3(gx, gy), dim3(kPackThreads), 0, s, dst, src,
                         rb0, chunks, ld);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bmm
