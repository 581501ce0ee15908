// D = A * B^T + C, direct kernel: one wave per 16x16 block of D, operand
// fragments loaded straight from global memory. Any shape; it is the kernel
// for small problems (where launch latency dominates) and the baseline the
// staged kernels are checked against.
//
// Layouts (mma.sync page, "Operand coordinates and ownership"): A is
// (batch, M_rep, K_rep, 16, 8) words, B (batch, N_rep, K_rep, 8, 8) words, C/D
// (batch, M_rep, N_rep, 16, 8) float32. The recurrence (mma.sync page,
// "Accumulation, transpose and alpha/beta"): the accumulator starts from C
// (or the scalar) once, then every K step adds into it in ascending order.
//
// Fragment map. One MFMA step covers 16 rows of D, 16 columns (two N atoms)
// and 32 K values (two K atoms). B is fed as the instruction's first operand
// and A as its second, so the instruction produces D transposed: lane l holds
// D[m = l%16][n = 4*(l/16) .. 4*(l/16)+3], which in the accumulator layout is
// one contiguous 16-byte piece of N atom (l/16)/2. Lane group g = l/16 takes K
// values 8g .. 8g+7 of the step for both operands: K atom g/2, words
// 4*(g%2) .. 4*(g%2)+3 (or K atom g, all 4 words, in the k = 8 layout). A's
// 16-row fragment for a step is then 1 KB of contiguous memory, and every
// lane moves exactly 16 bytes.
#include "common.h"
#include "launch.h"

namespace bmm {
namespace {

constexpr int kDirectWaves = 4;

template <int DT>
__global__ __launch_bounds__(kDirectWaves* kWave) void mma_direct_kernel(MmaArgs p,
                                                                        int64_t n_tiles,
                                                                        int64_t NT) {
  const int lane = threadIdx.x & 63;
  const int64_t tile = int64_t(blockIdx.x) * kDirectWaves + (threadIdx.x >> 6);
  if (tile >= n_tiles) return;
  const int64_t nt = tile % NT;
  const int64_t bm = tile / NT;  // b * M_rep + mr
  const int64_t b = bm / p.M_rep;

  const int m = lane & 15, g = lane >> 4;
  // Output: N atom and column offset of this lane's 4 accumulators.
  const int64_t na = 2 * nt + (g >> 1);
  const bool n_ok = na < p.N_rep;
  const int64_t d_off = ((bm * p.N_rep + na) * 16 + m) * 8 + 4 * (g & 1);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (!p.scaled) {
    if (p.C) {
      if (n_ok) acc = load16f(p.C + d_off);
    } else {
      acc = f32x4{p.c_scalar, p.c_scalar, p.c_scalar, p.c_scalar};
    }
  }

  // Operand fragments: A row m, B row n = lane % 16 of this tile's 16 columns.
  const int64_t nck = k_chunks(p);
  const uint32_t* a_ptr = p.A + bm * nck * 64 + a_lane_words(p.atom_k, m, g);
  const int64_t nb = 2 * nt + (m >> 3);
  const bool b_ok = nb < p.N_rep;
  const uint32_t* b_ptr =
      p.B + (b * p.N_rep + (b_ok ? nb : 0)) * nck * 32 + b_lane_words(p.atom_k, m & 7, g);
  const u32x4 zero = {0u, 0u, 0u, 0u};

  const int64_t steps = (nck + 3) / 4;
  int64_t s = 0;
  // Two steps per iteration keep two loads of each operand in flight.
  for (; s + 2 <= steps; s += 2) {
    const bool k0 = 4 * s + g < nck, k1 = 4 * s + 4 + g < nck;
    const u32x4 a0 = k0 ? load16(a_ptr + s * 256) : zero;
    const u32x4 a1 = k1 ? load16(a_ptr + s * 256 + 256) : zero;
    const u32x4 b0 = (b_ok && k0) ? load16(b_ptr + s * 128) : zero;
    const u32x4 b1 = (b_ok && k1) ? load16(b_ptr + s * 128 + 128) : zero;
    acc = mfma_16x16x32<DT>(b0, a0, acc);
    acc = mfma_16x16x32<DT>(b1, a1, acc);
  }
  for (; s < steps; ++s) {
    const bool k0 = 4 * s + g < nck;
    const u32x4 a0 = k0 ? load16(a_ptr + s * 256) : zero;
    const u32x4 b0 = (b_ok && k0) ? load16(b_ptr + s * 128) : zero;
    acc = mfma_16x16x32<DT>(b0, a0, acc);
  }
  if (!n_ok) return;
  if (p.scaled) {
    // alpha/beta form: C is read here, after the product
    const f32x4 cv = p.C ? load16f(p.C + d_off) : f32x4{p.c_scalar, p.c_scalar, p.c_scalar, p.c_scalar};
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(p.alpha, acc[e], p.beta * cv[e]);
  }
  store16f(p.D + d_off, acc);
}

}  // namespace

hipError_t launch_mma_direct(const MmaArgs& a, hipStream_t s) {
  const int64_t NT = (a.N_rep + 1) / 2;
  const int64_t n_tiles = a.batch * a.M_rep * NT;
  const int64_t blocks = (n_tiles + kDirectWaves - 1) / kDirectWaves;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (a.dtype == kBF16)
    hipLaunchKernelGGL(mma_direct_kernel<kBF16>, dim3(unsigned(blocks)),
                       dim3(kDirectWaves * kWave), 0, s, a, n_tiles, NT);
  else
    hipLaunchKernelGGL(mma_direct_kernel<kF16>, dim3(unsigned(blocks)),
                       dim3(kDirectWaves * kWave), 0, s, a, n_tiles, NT);
  return hipGetLastError();
}

}  // namespace bmm
