// D = A * B^T + C, kernel for few rows of D (small M): bound by streaming B
// from HBM once.
//
// Operand and accumulator layouts, fragment map and the C-then-D recurrence
// as in mma_direct.hip (mma.sync page of the TVM tirx docs: "Operand
// coordinates and ownership"; "Accumulation, transpose and alpha/beta").
//
// A workgroup owns 64 columns of D (8 N atoms; 32 columns for a single M
// atom) for up to 4 M atoms (64 rows).
// Its waves split the K steps into contiguous chunks, one per wave; each wave
// streams its part of B straight from HBM into registers with 16-byte
// non-temporal loads (B is read exactly once), keeps several K steps of loads
// in flight, and reuses each B fragment for every M atom. A (small, read by
// every workgroup) is loaded through the cache.
//
// The recurrence is kept: wave 0, which holds the first K chunk, starts from C
// (or the scalar); the other waves start from zero; the partial sums are then
// added in K order (((wave 0 + wave 1) + wave 2) + ...) through LDS, so every
// output is C plus its products in ascending K chunks, and the result is the
// same on every run.
#include "common.h"
#include "launch.h"

namespace bmm {
namespace {

// Columns per workgroup: 64 (8 N atoms, 4 MFMA blocks of 16) when the
// workgroup holds several M atoms; 32 for a single M atom, where twice the
// workgroups give HBM more streams in flight (measured 3-7% faster at
// 16 x 16384 x 16384, 20% slower at 64 rows).
template <int MR>
constexpr int n_atoms() { return MR == 1 ? 4 : 8; }
constexpr int kUnroll = 4;       // K steps whose loads are issued together

constexpr int kWaves = 8;        // waves per workgroup, one contiguous K chunk each

template <int DT, int MR, bool kHasC, bool kScaled>
__global__ __launch_bounds__(kWaves* kWave) void mma_skinny_kernel(MmaArgs p) {
  constexpr int W = kWaves;
  constexpr int kNAtoms = n_atoms<MR>();
  constexpr int kNBlocks = kNAtoms / 2;
  __shared__ __attribute__((aligned(16))) f32x4 red[W][MR][kNBlocks][kWave];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nt = blockIdx.x;                 // N tile of kNAtoms atoms
  const int64_t mg = blockIdx.y;                 // group of MR M atoms
  const int64_t b = blockIdx.z;
  const int m = lane & 15, g = lane >> 4;
  const int64_t m_atom0 = mg * MR;

  // ---- fragment pointers ----
  // B block nb: rows n = 16*nb + lane%16 of this tile -> atom 2*nb + m/8, row m%8.
  const int64_t nck = k_chunks(p);   // 8-value K chunks; a step covers 4
  const uint32_t* b_ptr[kNBlocks];
  bool b_ok[kNBlocks];
#pragma unroll
  for (int nb = 0; nb < kNBlocks; ++nb) {
    const int64_t atom = nt * kNAtoms + 2 * nb + (m >> 3);
    b_ok[nb] = atom < p.N_rep;
    b_ptr[nb] = p.B + (b * p.N_rep + (b_ok[nb] ? atom : 0)) * nck * 32 +
                b_lane_words(p.atom_k, m & 7, g);
  }
  const uint32_t* a_ptr[MR];
  bool a_ok[MR];
#pragma unroll
  for (int mi = 0; mi < MR; ++mi) {
    const int64_t atom = m_atom0 + mi;
    a_ok[mi] = atom < p.M_rep;
    a_ptr[mi] = p.A + (b * p.M_rep + (a_ok[mi] ? atom : 0)) * nck * 64 + a_lane_words(p.atom_k, m, g);
  }

  // ---- this wave's K steps ----
  const int64_t steps = (nck + 3) / 4;
  const int64_t chunk = (steps + W - 1) / W;
  const int64_t s_begin = wave * chunk < steps ? wave * chunk : steps;
  const int64_t s_end = s_begin + chunk < steps ? s_begin + chunk : steps;

  // ---- accumulators ----
  f32x4 acc[MR][kNBlocks];
  const int64_t d_col0 = nt * kNAtoms + (g >> 1);  // + 2 * nb
#pragma unroll
  for (int mi = 0; mi < MR; ++mi)
#pragma unroll
    for (int nb = 0; nb < kNBlocks; ++nb) {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (!kScaled && wave == 0) {
        if constexpr (kHasC) {
          const int64_t na = d_col0 + 2 * nb;
          if (a_ok[mi] && na < p.N_rep)
            v = load16f(p.C + (((b * p.M_rep + m_atom0 + mi) * p.N_rep + na) * 16 + m) * 8 +
                        4 * (g & 1));
        } else {
          v = f32x4{p.c_scalar, p.c_scalar, p.c_scalar, p.c_scalar};
        }
      }
      acc[mi][nb] = v;
    }

  const u32x4 zero = {0u, 0u, 0u, 0u};
  int64_t s = s_begin;
  // Full groups: every K chunk is inside K (the ragged step is the last one).
  for (; s + kUnroll <= s_end && 4 * (s + kUnroll) <= nck; s += kUnroll) {
    u32x4 bf[kUnroll][kNBlocks], af[kUnroll][MR];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
      for (int nb = 0; nb < kNBlocks; ++nb)
        bf[u][nb] = b_ok[nb] ? load16_nt(b_ptr[nb] + (s + u) * 128) : zero;
#pragma unroll
      for (int mi = 0; mi < MR; ++mi)
        af[u][mi] = a_ok[mi] ? load16(a_ptr[mi] + (s + u) * 256) : zero;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int mi = 0; mi < MR; ++mi)
#pragma unroll
        for (int nb = 0; nb < kNBlocks; ++nb)
          acc[mi][nb] = mfma_16x16x32<DT>(bf[u][nb], af[u][mi], acc[mi][nb]);
  }
  // Remaining steps one at a time, with the K tail zeroed in registers.
  for (; s < s_end; ++s) {
    const bool k_ok = 4 * s + g < nck;
    u32x4 bf[kNBlocks], af[MR];
#pragma unroll
    for (int nb = 0; nb < kNBlocks; ++nb)
      bf[nb] = (k_ok && b_ok[nb]) ? load16_nt(b_ptr[nb] + s * 128) : zero;
#pragma unroll
    for (int mi = 0; mi < MR; ++mi)
      af[mi] = (k_ok && a_ok[mi]) ? load16(a_ptr[mi] + s * 256) : zero;
#pragma unroll
    for (int mi = 0; mi < MR; ++mi)
#pragma unroll
      for (int nb = 0; nb < kNBlocks; ++nb)
        acc[mi][nb] = mfma_16x16x32<DT>(bf[nb], af[mi], acc[mi][nb]);
  }

  // ---- reduce the waves' partial sums in K order ----
#pragma unroll
  for (int mi = 0; mi < MR; ++mi)
#pragma unroll
    for (int nb = 0; nb < kNBlocks; ++nb) red[wave][mi][nb][lane] = acc[mi][nb];
  __syncthreads();
  constexpr int kOut = MR * kNBlocks * kWave;  // float4 outputs of the workgroup
  for (int o = threadIdx.x; o < kOut; o += W * kWave) {
    const int mi = o / (kNBlocks * kWave), nb = (o / kWave) % kNBlocks, l = o % kWave;
    f32x4 sum = red[0][mi][nb][l];
#pragma unroll
    for (int w = 1; w < W; ++w) sum += red[w][mi][nb][l];
    const int lm = l & 15, lg = l >> 4;
    const int64_t ma = m_atom0 + mi, na = nt * kNAtoms + 2 * nb + (lg >> 1);
    if (ma < p.M_rep && na < p.N_rep) {
      const int64_t off = (((b * p.M_rep + ma) * p.N_rep + na) * 16 + lm) * 8 + 4 * (lg & 1);
      if constexpr (kScaled) {
        // alpha/beta form: C is read here, after the product
        f32x4 cv = {p.c_scalar, p.c_scalar, p.c_scalar, p.c_scalar};
        if constexpr (kHasC) cv = load16f(p.C + off);
#pragma unroll
        for (int e = 0; e < 4; ++e) sum[e] = __builtin_fmaf(p.alpha, sum[e], p.beta * cv[e]);
      }
      store16f(p.D + off, sum);
    }
  }
}

template <int DT, int MR>
hipError_t launch_mr(const MmaArgs& a, hipStream_t s) {
  constexpr int kNAtoms = n_atoms<MR>();
  const int64_t n_tiles = (a.N_rep + kNAtoms - 1) / kNAtoms;
  const int64_t m_groups = (a.M_rep + MR - 1) / MR;
  if (n_tiles > 0x7fffffff || m_groups > 65535 || a.batch > 65535)
    return hipErrorInvalidConfiguration;
  dim3 grid(unsigned(n_tiles), unsigned(m_groups), unsigned(a.batch));
  auto kern = a.scaled ? (a.C ? mma_skinny_kernel<DT, MR, true, true> : mma_skinny_kernel<DT, MR, false, true>)
                       : (a.C ? mma_skinny_kernel<DT, MR, true, false> : mma_skinny_kernel<DT, MR, false, false>);
  hipLaunchKernelGGL(kern, grid, dim3(kWaves * kWave), 0, s, a);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const MmaArgs& a, hipStream_t s) {
  switch (a.M_rep) {
    case 1: return launch_mr<DT, 1>(a, s);
    case 2: return launch_mr<DT, 2>(a, s);
    case 3: return launch_mr<DT, 3>(a, s);
    default: return launch_mr<DT, 4>(a, s);
  }
}

}  // namespace

hipError_t launch_mma_skinny(const MmaArgs& a, hipStream_t s) {
  return a.dtype == kBF16 ? launch_dt<kBF16>(a, s) : launch_dt<kF16>(a, s);
}

}  // namespace bmm
