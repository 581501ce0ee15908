// D = A * B^T + C, LDS-staged kernel for large M and N.
//
// Operand and accumulator layouts, and the C-then-D recurrence, as in
// mma_direct.hip (mma.sync page of the TVM tirx docs: "Operand coordinates and
// ownership"; "Accumulation, transpose and alpha/beta").
//
// Macro tile 256 (M) x 256 (N), 4 waves in a 2 x 2 grid, each wave owning a
// 128 x 128 block of D = 8 x 8 MFMA blocks of 16 x 16 (64 accumulators of 4
// floats per lane). K advances in slabs of 64 (4 K atoms, two MFMA steps).
//
// Staging takes the role the pages give to TMA box loads ("cp.async.bulk.
// tensor" page): per slab, the A box is 16 M atoms x 4 K atoms (16 pieces of
// 2 KB, each contiguous in HBM) and the B box 32 N atoms x 4 K atoms (32
// pieces of 1 KB). 256 lanes move them in 16-byte chunks, consecutive lanes
// on consecutive chunks, first into registers (so the next slab's loads are in
// flight while the current slab is multiplied), then into one of two LDS
// stages. Chunks that fall outside the operands (ragged M, N or K) are zero.
//
// LDS image: atoms are stored whole (32-byte rows), with the two 16-byte
// halves of a row swapped on a row-dependent XOR so that a fragment read
// (lane l takes row l % 16, half (l / 16) % 2) hits distinct banks within
// every group of 8 or 16 lanes.
//
// Work order: workgroups are dispatched round-robin over the 8 XCDs; the
// linear tile index is remapped so each XCD receives a contiguous run of
// tiles, and runs are rasterised in bands of 8 M tiles, so the tiles that
// share A rows and B columns run on the same XCD and share its L2.
#include "common.h"
#include "launch.h"

namespace bmm {
namespace {

constexpr int kThreads = 256;
constexpr int kTileMAtoms = 16;   // 256 rows
constexpr int kTileNAtoms = 32;   // 256 columns
constexpr int kSlabKAtoms = 4;    // 64 K values
constexpr int kChunksA = kTileMAtoms * kSlabKAtoms * 32;  // 16-byte chunks per A slab
constexpr int kChunksB = kTileNAtoms * kSlabKAtoms * 16;
constexpr int kLoadsA = kChunksA / kThreads;              // 8 per thread
constexpr int kLoadsB = kChunksB / kThreads;              // 8 per thread
constexpr int kStageBytes = (kChunksA + kChunksB) * 16;   // 64 KB
constexpr int kBOffset = kChunksA * 16;
constexpr int kXcds = 8;
constexpr int kGroupM = 8;

// Half-swap of a 32-byte LDS row (see the file comment). A atoms have 16
// rows; B atoms have 8 and alternate parity with the N atom index.
__device__ __forceinline__ int swz_a(int row) { return ((row >> 2) ^ (row >> 3)) & 1; }
__device__ __forceinline__ int swz_b(int atom, int row) { return ((row >> 2) ^ atom) & 1; }

struct TileCoord {
  int64_t b, mt, nt;
};

// Linear workgroup id -> (batch, M tile, N tile); a bijection for any count.
__device__ __forceinline__ TileCoord tile_of(int64_t w, int64_t n_tiles, int64_t MT,
                                             int64_t NT) {
  const int64_t q = n_tiles / kXcds, r = n_tiles % kXcds;
  const int64_t xcd = w % kXcds, k = w / kXcds;
  const int64_t t = xcd * q + (xcd < r ? xcd : r) + k;
  const int64_t per_batch = MT * NT;
  TileCoord c;
  c.b = t / per_batch;
  const int64_t u = t % per_batch;
  const int64_t group = kGroupM * NT;
  const int64_t first_m = (u / group) * kGroupM;
  const int64_t gm = MT - first_m < kGroupM ? MT - first_m : kGroupM;
  const int64_t v = u % group;
  c.mt = first_m + v % gm;
  c.nt = v / gm;
  return c;
}

template <int DT, bool kHasC>
__global__ __launch_bounds__(kThreads, 1) void mma_tiled_kernel(MmaArgs p, int64_t n_tiles,
                                                               int64_t MT, int64_t NT) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const TileCoord tc = tile_of(blockIdx.x, n_tiles, MT, NT);
  const int64_t m_atom0 = tc.mt * kTileMAtoms, n_atom0 = tc.nt * kTileNAtoms;
  const int64_t K_rep = p.K_rep;

  // ---- per-thread staging addresses ----
  // Chunk q = r * 256 + tid of a slab. For A (128 chunks per M atom) the M
  // atom is 2r + tid/128 and the K atom, row and half depend on tid only; for
  // B (64 chunks per N atom) the N atom is 4r + tid/64. So each operand needs
  // one base pointer, an atom-row stride per r, and LDS offsets r * 4096 + c.
  const int a_t = tid >> 7, a_j = (tid >> 5) & 3, a_m = (tid >> 1) & 15, a_h = tid & 1;
  const int64_t a_row0 = m_atom0 + a_t;
  const uint32_t* a_base = p.A + ((tc.b * p.M_rep + a_row0) * K_rep + a_j) * kAtomWordsA +
                           a_m * 8 + a_h * 4;
  const int64_t a_rstride = 2 * K_rep * kAtomWordsA;  // words between r and r + 1
  const int a_lds = (a_t * kSlabKAtoms + a_j) * 512 + a_m * 32 + 16 * (a_h ^ swz_a(a_m));
  const int b_t = tid >> 6, b_j = (tid >> 4) & 3, b_r = (tid >> 1) & 7, b_h = tid & 1;
  const int64_t b_row0 = n_atom0 + b_t;
  const uint32_t* b_base = p.B + ((tc.b * p.N_rep + b_row0) * K_rep + b_j) * kAtomWordsB +
                           b_r * 8 + b_h * 4;
  const int64_t b_rstride = 4 * K_rep * kAtomWordsB;
  const int b_lds =
      kBOffset + (b_t * kSlabKAtoms + b_j) * 256 + b_r * 32 + 16 * (b_h ^ swz_b(b_t, b_r));
  // rows of this tile that exist (ragged last tiles): bit r set if chunk group r is in range
  uint32_t a_rows_ok = 0, b_rows_ok = 0;
#pragma unroll
  for (int r = 0; r < kLoadsA; ++r) a_rows_ok |= uint32_t(a_row0 + 2 * r < p.M_rep) << r;
#pragma unroll
  for (int r = 0; r < kLoadsB; ++r) b_rows_ok |= uint32_t(b_row0 + 4 * r < p.N_rep) << r;

  // ---- per-lane fragment offsets in a stage ----
  const int m = lane & 15, g = lane >> 4;
  const int a_frag = (wm * 8) * 2048 + (g >> 1) * 512 + m * 32 + 16 * ((g & 1) ^ swz_a(m));
  const int nb_atom = m >> 3, rr = m & 7;  // B row n = lane % 16 -> atom parity, row in atom
  const int b_frag = kBOffset + (wn * 8) * 2048 + nb_atom * 1024 + (g >> 1) * 256 + rr * 32 +
                     16 * ((g & 1) ^ swz_b(nb_atom, rr));

  const int64_t n_slabs = (K_rep + kSlabKAtoms - 1) / kSlabKAtoms;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 ra[kLoadsA], rb[kLoadsB];

  auto load_slab = [&](int64_t s) {
    const int64_t k0 = s * kSlabKAtoms;
    const bool a_k = k0 + a_j < K_rep, b_k = k0 + b_j < K_rep;
    const uint32_t* pa = a_base + k0 * kAtomWordsA;
    const uint32_t* pb = b_base + k0 * kAtomWordsB;
#pragma unroll
    for (int r = 0; r < kLoadsA; ++r)
      ra[r] = (a_k && ((a_rows_ok >> r) & 1)) ? load16(pa + r * a_rstride) : zero;
#pragma unroll
    for (int r = 0; r < kLoadsB; ++r)
      rb[r] = (b_k && ((b_rows_ok >> r) & 1)) ? load16(pb + r * b_rstride) : zero;
  };
  auto store_slab = [&](int stage) {
    char* base = smem + stage * kStageBytes;
#pragma unroll
    for (int r = 0; r < kLoadsA; ++r)
      *reinterpret_cast<u32x4*>(base + a_lds + r * (kThreads * 16)) = ra[r];
#pragma unroll
    for (int r = 0; r < kLoadsB; ++r)
      *reinterpret_cast<u32x4*>(base + b_lds + r * (kThreads * 16)) = rb[r];
  };

  // The first slab goes to LDS before C is loaded, so the staging registers
  // are free while the 256 accumulator registers fill.
  if (n_slabs > 0) {
    load_slab(0);
    store_slab(0);
  }

  // ---- accumulators: C (read once, here) or the scalar ----
  f32x4 acc[8][8];
  const int64_t d_row_atom0 = m_atom0 + wm * 8;
  const int64_t d_col_atom0 = n_atom0 + wn * 16 + (g >> 1);
  const bool interior = m_atom0 + kTileMAtoms <= p.M_rep && n_atom0 + kTileNAtoms <= p.N_rep;
  // lane's float offset in the accumulator layout, and the strides of its blocks
  const int64_t d_lane = (((tc.b * p.M_rep + d_row_atom0) * p.N_rep + d_col_atom0) * 16 + m) * 8 +
                         4 * (g & 1);
  const int64_t d_mstride = p.N_rep * kAtomFloats;  // next M atom
  if constexpr (kHasC) {
    // Blocks outside a ragged last tile read a clamped (valid) address: their
    // accumulators are never stored, and one branch-free path keeps the 256
    // accumulator registers in place.
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int64_t ma = d_row_atom0 + mb < p.M_rep ? d_row_atom0 + mb : p.M_rep - 1;
        const int64_t na = d_col_atom0 + 2 * nb < p.N_rep ? d_col_atom0 + 2 * nb : p.N_rep - 1;
        acc[mb][nb] = load16f(p.C + (((tc.b * p.M_rep + ma) * p.N_rep + na) * 16 + m) * 8 +
                              4 * (g & 1));
      }
  } else {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
        acc[mb][nb] = f32x4{p.c_scalar, p.c_scalar, p.c_scalar, p.c_scalar};
  }
  __syncthreads();

  // Fragments of one 32-deep K step: 8 B blocks and 8 A blocks of the wave.
  auto read_frags = [&](const char* base, int kk, u32x4 (&bf)[8], u32x4 (&af)[8]) {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
      bf[nb] = *reinterpret_cast<const u32x4*>(base + b_frag + nb * 2048 + kk * 512);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
      af[mb] = *reinterpret_cast<const u32x4*>(base + a_frag + mb * 2048 + kk * 1024);
  };
  auto mfma_step = [&](const u32x4 (&bf)[8], const u32x4 (&af)[8]) {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) acc[mb][nb] = mfma_16x16x32<DT>(bf[nb], af[mb], acc[mb][nb]);
  };

  for (int64_t s = 0; s < n_slabs; ++s) {
    const int stage = int(s & 1);
    const bool more = s + 1 < n_slabs;
    const char* base = smem + stage * kStageBytes;
    u32x4 bf0[8], af0[8], bf1[8], af1[8];
    read_frags(base, 0, bf0, af0);
    if (more) load_slab(s + 1);
    read_frags(base, 1, bf1, af1);   // in flight during the first step's MFMAs
    mfma_step(bf0, af0);
    mfma_step(bf1, af1);
    if (more) store_slab(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: 16-byte stores, one 1 KB contiguous block per MFMA block ----
  if (interior) {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
        store16f(p.D + d_lane + mb * d_mstride + nb * 2 * kAtomFloats, acc[mb][nb]);
  } else {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
        if (d_row_atom0 + mb < p.M_rep && d_col_atom0 + 2 * nb < p.N_rep)
          store16f(p.D + d_lane + mb * d_mstride + nb * 2 * kAtomFloats, acc[mb][nb]);
  }
}

}  // namespace

hipError_t launch_mma_tiled(const MmaArgs& a, hipStream_t s) {
  const int64_t MT = (a.M_rep + kTileMAtoms - 1) / kTileMAtoms;
  const int64_t NT = (a.N_rep + kTileNAtoms - 1) / kTileNAtoms;
  const int64_t n_tiles = a.batch * MT * NT;
  if (n_tiles > 0x7fffffff) return hipErrorInvalidConfiguration;
  auto kern = a.dtype == kBF16 ? (a.C ? mma_tiled_kernel<kBF16, true> : mma_tiled_kernel<kBF16, false>)
                               : (a.C ? mma_tiled_kernel<kF16, true> : mma_tiled_kernel<kF16, false>);
  hipLaunchKernelGGL(kern, dim3(unsigned(n_tiles)), dim3(kThreads), 0, s, a, n_tiles, MT, NT);
  return hipGetLastError();
}

}  // namespace bmm
