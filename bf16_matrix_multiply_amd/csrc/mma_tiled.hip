// D = A * B^T + C, LDS-staged kernel for large M and N.
//
// Operand and accumulator layouts, and the C-then-D recurrence, as in
// mma_direct.hip (mma.sync page of the TVM tirx docs: "Operand coordinates and
// ownership"; "Accumulation, transpose and alpha/beta").
//
// Macro tile 256 (M) x 256 (N), 4 waves in a 2 x 2 grid, each wave owning a
// 128 x 128 block of D = 8 x 8 MFMA blocks of 16 x 16 (64 accumulators of 4
// floats per lane, held in AGPRs). K advances in slabs of 32 (2 K atoms, one
// MFMA step).
//
// Staging takes the role the pages give to TMA box loads ("cp.async.bulk.
// tensor" page): per slab, the A box is 16 M atoms x 2 K atoms (16 pieces of
// 1 KB, each contiguous in HBM) and the B box 32 N atoms x 2 K atoms (32
// pieces of 512 B). They are moved by direct-to-LDS buffer loads (each lane's
// 16 bytes land at M0 + 16 * lane), four slabs deep: a ring of four 32 KB LDS
// stages, with slab s+4 loaded into the stage slab s has just left. Rows past
// M_rep / N_rep and K atoms past K_rep read as zero through the buffer range
// check, so the loop has no branches; slabs past the end are loaded as zeros
// and multiplied harmlessly, so the ring always holds three slabs in flight.
//
// Per slab each wave: 32 MFMAs on the fragments already in registers; wait for
// its own loads of the next slab and for its fragment reads; barrier; issue
// the loads of slab s+4; read the next slab's fragments; 32 more MFMAs. The
// barrier is a bare s_barrier with counted waits, so loads of later slabs stay
// in flight across it.
//
// LDS image: atoms are stored whole (32-byte rows); the lane that loads a
// chunk is chosen so that the two 16-byte halves of a row are swapped on a
// row-dependent XOR, which spreads a fragment read (lane l takes row l % 16,
// half (l / 16) % 2) over the banks.
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
constexpr int kSlabKAtoms = 2;    // 32 K values: one MFMA step
constexpr int kChunksA = kTileMAtoms * kSlabKAtoms * 32;  // 16-byte chunks per A slab (1024)
constexpr int kChunksB = kTileNAtoms * kSlabKAtoms * 16;  // (1024)
constexpr int kLoadsA = kChunksA / kThreads;              // 4 per thread
constexpr int kLoadsB = kChunksB / kThreads;              // 4 per thread
constexpr int kLoadsPerSlab = kLoadsA + kLoadsB;
constexpr int kStages = 4;
constexpr int kXcds = 8;
constexpr int kGroupM = 8;
// Buffer-resource word 3 for raw (unswizzled, untyped) loads on CDNA, and an
// offset that every resource here treats as out of range (reads return 0).
constexpr int kBufferFlags = 0x00020000;
constexpr uint32_t kOutOfRange = 0x7fffffffu;

// s_waitcnt immediate (gfx9 encoding): vmcnt in bits [3:0] and [15:14],
// expcnt [6:4], lgkmcnt [11:8].
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}
constexpr int kWaitVmcnt0 = waitcnt_imm(0, 15);

struct Stage {
  u32x4 a[kChunksA];
  u32x4 b[kChunksB];
};

// LDS-qualified views, so that volatile reads stay ds_read instructions.
typedef __attribute__((address_space(3))) const char lds_cchar;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

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
  // Four separate objects (not one array) so that the compiler can tell the
  // ring slots apart when it places waits for the direct-to-LDS loads.
  __shared__ __attribute__((aligned(1024))) Stage st0, st1, st2, st3;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const TileCoord tc = tile_of(blockIdx.x, n_tiles, MT, NT);
  const int64_t m_atom0 = tc.mt * kTileMAtoms, n_atom0 = tc.nt * kTileNAtoms;
  const int64_t K_rep = p.K_rep;

  // ---- direct-to-LDS staging ----
  // LDS chunk q = r * 256 + tid of a stage region is written by lane tid % 64
  // of wave tid / 64 in load r. A region: M atom q >> 6 = 4r + wave, K atom
  // (q >> 5) & 1, row (q >> 1) & 15, stored half q & 1. B region: N atom
  // q >> 5 = 8r + tid / 32, K atom (q >> 4) & 1, row (q >> 1) & 7. The global
  // half a lane fetches is the stored half XOR the row's swap bit.
  const int a_j = (tid >> 5) & 1, a_m = (tid >> 1) & 15, a_h = (tid & 1) ^ swz_a(a_m);
  const int b_i = tid >> 5, b_j = (tid >> 4) & 1, b_r = (tid >> 1) & 7;
  const int b_h = (tid & 1) ^ swz_b(b_i & 1, b_r);
  const int64_t a_row_bytes = K_rep * 512, b_row_bytes = K_rep * 256;
  const int64_t a_left = (p.M_rep - m_atom0) * a_row_bytes;
  const int64_t b_left = (p.N_rep - n_atom0) * b_row_bytes;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(p.A + (tc.b * p.M_rep + m_atom0) * K_rep * kAtomWordsA), 0,
      int(a_left < kOutOfRange ? a_left : kOutOfRange), kBufferFlags);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(p.B + (tc.b * p.N_rep + n_atom0) * K_rep * kAtomWordsB), 0,
      int(b_left < kOutOfRange ? b_left : kOutOfRange), kBufferFlags);
  uint32_t a_voff[kLoadsA], b_voff[kLoadsB];
#pragma unroll
  for (int r = 0; r < kLoadsA; ++r)
    a_voff[r] = uint32_t((4 * r + wave) * a_row_bytes + a_j * 512 + a_m * 32 + a_h * 16);
#pragma unroll
  for (int r = 0; r < kLoadsB; ++r)
    b_voff[r] = uint32_t((8 * r + b_i) * b_row_bytes + b_j * 256 + b_r * 32 + b_h * 16);

  // Loads of slab k into stage st (slabs past K_rep, and K atoms past it, read 0).
  auto issue = [&](Stage& st, int64_t k) {
    const uint32_t koff_a = uint32_t(k * kSlabKAtoms * 512), koff_b = uint32_t(k * kSlabKAtoms * 256);
    const bool a_k = k * kSlabKAtoms + a_j < K_rep, b_k = k * kSlabKAtoms + b_j < K_rep;
#pragma unroll
    for (int r = 0; r < kLoadsA; ++r)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          a_rsrc, (__attribute__((address_space(3))) void*)&st.a[r * kThreads + wave * kWave], 16,
          a_k ? a_voff[r] : kOutOfRange, koff_a, 0, 0);
#pragma unroll
    for (int r = 0; r < kLoadsB; ++r)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          b_rsrc, (__attribute__((address_space(3))) void*)&st.b[r * kThreads + wave * kWave], 16,
          b_k ? b_voff[r] : kOutOfRange, koff_b, 0, 0);
  };

  // ---- per-lane fragment offsets (bytes) in a stage region ----
  const int m = lane & 15, g = lane >> 4;
  const int a_frag = (wm * 8) * 1024 + (g >> 1) * 512 + m * 32 + 16 * ((g & 1) ^ swz_a(m));
  const int nb_atom = m >> 3, rr = m & 7;  // B row n = lane % 16 -> atom parity, row in atom
  const int b_frag = (wn * 8) * 1024 + nb_atom * 512 + (g >> 1) * 256 + rr * 32 +
                     16 * ((g & 1) ^ swz_b(nb_atom, rr));

  // ---- accumulators: C (read once, here) or the scalar ----
  f32x4 acc[8][8];
  const int64_t d_row_atom0 = m_atom0 + wm * 8;
  const int64_t d_col_atom0 = n_atom0 + wn * 16 + (g >> 1);
  const bool interior = m_atom0 + kTileMAtoms <= p.M_rep && n_atom0 + kTileNAtoms <= p.N_rep;
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

  // Slabs 0..3 into the ring; C (issued first) and slab 0 must have landed.
  issue(st0, 0);
  issue(st1, 1);
  issue(st2, 2);
  issue(st3, 3);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(3 * kLoadsPerSlab, 15));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");

  u32x4 bf[2][8], af[2][8];
  // Fragment reads are volatile so that they stay where they are written
  // (issued a half slab ahead of their MFMAs) instead of being sunk to their
  // first use.
  auto read_frags = [&](const Stage& st, u32x4 (&b)[8], u32x4 (&a)[8]) {
    const lds_cchar* sa = (const lds_cchar*)(st.a);
    const lds_cchar* sb = (const lds_cchar*)(st.b);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
      b[nb] = *reinterpret_cast<const volatile lds_u32x4*>(sb + b_frag + nb * 1024);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
      a[mb] = *reinterpret_cast<const volatile lds_u32x4*>(sa + a_frag + mb * 1024);
  };
  auto mfma_rows = [&](const u32x4 (&b)[8], const u32x4 (&a)[8], int mb0) {
#pragma unroll
    for (int mb = mb0; mb < mb0 + 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) acc[mb][nb] = mfma_16x16x32<DT>(b[nb], a[mb], acc[mb][nb]);
  };

  read_frags(st0, bf[0], af[0]);

  // One slab: its fragments are in registers set F; `cur` is its stage,
  // `nxt` the next slab's.
  auto slab = [&](int64_t s, Stage& cur, const Stage& nxt, u32x4 (&bc)[8], u32x4 (&ac)[8],
                  u32x4 (&bn)[8], u32x4 (&an)[8]) {
    __builtin_amdgcn_sched_barrier(0);
    mfma_rows(bc, ac, 0);
    // own loads of slab s+1 landed (slabs s+2, s+3 may still be in flight);
    // own fragment reads of this stage done
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * kLoadsPerSlab, 0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    issue(cur, s + kStages);
    read_frags(nxt, bn, an);
    mfma_rows(bc, ac, 4);
    // order after the barrier: the next slab's 16 fragment reads first, then
    // the 32 MFMAs with the 8 loads of slab s+4 spread among them
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
#pragma unroll
    for (int i = 0; i < kLoadsPerSlab; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  };
  const int64_t n_slabs = (K_rep + kSlabKAtoms - 1) / kSlabKAtoms;
  for (int64_t s = 0; s < n_slabs; s += kStages) {
    slab(s + 0, st0, st1, bf[0], af[0], bf[1], af[1]);
    slab(s + 1, st1, st2, bf[1], af[1], bf[0], af[0]);
    slab(s + 2, st2, st3, bf[0], af[0], bf[1], af[1]);
    slab(s + 3, st3, st0, bf[1], af[1], bf[0], af[0]);
  }
  // No load may still be writing LDS when the workgroup ends.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

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
  // Buffer offsets inside one tile's 16 A atom rows must stay below 2^31.
  if (a.K_rep >= kTiledMaxKRep) return hipErrorInvalidValue;
  auto kern = a.dtype == kBF16 ? (a.C ? mma_tiled_kernel<kBF16, true> : mma_tiled_kernel<kBF16, false>)
                               : (a.C ? mma_tiled_kernel<kF16, true> : mma_tiled_kernel<kF16, false>);
  hipLaunchKernelGGL(kern, dim3(unsigned(n_tiles)), dim3(kThreads), 0, s, a, n_tiles, MT, NT);
  return hipGetLastError();
}

}  // namespace bmm
