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
#include <type_traits>

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
// Buffer-resource word 3 for raw (unswizzled, untyped) loads on CDNA, and an
// offset that every resource here treats as out of range (reads return 0).
constexpr int kBufferFlags = 0x00020000;
constexpr uint32_t kOutOfRange = 0x7fffffffu;
// s_waitcnt immediate: vmcnt(0), expcnt and lgkmcnt at their maxima (no wait).
constexpr int kWaitVmcnt0 = 0x0f70;
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

  // ---- per-thread staging offsets ----
  // Chunk q = r * 256 + tid of a slab. For A (128 chunks per M atom) the M
  // atom is 2r + tid/128 and the K atom, row and half depend on tid only; for
  // B (64 chunks per N atom) the N atom is 4r + tid/64. Loads go through
  // buffer resources based at the tile's first atom row, whose size ends at
  // the operand's last row: rows past M_rep (N_rep) fall outside and read as
  // zero, and K atoms past K_rep are pushed outside explicitly.
  const int a_t = tid >> 7, a_j = (tid >> 5) & 3, a_m = (tid >> 1) & 15, a_h = tid & 1;
  const int b_t = tid >> 6, b_j = (tid >> 4) & 3, b_r = (tid >> 1) & 7, b_h = tid & 1;
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
    a_voff[r] = uint32_t((2 * r + a_t) * a_row_bytes + a_j * 512 + a_m * 32 + a_h * 16);
#pragma unroll
  for (int r = 0; r < kLoadsB; ++r)
    b_voff[r] = uint32_t((4 * r + b_t) * b_row_bytes + b_j * 256 + b_r * 32 + b_h * 16);
  const int a_lds = (a_t * kSlabKAtoms + a_j) * 512 + a_m * 32 + 16 * (a_h ^ swz_a(a_m));
  const int b_lds =
      kBOffset + (b_t * kSlabKAtoms + b_j) * 256 + b_r * 32 + 16 * (b_h ^ swz_b(b_t, b_r));

  // ---- per-lane fragment offsets in a stage ----
  const int m = lane & 15, g = lane >> 4;
  const int a_frag = (wm * 8) * 2048 + (g >> 1) * 512 + m * 32 + 16 * ((g & 1) ^ swz_a(m));
  const int nb_atom = m >> 3, rr = m & 7;  // B row n = lane % 16 -> atom parity, row in atom
  const int b_frag = kBOffset + (wn * 8) * 2048 + nb_atom * 1024 + (g >> 1) * 256 + rr * 32 +
                     16 * ((g & 1) ^ swz_b(nb_atom, rr));

  const int64_t n_slabs = (K_rep + kSlabKAtoms - 1) / kSlabKAtoms;
  u32x4 ga[kLoadsA], gb[kLoadsB];   // one slab in flight from HBM / L2

  auto load_slab = [&](int64_t s) {
    const int32_t koff_a = int32_t(s * kSlabKAtoms * 512), koff_b = int32_t(s * kSlabKAtoms * 256);
    const bool a_k = s * kSlabKAtoms + a_j < K_rep, b_k = s * kSlabKAtoms + b_j < K_rep;
#pragma unroll
    for (int r = 0; r < kLoadsA; ++r)
      ga[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            a_rsrc, a_k ? a_voff[r] : kOutOfRange, koff_a, 0));
#pragma unroll
    for (int r = 0; r < kLoadsB; ++r)
      gb[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            b_rsrc, b_k ? b_voff[r] : kOutOfRange, koff_b, 0));
  };
  auto store_slab = [&](int stage) {
    char* base = smem + stage * kStageBytes;
#pragma unroll
    for (int r = 0; r < kLoadsA; ++r)
      *reinterpret_cast<u32x4*>(base + a_lds + r * (kThreads * 16)) = ga[r];
#pragma unroll
    for (int r = 0; r < kLoadsB; ++r)
      *reinterpret_cast<u32x4*>(base + b_lds + r * (kThreads * 16)) = gb[r];
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

  // Software pipeline, one barrier per slab. Entering iteration s: slab s is
  // in LDS stage s&1, the first step's fragments F0 of slab s are in
  // registers, and slab s+1 is in flight into ga/gb.
  //   1. read F1 (second step of slab s) from LDS      | 64 MFMAs on F0
  //   2. write slab s+1 from ga/gb into the other stage |
  //   3. issue the global loads of slab s+2             |
  //   4. barrier (slab s+1 visible; stage s&1 no longer read)
  //   5. read F0 of slab s+1                            | 64 MFMAs on F1
  u32x4 bf0[8], af0[8], bf1[8], af1[8];
  if (n_slabs > 0) read_frags(smem, 0, bf0, af0);
  // Let C land before the loop, so no wait inside the loop is charged to it
  // (vmcnt(0), other counters untouched).
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  if (n_slabs > 1) load_slab(1);
  // One slab. kWrite: slab s+1 exists (write it to LDS, read its first
  // fragments after the barrier); kLoad: slab s+2 exists (issue its loads).
  // The body has no branches, and scheduling groups interleave the LDS writes
  // and the global loads with the MFMAs instead of leaving them behind them.
  auto slab = [&](int64_t s, auto write_tag, auto load_tag) {
    constexpr bool kWrite = decltype(write_tag)::value, kLoad = decltype(load_tag)::value;
    const int stage = int(s & 1);
    const char* base = smem + stage * kStageBytes;
    read_frags(base, 1, bf1, af1);
    mfma_step(bf0, af0);
    if constexpr (kWrite) store_slab(stage ^ 1);
    if constexpr (kLoad) load_slab(s + 2);
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);   // 16 LDS fragment reads
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);   // 16 MFMAs
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // 2 MFMAs
      if constexpr (kWrite) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
      if constexpr (kLoad) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // global load
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);   // last 16 MFMAs
    __syncthreads();
    if constexpr (kWrite) read_frags(smem + (stage ^ 1) * kStageBytes, 0, bf0, af0);
    mfma_step(bf1, af1);
    if constexpr (kWrite) __builtin_amdgcn_sched_group_barrier(0x100, 16, 1);
    __builtin_amdgcn_sched_group_barrier(0x008, 64, 1);
  };
  using T = std::true_type;
  using F = std::false_type;
  int64_t s = 0;
  for (; s + 2 < n_slabs; ++s) slab(s, T{}, T{});
  if (s + 1 < n_slabs) slab(s++, T{}, F{});
  if (s < n_slabs) slab(s, F{}, F{});

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
