// D = A * B^T + C, LDS-staged kernel for large M and N.
//
// Operand and accumulator layouts, and the C-then-D recurrence, as in
// mma_direct.hip (mma.sync page of the TVM tirx docs: "Operand coordinates and
// ownership"; "Accumulation, transpose and alpha/beta").
//
// Macro tiles (TM x TN of D) and their schedules:
// - without split-K or alpha/beta, every tile: 4 waves in a 2 x 2 grid, each
//   TM/2 x TN/2 of D (mma_tiled4_kernel), v_mfma_f32_16x16x32_{bf16,f16}; one
//   workgroup per CU for 256 rows (one wave per SIMD), two for 128 x 128; with
//   alpha/beta the same pipeline for 256 x 128 and for 256 x 256 grids of more
//   than one round (the product from zero, C read in the epilogue);
// - with split-K, or alpha/beta on the other grids: 256 x 256 and 256 x 128 run
//   8 waves (two per SIMD) in two groups that alternate ("ping-pong", below),
//   16x16x32; 128 x 128 runs 4 waves (two workgroups per CU), one group,
//   v_mfma_f32_32x32x16.
// All of them give the same bits: each 32-deep step adds the same 32 products
// per output to the same accumulator, in the same order of steps.
//
// Why 16x16x32 in the ping-pong path: at 8192^3 on normal(0,1) bf16 operands
// the chip runs at its 1400 W power limit, so speed is set by energy per flop.
// Per flop, 16x16x32 reads and writes half the accumulator registers of
// 32x32x16 (4 + 4 per 8192 products against 16 + 16 per 16384), for the same
// LDS bytes. Measured on MI355X in one process: 8192^3 803.3 -> 760.0 us,
// 8192^3 on quarter-integer operands 719.5 -> 674.9 us, 4096^3 88.8 -> 84.0 us,
// with the same bits: each 16x16x32 step sums the same 32 products per output
// into the same accumulator as two 32x32x16 steps.
//
// 16x16x32 fragment map (B fed as the first operand, A as the second, so the
// result is D transposed): lane l supplies row n = l % 16 of a 16-column block
// of B and row m = l % 16 of a 16-row block of A, each with the 8 K values of
// chunk l / 16 of the 32-deep step (k = 16 layout: atom chunk / 2, half
// chunk % 2; k = 8 layout: atom chunk), and receives
// D[m = l % 16][n = 4 * (l / 16) .. + 3]: one contiguous 16-byte piece of an
// accumulator atom.
// 32x32x16 fragment map (128 x 128 tile): lane l supplies row l % 32 of a
// 32-column block of B and of a 32-row block of A with the 8 K values of chunk
// l / 32 of a 16-deep half step, and register r = 4q + t receives
// D[m = l % 32][n = 8q + 4 * (l / 32) + t].
//
// K advances in slabs of 32 values (four 8-value chunks: 2 atoms of k = 16 or
// 4 of k = 8). Staging takes the role the pages give to TMA box loads
// ("cp.async.bulk.tensor" page). The LDS image of a slab is fragment-major:
// every 1 KB holds one operand fragment in lane order, so one direct-to-LDS
// buffer load (each lane's 16 bytes land at M0 + 16 * lane) writes exactly one
// fragment, gathered from the packed atoms in HBM, and one ds_read_b128 per
// lane reads it back contiguously (no bank conflicts). Loads run four slabs
// deep: a ring of four stages, with slab s+4 loaded into the stage slab s has
// just left. Rows past M_rep / N_rep read as zero through the buffer range
// check and K chunks past the end are given an out-of-range offset, so the
// loop has no branches; slabs past the end load as zeros and are multiplied
// harmlessly. A second grid axis, when present, splits K (split-K form).
//
// Ping-pong schedule (256 x 256: each wave owns 128 x 64 of D; 256 x 128: 64 x
// 64): waves 0-3 (group 0, the upper 128 rows) and waves 4-7 (group 1, the
// lower 128 rows) share the four SIMDs, one wave of each per SIMD. Every slab
// has two phases, each ended by a workgroup barrier. In phase 0 group 0 issues
// the slab's MFMAs back to back while group 1 reads its fragments of the slab
// from LDS and issues its loads of slab t+3; in phase 1 the roles swap (group
// 1 multiplies, group 0 reads its fragments of slab t+1 and issues its loads
// of slab t+4). So on every SIMD one wave keeps the MFMA pipe busy while the
// other does the memory work and waits, and at a barrier the waiting wave
// starts its MFMAs while the last ones of the other wave drain. Both groups
// run the same number of barriers. Each barrier is a bare s_barrier after a
// counted wait, so loads of later slabs stay in flight across it.
//
// 4-wave tiles (no split-K): in the 256 x 256 tile a wave's 64
// accumulators of 4 floats fill the 256 accumulator registers, so it holds a
// 128 x 128 block and reads a third fewer LDS bytes per MFMA than a ping-pong
// wave. A wave keeps the pipe fed by placing the next slab's fragment reads and
// loads between the MFMAs of the current slab, with one barrier per slab.
// Measured against the earlier schedules, same bits: 8192^3 normal bf16 with a
// C tensor 0.1-1.1% faster than ping-pong on three boxes (the chip is at its
// power limit there), 1.1-2.0% with a scalar C, 1.6-2.4% on 4096^3
// quarter-integer operands; the 256 x 128 tile 7-13% faster than ping-pong
// (8192 x 1024 x 8192 110.6 against 119.3 us, 2304 x 2048 x 4096 45.8 against
// 52.9 us), where the ping-pong phases of 16 MFMAs per wave left the pipe half
// idle; the 128 x 128 tile 5-9% faster than the one-group 32x32x16 schedule
// (2048^3 23.0 against 25.3 us, 2048 x 2048 x 8192 69.5 against 74.4 us).
// With alpha/beta the accumulators start from zero and the epilogue reads C in
// batches of up to 16 blocks, with no branch around the reads, before the
// batch's stores; the launch takes this pipeline only for the grids where it
// measured faster (the launch code below lists them).
//
// The 128 x 128 tile with split-K or alpha/beta (two workgroups per CU, one
// wave per SIMD each) keeps a one-group schedule: per slab, the MFMAs of the first 16-value half on
// fragments already in registers; wait for its own loads of the next slab and
// its fragment reads; barrier; issue the loads of slab s+4; read the next
// slab's fragments; the MFMAs of the second half.
//
// C is read and D written with non-temporal accesses (each is touched once);
// split-K partial sums are stored through the caches instead, since the
// reduce reads them right after (1024 x 1024 x 65536, 16 splits: 138 against
// 145 us for the whole split-K call).
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

// Macro tile shapes (TM x TN of D):
// - 256 x 256: 8 waves (two per SIMD) in a 2 x 4 grid, each 128 x 64 of D, one
//   workgroup per CU;
// - 256 x 128: 8 waves in a 4 x 2 grid, each 64 x 64, a 96 KB ring, one
//   workgroup per CU, for problems with too few 256 x 256 tiles to fill the
//   chip but enough of these;
// - 128 x 128: 4 waves in a 2 x 2 grid, each 64 x 64, a 64 KB ring, two
//   workgroups per CU.
// Every wave covers 64 columns. kWaveBlocksM/N count 32-row / 32-column
// blocks per wave; a stage holds TM / 16 A and TN / 16 B fragments of 1 KB.
template <int TM, int TN>
struct Tile {
  static constexpr int kWaves = TM == 256 ? 8 : 4;
  static constexpr int kWavesN = TN / 64;                 // wave grid columns
  static constexpr int kWaveBlocksM = TM / 32 / (kWaves / kWavesN);  // 32-row blocks per wave
  static constexpr int kWaveBlocksN = 2;                  // 32-column blocks per wave
  static constexpr int kTileMAtoms = TM / 16;
  static constexpr int kTileNAtoms = TN / 8;
  static constexpr int kFragsA = TM / 16;   // per slab: TM/32 blocks of 32 rows x 2 K halves
  static constexpr int kFragsB = TN / 16;   // per slab: TN/32 blocks of 32 columns x 2 K halves
  // Loads per wave per slab: one per fragment, spread over the waves.
  static constexpr int kLoadsA = kFragsA / kWaves, kLoadsB = kFragsB / kWaves;
  static constexpr int kLoadsPerSlab = kLoadsA + kLoadsB;
  static_assert(kLoadsA * kWaves == kFragsA && kLoadsB * kWaves == kFragsB,
                "one load per fragment");
  static_assert(kWaveBlocksM * 32 * (kWaves / kWavesN) == TM, "wave grid covers the tile");
};
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

// One ring stage: fragment f of each operand is 64 lanes x 16 bytes.
template <int TM, int TN>
struct Stage {
  u32x4 a[Tile<TM, TN>::kFragsA][kWave];
  u32x4 b[Tile<TM, TN>::kFragsB][kWave];
};

typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int DT>
__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 x, u32x4 y, f32x16 acc) {
  if constexpr (DT == kBF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x),
                                                   __builtin_bit_cast(bf16x8, y), acc, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, x),
                                                  __builtin_bit_cast(f16x8, y), acc, 0, 0, 0);
  }
}

struct TileCoord {
  int64_t b, mt, nt;
};

// Linear workgroup id w of n -> linear work index, so that the workgroups one
// XCD receives (w = xcd, xcd + 8, ...) take a contiguous run of the work; a
// bijection for any count.
__device__ __forceinline__ int64_t xcd_run(int64_t w, int64_t n) {
  const int64_t q = n / kXcds, r = n % kXcds;
  const int64_t xcd = w % kXcds, k = w / kXcds;
  return xcd * q + (xcd < r ? xcd : r) + k;
}

// Linear tile index t -> (batch, M tile, N tile), in bands of kGroupM M tiles.
__device__ __forceinline__ TileCoord tile_at(int64_t t, int64_t MT, int64_t NT) {
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

template <int TM, int TN, int DT, int KA, bool kHasC, bool kScaled>
__global__ __launch_bounds__((Tile<TM, TN>::kWaves * kWave))
__attribute__((amdgpu_waves_per_eu(2))) void mma_tiled_kernel(MmaArgs p, int64_t n_tiles,
                                                              int64_t MT, int64_t NT) {
  using T = Tile<TM, TN>;
  using Stage = bmm::Stage<TM, TN>;
  constexpr int kWaves = T::kWaves, kWaveBlocksM = T::kWaveBlocksM, kWaveBlocksN = T::kWaveBlocksN;
  constexpr int kTileMAtoms = T::kTileMAtoms, kTileNAtoms = T::kTileNAtoms;
  constexpr int kLoadsA = T::kLoadsA, kLoadsB = T::kLoadsB, kLoadsPerSlab = T::kLoadsPerSlab;
  // Four separate objects (not one array) so that the compiler can tell the
  // ring slots apart when it places waits for the direct-to-LDS loads.
  __shared__ __attribute__((aligned(1024))) Stage st0, st1, st2, st3;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / T::kWavesN, wn = wave % T::kWavesN;
  // Work item of this workgroup. With splits, the (split, tile) pairs are laid
  // out split by split and each XCD takes a contiguous run of them, so the
  // workgroups sharing an XCD's L2 share their K range and most of their A and
  // B panels (1024 x 1024 x 65536, 16 splits: 2 splits x 16 tiles per XCD,
  // instead of 2 tiles of every split).
  const int64_t lin = int64_t(blockIdx.y) * n_tiles + blockIdx.x;
  const int64_t work = xcd_run(lin, n_tiles * int64_t(p.splits > 1 ? p.splits : 1));
  const int64_t split = work / n_tiles;
  const TileCoord tc = tile_at(work % n_tiles, MT, NT);
  const int64_t m_atom0 = tc.mt * kTileMAtoms, n_atom0 = tc.nt * kTileNAtoms;

  // ---- direct-to-LDS staging ----
  // Wave w loads fragments f = 8r + w of A and of B (f = 4r + w for the
  // 4-wave tile), one 1 KB fragment per load.
  // - 16x16x32 (8 waves): A fragment f is M atom f, 16 rows x 32 K values
  //   (two adjacent K atoms: 1 KB contiguous in HBM); B fragment f is N atoms
  //   2f and 2f + 1, 16 columns x 32 K. Lane l fetches row l % 16 (B: row l % 8
  //   of N atom 2f + (l / 8) % 2) with the 8 K values of chunk l / 16.
  // - 32x32x16 (4 waves): fragment f covers 32-row block f / 2 and the
  //   16-deep half f % 2 = w % 2 of the slab. Lane l of an A fragment fetches
  //   row l % 16 of M atom 2 * (f / 2) + (l / 16) % 2, and of a B fragment row
  //   l % 8 of N atom 4 * (f / 2) + (l / 8) % 4; in both, the 8 K values of
  //   chunk cs = 2 * (f % 2) + l / 32 of the slab's four 8-value chunks.
  // In both maps a chunk is atom chunk / 2, half chunk % 2 of the k = 16
  // layout, or atom chunk of the k = 8 layout.
  const int kj = wave & 1;
  const int cs = 2 * kj + (lane >> 5);
  const int64_t nck = k_chunks(p);
  // Split-K: split s sums the 32-value steps
  // [s * steps / S, (s + 1) * steps / S) and writes its partial sum to
  // D + s * part_floats; without splits the whole K goes to D.
  int64_t kc0 = 0, kcn = nck;  // first 8-value chunk and chunk count of this split
  float* const Dout = p.splits > 1 ? p.D + split * p.part_floats : p.D;
  if (p.splits > 1) {
    const int64_t sp = split;
    kc0 = 4 * (sp * p.steps / p.splits);
    const int64_t kc1 = 4 * ((sp + 1) * p.steps / p.splits);
    kcn = (kc1 < nck ? kc1 : nck) - kc0;
  }
  const int64_t a_row_bytes = nck * 256, b_row_bytes = nck * 128;
  const int64_t a_left = (p.M_rep - m_atom0) * a_row_bytes - kc0 * 256;
  const int64_t b_left = (p.N_rep - n_atom0) * b_row_bytes - kc0 * 128;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(p.A + (tc.b * p.M_rep + m_atom0) * nck * 64 + kc0 * 64), 0,
      int(a_left < kOutOfRange ? a_left : kOutOfRange), kBufferFlags);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(p.B + (tc.b * p.N_rep + n_atom0) * nck * 32 + kc0 * 32), 0,
      int(b_left < kOutOfRange ? b_left : kOutOfRange), kBufferFlags);
  // Fixed-size arrays: a size that depends on the template arguments, in an
  // array the lambda below captures, makes the host-side compilation drop the
  // kernel's launch stub without a diagnostic.
  constexpr int kMaxLoads = 2;
  static_assert(kLoadsA <= kMaxLoads && kLoadsB <= kMaxLoads, "offset arrays too small");
  uint32_t a_voff[kMaxLoads], b_voff[kMaxLoads];
  constexpr bool kM16 = kWaves == 8;   // the ping-pong path multiplies with 16x16x32
  const int g16 = lane >> 4;           // its lanes' 8-value chunk of the slab
  if constexpr (kM16) {
#pragma unroll
    for (int r = 0; r < kLoadsA; ++r) {
      const int f = kWaves * r + wave;
      a_voff[r] = uint32_t(f * a_row_bytes +
                           (KA == 16 ? (g16 >> 1) * 512 + (lane & 15) * 32 + (g16 & 1) * 16
                                     : g16 * 256 + (lane & 15) * 16));
    }
#pragma unroll
    for (int r = 0; r < kLoadsB; ++r) {
      const int f = kWaves * r + wave;
      b_voff[r] = uint32_t((2 * f + ((lane >> 3) & 1)) * b_row_bytes +
                           (KA == 16 ? (g16 >> 1) * 256 + (lane & 7) * 32 + (g16 & 1) * 16
                                     : g16 * 128 + (lane & 7) * 16));
    }
  } else {
#pragma unroll
    for (int r = 0; r < kLoadsA; ++r) {
      const int blk = (kWaves * r + wave) >> 1;
      a_voff[r] = uint32_t((2 * blk + ((lane >> 4) & 1)) * a_row_bytes +
                           (KA == 16 ? kj * 512 + (lane & 15) * 32 + (lane >> 5) * 16
                                     : cs * 256 + (lane & 15) * 16));
    }
#pragma unroll
    for (int r = 0; r < kLoadsB; ++r) {
      const int blk = (kWaves * r + wave) >> 1;
      b_voff[r] = uint32_t((4 * blk + ((lane >> 3) & 3)) * b_row_bytes +
                           (KA == 16 ? kj * 256 + (lane & 7) * 32 + (lane >> 5) * 16
                                     : cs * 128 + (lane & 7) * 16));
    }
  }

  // Loads of slab k into stage st (slabs past the end, and K chunks past it,
  // read 0). With k = 16 atoms both halves of an atom are valid together; in
  // the 32x32x16 map the test is then uniform over the wave.
  auto issue = [&](Stage& st, int64_t k) {
    const uint32_t koff_a = uint32_t(k * 1024), koff_b = uint32_t(k * 512);
    const bool k_ok = kM16 ? 4 * k + g16 < kcn : KA == 16 ? 4 * k + 2 * kj < kcn : 4 * k + cs < kcn;
#pragma unroll
    for (int r = 0; r < kLoadsA; ++r)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          a_rsrc, (__attribute__((address_space(3))) void*)&st.a[kWaves * r + wave][0], 16,
          k_ok ? a_voff[r] : kOutOfRange, koff_a, 0, 0);
#pragma unroll
    for (int r = 0; r < kLoadsB; ++r)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          b_rsrc, (__attribute__((address_space(3))) void*)&st.b[kWaves * r + wave][0], 16,
          k_ok ? b_voff[r] : kOutOfRange, koff_b, 0, 0);
  };

  if constexpr (kM16) {
    // ---- two groups in ping-pong, 16x16x32 (schedule above) ----
    // Wave (wm, wn) owns 16-row blocks pm and 16-column blocks qn of D; lane l
    // carries row l % 16 of each block and its columns 4 * (l / 16) .. + 3:
    // one 16-byte piece of one accumulator atom per block.
    constexpr int kBM = T::kWaveBlocksM * 2, kBN = 4;   // 16-row / 16-column blocks per wave
    f32x4 acc[kBM][kBN];
    const int64_t lane_row_atom = m_atom0 + kBM * wm;                      // + pm
    const int64_t lane_col_atom = n_atom0 + 2 * kBN * wn + (g16 >> 1);     // + 2 qn
    const bool interior = m_atom0 + kTileMAtoms <= p.M_rep && n_atom0 + kTileNAtoms <= p.N_rep;
    const int64_t d_lane =
        (((tc.b * p.M_rep + lane_row_atom) * p.N_rep + lane_col_atom) * 16 + (lane & 15)) * 8 +
        4 * (g16 & 1);
    const int64_t d_mstride = p.N_rep * kAtomFloats;  // next M atom
    auto init_acc = [&]() {
      if constexpr (kScaled) {
#pragma unroll
        for (int pm = 0; pm < kBM; ++pm)
#pragma unroll
          for (int qn = 0; qn < kBN; ++qn) acc[pm][qn] = f32x4{0.f, 0.f, 0.f, 0.f};
      } else if constexpr (kHasC) {
        if (interior) {
          const float* cl = p.C + d_lane;
#pragma unroll
          for (int pm = 0; pm < kBM; ++pm)
#pragma unroll
            for (int qn = 0; qn < kBN; ++qn)
              acc[pm][qn] = load16f_nt(cl + pm * d_mstride + 2 * qn * kAtomFloats);
        } else {
#pragma unroll
          for (int pm = 0; pm < kBM; ++pm)
#pragma unroll
            for (int qn = 0; qn < kBN; ++qn) {
              const int64_t ra = lane_row_atom + pm, ca = lane_col_atom + 2 * qn;
              const int64_t ma = ra < p.M_rep ? ra : p.M_rep - 1;
              const int64_t na = ca < p.N_rep ? ca : p.N_rep - 1;
              acc[pm][qn] = load16f_nt(p.C + (((tc.b * p.M_rep + ma) * p.N_rep + na) * 16 +
                                              (lane & 15)) * 8 + 4 * (g16 & 1));
            }
        }
      } else {
#pragma unroll
        for (int pm = 0; pm < kBM; ++pm)
#pragma unroll
          for (int qn = 0; qn < kBN; ++qn)
            acc[pm][qn] = f32x4{p.c_scalar, p.c_scalar, p.c_scalar, p.c_scalar};
      }
    };
    auto sync = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
    };
    const int64_t n_slabs = (kcn + 3) / 4;
    u32x4 F[kBN + kBM];   // this wave's fragments of one slab: B blocks, then A blocks
    auto read_slab = [&](const Stage& st) {
#pragma unroll
      for (int i = 0; i < kBN; ++i)
        F[i] = *(const volatile lds_u32x4*)&st.b[kBN * wn + i][lane];
#pragma unroll
      for (int i = 0; i < kBM; ++i)
        F[kBN + i] = *(const volatile lds_u32x4*)&st.a[kBM * wm + i][lane];
    };
    auto mfma_slab = [&]() {
#pragma unroll
      for (int pm = 0; pm < kBM; ++pm)
#pragma unroll
        for (int qn = 0; qn < kBN; ++qn)
          acc[pm][qn] = mfma_16x16x32<DT>(F[qn], F[kBN + pm], acc[pm][qn]);
    };
    // Ring invariant: a group's own loads of a slab are waited for (counted
    // vmcnt) in its memory phase two slabs before the slab is read, and the
    // barrier ending that phase publishes them. A stage is reloaded only in a
    // phase after both groups' reads of it have completed (lgkmcnt(0)) and a
    // barrier has passed.
    // Each group does its own set-up so the register allocator sees two simple
    // straight-line loops. The group test must be uniform (a scalar branch):
    // a wave may never run the other group's barriers with its lanes masked off.
    const bool group0 = __builtin_amdgcn_readfirstlane(wave) < 4;
    if (group0) {
      init_acc();
      issue(st0, 0);
      issue(st1, 1);
      issue(st2, 2);
      issue(st3, 3);
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(3 * kLoadsPerSlab, 15));  // C, slab 0 landed
      sync();
      read_slab(st0);
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * kLoadsPerSlab, 0));  // slab 1 landed
      sync();
      auto slab = [&](int64_t t, Stage& cur, const Stage& next) {
        mfma_slab();                                                     // phase 0
        sync();
        read_slab(next);                                                 // phase 1
        issue(cur, t + 4);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * kLoadsPerSlab, 0));  // slab t+2 landed
        sync();
      };
      for (int64_t s = 0; s < n_slabs; s += kStages) {
        slab(s + 0, st0, st1);
        slab(s + 1, st1, st2);
        slab(s + 2, st2, st3);
        slab(s + 3, st3, st0);
      }
    } else {
      init_acc();
      issue(st0, 0);
      issue(st1, 1);
      issue(st2, 2);
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * kLoadsPerSlab, 15));  // C, slab 0 landed
      sync();
      sync();
      auto slab = [&](int64_t t, Stage& prev, const Stage& cur) {
        read_slab(cur);                                                  // phase 0
        issue(prev, t + 3);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * kLoadsPerSlab, 0));  // slab t+1 landed
        sync();
        mfma_slab();                                                     // phase 1
        sync();
      };
      for (int64_t s = 0; s < n_slabs; s += kStages) {
        slab(s + 0, st3, st0);
        slab(s + 1, st0, st1);
        slab(s + 2, st1, st2);
        slab(s + 3, st2, st3);
      }
    }
    // No load may still be writing LDS when the workgroup ends.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

    // ---- epilogue: one 16-byte store per block ----
    // With alpha/beta and a C tensor, the C blocks of a group of kEpi blocks are
    // all requested before the group's stores, so their reads overlap instead of
    // waiting one by one. (D may be C: every element's C is read before its own
    // D is written.)
    constexpr int kEpi = kBM * kBN < 16 ? kBM * kBN : 16;
#pragma unroll
    for (int g0 = 0; g0 < kBM * kBN; g0 += kEpi) {
      f32x4 cv[16];   // fixed size: used up to kEpi
#pragma unroll
      for (int j = 0; j < kEpi; ++j) {
        cv[j] = f32x4{p.c_scalar, p.c_scalar, p.c_scalar, p.c_scalar};
        if constexpr (kScaled && kHasC) {
          // no branch around the read (lanes past the edge read a clamped,
          // in-bounds block and store nothing): a branch per read would make
          // each read wait for the previous one
          const int pm = (g0 + j) / kBN, qn = (g0 + j) % kBN;
          const int64_t ra = lane_row_atom + pm, ca = lane_col_atom + 2 * qn;
          const int64_t off =
              interior ? d_lane + pm * d_mstride + 2 * qn * kAtomFloats
                       : (((tc.b * p.M_rep + (ra < p.M_rep ? ra : p.M_rep - 1)) * p.N_rep +
                           (ca < p.N_rep ? ca : p.N_rep - 1)) * 16 + (lane & 15)) * 8 +
                             4 * (g16 & 1);
          cv[j] = load16f_nt(p.C + off);
        }
      }
#pragma unroll
      for (int j = 0; j < kEpi; ++j) {
        const int pm = (g0 + j) / kBN, qn = (g0 + j) % kBN;
        f32x4 v = acc[pm][qn];
        float* dst = Dout + d_lane + pm * d_mstride + 2 * qn * kAtomFloats;
        const bool ok =
            interior || (lane_row_atom + pm < p.M_rep && lane_col_atom + 2 * qn < p.N_rep);
        if constexpr (kScaled) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(p.alpha, v[e], p.beta * cv[j][e]);
        }
        if (ok) {
          if (p.splits > 1)
            store16f(dst, v);   // partial sums: read back by the reduce right away
          else
            store16f_nt(dst, v);
        }
      }
    }
  } else {
  // ---- accumulators: C (read once, here) or the scalar ----
    // Block (pm, qn) of the wave: rows 32 * (4 wm + pm) .. +31, columns
    // 32 * (2 wn + qn) .. +31 of the tile. Lane l, register 4q + t: row l % 32,
    // column 8q + 4 (l / 32) + t of the block.
    f32x16 acc[kWaveBlocksM][kWaveBlocksN];
    const int64_t lane_row_atom = m_atom0 + 2 * (kWaveBlocksM * wm) + ((lane >> 4) & 1);  // + 2 pm
    const int64_t lane_col_atom = n_atom0 + 4 * (kWaveBlocksN * wn);                     // + 4 qn + q
    const bool interior = m_atom0 + kTileMAtoms <= p.M_rep && n_atom0 + kTileNAtoms <= p.N_rep;
    const int64_t d_lane =
        (((tc.b * p.M_rep + lane_row_atom) * p.N_rep + lane_col_atom) * 16 + (lane & 15)) * 8 +
        4 * (lane >> 5);
    const int64_t d_mstride = p.N_rep * kAtomFloats;  // next M atom
    auto init_acc = [&]() {
      if constexpr (kScaled) {
        // alpha/beta form: the product starts from zero, C is read in the epilogue
#pragma unroll
        for (int pm = 0; pm < kWaveBlocksM; ++pm)
#pragma unroll
          for (int qn = 0; qn < kWaveBlocksN; ++qn) acc[pm][qn] = f32x16{};
      } else if constexpr (kHasC) {
        auto set4 = [&](int pm, int qn, int q, f32x4 v) {
          acc[pm][qn][4 * q + 0] = v[0];
          acc[pm][qn][4 * q + 1] = v[1];
          acc[pm][qn][4 * q + 2] = v[2];
          acc[pm][qn][4 * q + 3] = v[3];
        };
        if (interior) {
          // one lane address; the pieces differ by constants and a uniform stride
          const float* cl = p.C + d_lane;
#pragma unroll
          for (int pm = 0; pm < kWaveBlocksM; ++pm)
#pragma unroll
            for (int qn = 0; qn < kWaveBlocksN; ++qn)
#pragma unroll
              for (int q = 0; q < 4; ++q)
                set4(pm, qn, q, load16f_nt(cl + 2 * pm * d_mstride + (4 * qn + q) * kAtomFloats));
        } else {
          // Blocks outside a ragged last tile read a clamped (valid) address:
          // their accumulators are never stored.
#pragma unroll
          for (int pm = 0; pm < kWaveBlocksM; ++pm)
#pragma unroll
            for (int qn = 0; qn < kWaveBlocksN; ++qn)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int64_t ra = lane_row_atom + 2 * pm, ca = lane_col_atom + 4 * qn + q;
                const int64_t ma = ra < p.M_rep ? ra : p.M_rep - 1;
                const int64_t na = ca < p.N_rep ? ca : p.N_rep - 1;
                set4(pm, qn, q, load16f_nt(p.C + (((tc.b * p.M_rep + ma) * p.N_rep + na) * 16 +
                                                  (lane & 15)) * 8 + 4 * (lane >> 5)));
              }
        }
      } else {
#pragma unroll
        for (int pm = 0; pm < kWaveBlocksM; ++pm)
#pragma unroll
          for (int qn = 0; qn < kWaveBlocksN; ++qn)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[pm][qn][e] = p.c_scalar;
      }
    };

    // ---- one group (128 x 128 tile) ----
      init_acc();
      // Slabs 0..3 into the ring; C (issued first) and slab 0 must have landed.
      issue(st0, 0);
      issue(st1, 1);
      issue(st2, 2);
      issue(st3, 3);
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(3 * kLoadsPerSlab, 15));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
  
      // Fragments of one slab: [K half][block]. Reads are volatile LDS loads so
      // they stay where they are written (a half slab ahead of their MFMAs)
      // instead of being sunk to their first use.
      using FragB = u32x4[2][kWaveBlocksN];
      using FragA = u32x4[2][kWaveBlocksM];
      FragB fb[2];
      FragA fa[2];
      auto read_frags = [&](const Stage& st, FragB& b, FragA& a) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int i = 0; i < kWaveBlocksN; ++i)
            b[j][i] = *(const volatile lds_u32x4*)&st.b[2 * (kWaveBlocksN * wn + i) + j][lane];
#pragma unroll
          for (int i = 0; i < kWaveBlocksM; ++i)
            a[j][i] = *(const volatile lds_u32x4*)&st.a[2 * (kWaveBlocksM * wm + i) + j][lane];
        }
      };
      auto mfma_katom = [&](const u32x4 (&b)[kWaveBlocksN], const u32x4 (&a)[kWaveBlocksM]) {
#pragma unroll
        for (int pm = 0; pm < kWaveBlocksM; ++pm)
#pragma unroll
          for (int qn = 0; qn < kWaveBlocksN; ++qn)
            acc[pm][qn] = mfma_32x32x16<DT>(b[qn], a[pm], acc[pm][qn]);
      };
  
      read_frags(st0, fb[0], fa[0]);
  
      auto slab = [&](int64_t s, Stage& cur, const Stage& nxt, FragB& bc, FragA& ac, FragB& bn,
                      FragA& an) {
        __builtin_amdgcn_sched_barrier(0);
        mfma_katom(bc[0], ac[0]);
        // own loads of slab s+1 landed (slabs s+2, s+3 may still be in flight);
        // own fragment reads of this stage done
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * kLoadsPerSlab, 0));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        issue(cur, s + kStages);
        read_frags(nxt, bn, an);
        mfma_katom(bc[1], ac[1]);
        // The compiler interleaves these: the MFMAs of the second K half go
        // first, so the pipe has work right after the barrier, with the loads of
        // slab s+4 and the next slab's fragment reads spread among them.
      };
      const int64_t n_slabs = (kcn + 3) / 4;
      for (int64_t s = 0; s < n_slabs; s += kStages) {
        slab(s + 0, st0, st1, fb[0], fa[0], fb[1], fa[1]);
        slab(s + 1, st1, st2, fb[1], fa[1], fb[0], fa[0]);
        slab(s + 2, st2, st3, fb[0], fa[0], fb[1], fa[1]);
        slab(s + 3, st3, st0, fb[1], fa[1], fb[0], fa[0]);
      }
    // No load may still be writing LDS when the workgroup ends.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  
    // ---- epilogue: per block, four 16-byte stores (one per N atom) ----
    // With alpha/beta and a C tensor, all of the wave's C reads are requested
    // before its stores (D may be C: every element's C is read before its own D
    // is written).
    constexpr int kStores = kWaveBlocksM * kWaveBlocksN * 4;
    static_assert(kStores <= 16, "one batch of C reads");
    f32x4 cv[16];   // fixed size: used up to kStores
#pragma unroll
    for (int j = 0; j < kStores; ++j) {
      cv[j] = f32x4{p.c_scalar, p.c_scalar, p.c_scalar, p.c_scalar};
      if constexpr (kScaled && kHasC) {
        // no branch around the read: lanes past the edge read a clamped block
        const int pm = j / (4 * kWaveBlocksN), qn = (j / 4) % kWaveBlocksN, q = j % 4;
        const int64_t ra = lane_row_atom + 2 * pm, ca = lane_col_atom + 4 * qn + q;
        const int64_t off =
            interior ? d_lane + 2 * pm * d_mstride + (4 * qn + q) * kAtomFloats
                     : (((tc.b * p.M_rep + (ra < p.M_rep ? ra : p.M_rep - 1)) * p.N_rep +
                         (ca < p.N_rep ? ca : p.N_rep - 1)) * 16 + (lane & 15)) * 8 +
                           4 * (lane >> 5);
        cv[j] = load16f_nt(p.C + off);
      }
    }
#pragma unroll
    for (int j = 0; j < kStores; ++j) {
      const int pm = j / (4 * kWaveBlocksN), qn = (j / 4) % kWaveBlocksN, q = j % 4;
      f32x4 v = {acc[pm][qn][4 * q + 0], acc[pm][qn][4 * q + 1], acc[pm][qn][4 * q + 2],
                 acc[pm][qn][4 * q + 3]};
      float* dst = Dout + d_lane + 2 * pm * d_mstride + (4 * qn + q) * kAtomFloats;
      const bool ok =
          interior || (lane_row_atom + 2 * pm < p.M_rep && lane_col_atom + 4 * qn + q < p.N_rep);
      if constexpr (kScaled) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(p.alpha, v[e], p.beta * cv[j][e]);
      }
      if (ok) {
        if (p.splits > 1)
          store16f(dst, v);   // partial sums: read back by the reduce right away
        else
          store16f_nt(dst, v);
      }
    }
  }
}

// TM x TN tiles without split-K or alpha/beta: 4 waves in a 2 x 2 grid, each
// TM/2 x TN/2 of D as TM/32 x TN/32 blocks of 16 x 16 (256 x 256: 64
// accumulators of 4 floats, all 256 accumulator registers; 256 x 128: 32;
// 128 x 128: 16), and v_mfma_f32_16x16x32. Fragment maps, LDS image and ring
// are those of the ping-pong tiles; each wave loads fragments f = 4 r + wave
// of a slab. Per slab a wave multiplies TN/32 B and TM/32 A fragments
// (256 x 256: 16 reads for 64 MFMAs, against 12 for 32 in the ping-pong
// tiles). The next slab's fragments go to a second register set while the
// current one is multiplied. 256-row tiles run one workgroup per CU (one wave
// per SIMD); 128 x 128 tiles (64 KB of LDS) two.
template <int TM, int TN, int DT, int KA, bool kHasC, bool kScaled>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(TM == 256 ? 1 : 2, TM == 256 ? 1 : 2)))
void mma_tiled4_kernel(MmaArgs p, int64_t n_tiles, int64_t MT, int64_t NT) {
  using T = Tile<TM, TN>;
  using St = Stage<TM, TN>;
  constexpr int kW = 4;                               // waves
  constexpr int kTileMAtoms = T::kTileMAtoms, kTileNAtoms = T::kTileNAtoms;
  constexpr int kBM = TM / 32;                        // 16-row blocks per wave (TM / 2 rows)
  constexpr int kBN = TN / 32;                        // 16-column blocks per wave (TN / 2 columns)
  constexpr int kLoadsA = TM / 64, kLoadsB = TN / 64; // fragments a wave loads per slab
  constexpr int kLoads = kLoadsA + kLoadsB;           // direct-to-LDS loads per wave per slab
  __shared__ __attribute__((aligned(1024))) St st0, st1, st2, st3;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave >> 1, wn = wave & 1;
  const int g16 = lane >> 4;
  const int64_t work = xcd_run(blockIdx.x, n_tiles);
  const TileCoord tc = tile_at(work, MT, NT);
  const int64_t m_atom0 = tc.mt * kTileMAtoms, n_atom0 = tc.nt * kTileNAtoms;
  const int64_t kcn = k_chunks(p);
  const int64_t a_row_bytes = kcn * 256, b_row_bytes = kcn * 128;
  const int64_t a_left = (p.M_rep - m_atom0) * a_row_bytes;
  const int64_t b_left = (p.N_rep - n_atom0) * b_row_bytes;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(p.A + (tc.b * p.M_rep + m_atom0) * kcn * 64), 0,
      int(a_left < kOutOfRange ? a_left : kOutOfRange), kBufferFlags);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(p.B + (tc.b * p.N_rep + n_atom0) * kcn * 32), 0,
      int(b_left < kOutOfRange ? b_left : kOutOfRange), kBufferFlags);
  // 16x16x32 gather offsets, as in the ping-pong tiles.
  // Fixed sizes here and below (used up to kLoadsA/B, kBM, kBN, kF): arrays sized by a
  // template argument and captured by a lambda make the host-side compilation
  // drop the kernel's launch stub without a diagnostic.
  uint32_t a_voff[4], b_voff[4];
#pragma unroll
  for (int r = 0; r < kLoadsA; ++r) {
    const int f = kW * r + wave;
    a_voff[r] = uint32_t(f * a_row_bytes +
                         (KA == 16 ? (g16 >> 1) * 512 + (lane & 15) * 32 + (g16 & 1) * 16
                                   : g16 * 256 + (lane & 15) * 16));
  }
#pragma unroll
  for (int r = 0; r < kLoadsB; ++r) {
    const int f = kW * r + wave;
    b_voff[r] = uint32_t((2 * f + ((lane >> 3) & 1)) * b_row_bytes +
                         (KA == 16 ? (g16 >> 1) * 256 + (lane & 7) * 32 + (g16 & 1) * 16
                                   : g16 * 128 + (lane & 7) * 16));
  }
  auto issue = [&](St& st, int64_t k) {
    const uint32_t koff_a = uint32_t(k * 1024), koff_b = uint32_t(k * 512);
    const bool k_ok = 4 * k + g16 < kcn;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r < kLoadsA)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            a_rsrc, (__attribute__((address_space(3))) void*)&st.a[kW * r + wave][0], 16,
            k_ok ? a_voff[r] : kOutOfRange, koff_a, 0, 0);
      if (r < kLoadsB)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            b_rsrc, (__attribute__((address_space(3))) void*)&st.b[kW * r + wave][0], 16,
            k_ok ? b_voff[r] : kOutOfRange, koff_b, 0, 0);
    }
  };

  // Wave (wm, wn) owns 16-row blocks pm and 16-column blocks qn of D; lane l
  // carries row l % 16 of each block and its columns 4 * (l / 16) .. + 3.
  f32x4 acc[8][8];                  // [pm][qn], pm < kBM, qn < kBN
  const int64_t lane_row_atom = m_atom0 + kBM * wm;                // + pm
  const int64_t lane_col_atom = n_atom0 + 2 * kBN * wn + (g16 >> 1);   // + 2 qn
  const bool interior = m_atom0 + kTileMAtoms <= p.M_rep && n_atom0 + kTileNAtoms <= p.N_rep;
  const int64_t d_lane =
      (((tc.b * p.M_rep + lane_row_atom) * p.N_rep + lane_col_atom) * 16 + (lane & 15)) * 8 +
      4 * (g16 & 1);
  const int64_t d_mstride = p.N_rep * kAtomFloats;   // next M atom
  if constexpr (kHasC && !kScaled) {
    if (interior) {
      const float* cl = p.C + d_lane;
#pragma unroll
      for (int pm = 0; pm < kBM; ++pm)
#pragma unroll
        for (int qn = 0; qn < kBN; ++qn)
          acc[pm][qn] = load16f_nt(cl + pm * d_mstride + 2 * qn * kAtomFloats);
    } else {
#pragma unroll
      for (int pm = 0; pm < kBM; ++pm)
#pragma unroll
        for (int qn = 0; qn < kBN; ++qn) {
          const int64_t ra = lane_row_atom + pm, ca = lane_col_atom + 2 * qn;
          const int64_t ma = ra < p.M_rep ? ra : p.M_rep - 1;
          const int64_t na = ca < p.N_rep ? ca : p.N_rep - 1;
          acc[pm][qn] = load16f_nt(p.C + (((tc.b * p.M_rep + ma) * p.N_rep + na) * 16 +
                                          (lane & 15)) * 8 + 4 * (g16 & 1));
        }
    }
  } else {
#pragma unroll
    for (int pm = 0; pm < kBM; ++pm)
#pragma unroll
      for (int qn = 0; qn < kBN; ++qn) {
        // Pinned to accumulator registers one by one: equal starting values
        // would otherwise be merged, and the loop would then copy them. (The
        // alpha/beta form starts the product from zero; C enters at the end.)
        const float c0 = kScaled ? 0.f : p.c_scalar;
        f32x4 v = f32x4{c0, c0, c0, c0};
        asm volatile("" : "+a"(v));
        acc[pm][qn] = v;
      }
  }

  constexpr int kF = kBN + kBM;
  u32x4 F0[16], F1[16];   // one slab's fragments: B blocks 0..kBN-1, then A blocks 0..kBM-1
  auto read_slab = [&](const St& st, u32x4 (&F)[16]) {
#pragma unroll
    for (int i = 0; i < kBN; ++i) F[i] = *(const volatile lds_u32x4*)&st.b[kBN * wn + i][lane];
#pragma unroll
    for (int i = 0; i < kBM; ++i) F[kBN + i] = *(const volatile lds_u32x4*)&st.a[kBM * wm + i][lane];
  };
  auto mma = [&](int pm, int qn, const u32x4 (&F)[16]) {
    acc[pm][qn] = mfma_16x16x32<DT>(F[qn], F[kBN + pm], acc[pm][qn]);
  };
  const int64_t n_slabs = (kcn + 3) / 4;
  issue(st0, 0);
  issue(st1, 1);
  issue(st2, 2);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * kLoads, 15));   // C, slab 0 landed
  __builtin_amdgcn_s_barrier();
  read_slab(st0, F0);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(kLoads, 0));        // slab 1 landed, F0 read
  // Slab s multiplies Fc. The barrier after its first two MFMAs publishes every
  // wave's loads of slab s+1 (each wave waited for its own at the end of slab
  // s-1) while those two MFMAs run; after it the wave reads slab s+1 into Fn
  // and loads slab s+3 into the stage that slab s-1 has left (its reads ended
  // with lgkmcnt(0) before the previous barrier). The scheduling groups place
  // a fragment read after every second MFMA, then a load after every third.
  auto slab = [&](int64_t s, const St& st_next, St& st_load, const u32x4 (&Fc)[16],
                  u32x4 (&Fn)[16]) {
    __builtin_amdgcn_sched_barrier(0);
    mma(0, 0, Fc);
    mma(0, 1, Fc);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    read_slab(st_next, Fn);
    issue(st_load, s + 3);
#pragma unroll
    for (int i = 2; i < kBM * kBN; ++i) mma(i / kBN, i % kBN, Fc);
    // 256 x 256 (64 MFMAs): a read after every second MFMA, then a load after
    // every third; 256 x 128 (32 MFMAs): a read after every MFMA, then a load
    // after every third; 128 x 128 (16 MFMAs): a read, then a load, after every MFMA.
    constexpr int kPerRead = kBM * kBN >= 64 ? 2 : 1;
    constexpr int kPerLoad = kBM * kBN >= 32 ? 3 : 1;
#pragma unroll
    for (int i = 0; i < kF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, kPerRead, 0);   // MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);          // 1 LDS read
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, kPerLoad, 0);   // MFMAs
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // 1 vector memory read
    }
    constexpr int kRest = kBM * kBN - 2 - kPerRead * kF - kPerLoad * kLoads;
    static_assert(kRest >= 0, "the slab's MFMAs cover its reads and loads");
    if constexpr (kRest > 0) __builtin_amdgcn_sched_group_barrier(0x008, kRest, 0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(kLoads, 0));   // own slab s+2 landed, Fn read
  };
  for (int64_t s = 0; s < n_slabs; s += kStages) {
    slab(s + 0, st1, st3, F0, F1);
    slab(s + 1, st2, st0, F1, F0);
    slab(s + 2, st3, st1, F0, F1);
    slab(s + 3, st0, st2, F1, F0);
  }
  // No load may still be writing LDS when the workgroup ends.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  if constexpr (!kScaled) {
#pragma unroll
    for (int pm = 0; pm < kBM; ++pm)
#pragma unroll
      for (int qn = 0; qn < kBN; ++qn) {
        const bool ok =
            interior || (lane_row_atom + pm < p.M_rep && lane_col_atom + 2 * qn < p.N_rep);
        if (ok) store16f_nt(p.D + d_lane + pm * d_mstride + 2 * qn * kAtomFloats, acc[pm][qn]);
      }
  } else {
    // alpha/beta: D = fma(alpha, product, beta * C), one rounding after the
    // product. The C blocks of a group of up to 16 are all requested, with no
    // branch around the reads (lanes past the edge read a clamped block and
    // store nothing), before the group's stores, so that the reads overlap.
    // (D may be C: every element's C is read before its own D is written.)
    constexpr int kEpi = kBM * kBN < 16 ? kBM * kBN : 16;
#pragma unroll
    for (int g0 = 0; g0 < kBM * kBN; g0 += kEpi) {
      f32x4 cv[16];   // fixed size: used up to kEpi
#pragma unroll
      for (int j = 0; j < kEpi; ++j) {
        cv[j] = f32x4{p.c_scalar, p.c_scalar, p.c_scalar, p.c_scalar};
        if constexpr (kHasC) {
          const int pm = (g0 + j) / kBN, qn = (g0 + j) % kBN;
          const int64_t ra = lane_row_atom + pm, ca = lane_col_atom + 2 * qn;
          const int64_t off =
              interior ? d_lane + pm * d_mstride + 2 * qn * kAtomFloats
                       : (((tc.b * p.M_rep + (ra < p.M_rep ? ra : p.M_rep - 1)) * p.N_rep +
                           (ca < p.N_rep ? ca : p.N_rep - 1)) * 16 + (lane & 15)) * 8 +
                             4 * (g16 & 1);
          cv[j] = load16f_nt(p.C + off);
        }
      }
#pragma unroll
      for (int j = 0; j < kEpi; ++j) {
        const int pm = (g0 + j) / kBN, qn = (g0 + j) % kBN;
        f32x4 v = acc[pm][qn];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(p.alpha, v[e], p.beta * cv[j][e]);
        const bool ok =
            interior || (lane_row_atom + pm < p.M_rep && lane_col_atom + 2 * qn < p.N_rep);
        if (ok) store16f_nt(p.D + d_lane + pm * d_mstride + 2 * qn * kAtomFloats, v);
      }
    }
  }
}

template <int TM, int TN>
hipError_t launch_tm(const MmaArgs& a, hipStream_t s) {
  constexpr int kTileMAtoms = Tile<TM, TN>::kTileMAtoms, kTileNAtoms = Tile<TM, TN>::kTileNAtoms;
  const int64_t MT = (a.M_rep + kTileMAtoms - 1) / kTileMAtoms;
  const int64_t NT = (a.N_rep + kTileNAtoms - 1) / kTileNAtoms;
  const int64_t n_tiles = a.batch * MT * NT;
  if (n_tiles > 0x7fffffff) return hipErrorInvalidConfiguration;
  // Buffer offsets inside one tile's atom rows must stay below 2^31.
  if (k_chunks(a) * 8 >= kTiledMaxK) return hipErrorInvalidValue;
  auto pick = [&](auto dt, auto ka) {
    constexpr int D = decltype(dt)::value, KA = decltype(ka)::value;
    if (a.scaled)
      return a.C ? mma_tiled_kernel<TM, TN, D, KA, true, true>
                 : mma_tiled_kernel<TM, TN, D, KA, false, true>;
    return a.C ? mma_tiled_kernel<TM, TN, D, KA, true, false>
               : mma_tiled_kernel<TM, TN, D, KA, false, false>;
  };
  auto pick_ka = [&](auto dt) {
    return a.atom_k == 16 ? pick(dt, std::integral_constant<int, 16>{})
                          : pick(dt, std::integral_constant<int, 8>{});
  };
  auto kern = a.dtype == kBF16 ? pick_ka(std::integral_constant<int, kBF16>{})
                               : pick_ka(std::integral_constant<int, kF16>{});
  const unsigned splits = a.splits > 1 ? unsigned(a.splits) : 1u;
  {
    // The alpha/beta form takes the 4-wave pipeline where it measured faster
    // than the ping-pong and one-group schedules (same bits): every 256 x 128
    // grid (8192 x 1024 x 8192: 111.2 against 119.4 us; 2304 x 2304 x 4096: 49.8
    // against 55.2) and 256 x 256 grids of more than one round of the chip's 256
    // CUs (8192^3: 743.7 against 754.8). One round of 256 x 256 tiles (4096^3 with
    // a C tensor: 94.2 against 92.2) and the 128 x 128 tile (2048^3: 24.3 against
    // 23.6) keep the older schedules.
    constexpr int64_t kOneRound = 256;
    const bool four_wave =
        !a.scaled || (TM == 256 && (TN == 128 || n_tiles > kOneRound));
    if (splits == 1 && four_wave) {
      auto pick4 = [&](auto dt, auto ka) {
        constexpr int D = decltype(dt)::value, KA = decltype(ka)::value;
        if (a.scaled)
          return a.C ? mma_tiled4_kernel<TM, TN, D, KA, true, true>
                     : mma_tiled4_kernel<TM, TN, D, KA, false, true>;
        return a.C ? mma_tiled4_kernel<TM, TN, D, KA, true, false>
                   : mma_tiled4_kernel<TM, TN, D, KA, false, false>;
      };
      auto pick4_ka = [&](auto dt) {
        return a.atom_k == 16 ? pick4(dt, std::integral_constant<int, 16>{})
                              : pick4(dt, std::integral_constant<int, 8>{});
      };
      auto k4 = a.dtype == kBF16 ? pick4_ka(std::integral_constant<int, kBF16>{})
                                 : pick4_ka(std::integral_constant<int, kF16>{});
      hipLaunchKernelGGL(k4, dim3(unsigned(n_tiles)), dim3(256), 0, s, a, n_tiles, MT, NT);
      return hipGetLastError();
    }
  }
  constexpr unsigned kThreads = Tile<TM, TN>::kWaves * kWave;  // (no comma inside the macro)
  hipLaunchKernelGGL(kern, dim3(unsigned(n_tiles), splits), dim3(kThreads), 0, s, a, n_tiles, MT,
                     NT);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mma_tiled(const MmaArgs& a, hipStream_t s) {
  if (a.tile == 128) return launch_tm<128, 128>(a, s);
  return a.tile_n == 128 ? launch_tm<256, 128>(a, s) : launch_tm<256, 256>(a, s);
}

}  // namespace bmm
