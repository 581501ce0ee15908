// Row-major (or K-major) halves -> packed b32 atoms (the operand layouts of the mma.sync
// page, "Operand coordinates and ownership", built from row-major matrices as
// in the page's worked example).
//
// Eight consecutive K values of one row are, in memory, exactly the four
// packed words of half an atom row (even K in the low half of each word on
// this little-endian machine), so packing is a permutation of 16-byte chunks:
// output chunk (row block rb, c) with c = (kr, i, h) comes from source row
// R*rb + i, K offset 16*kr + 8*h (with an atom K of 8: c = (kr, i), K offset
// 8*kr).
//
// Two kernels, chosen by the size of the packed operand:
// - up to 128 MiB (half the 256 MB Infinity Cache), pack_staged_kernel: lanes
//   read whole 1 KB runs of one source row, the chunks are permuted through
//   LDS, and the workgroup's 32 KB output span is written contiguously through
//   the caches, so the multiply that reads it next finds part of it there
//   (8192^3 bf16: the whole step 3% faster than with pack_kernel and
//   streaming stores);
// - above that, pack_kernel (no LDS; row pieces of 128 bytes, 256-byte output
//   runs) with non-temporal stores, which do not flush the caches the
//   multiply then streams through (16 x 16384 x 16384: the skinny multiply
//   87 us, against 115 us after cached stores; this kernel also packs a
//   512 MiB operand 1-4% faster than the staged one).
#include "common.h"
#include "launch.h"

namespace bmm {
namespace {

constexpr int kPackThreads = 256;
constexpr int64_t kCachedPackBytes = int64_t(128) << 20;  // largest output of the staged kernel
constexpr int kPackUnroll = 4;
// The 16-row chunk order below is a permutation of 4 waves x 4 iterations x 64 lanes.
static_assert(kPackThreads == 256 && kPackUnroll == 4, "chunk order assumes 1024 chunks per block");

// pack_kernel: a block takes 1024 consecutive output chunks; the order in
// which its lanes take them (below) keeps both the row reads and the chunk
// writes in runs of 128 bytes or more.
template <int R, int KA>
__global__ __launch_bounds__(kPackThreads) void pack_kernel(uint32_t* __restrict__ dst,
                                                            const uint16_t* __restrict__ src,
                                                            int64_t rb0, int32_t chunks_per_rb,
                                                            int64_t ld) {
  constexpr int kLog2R = R == 16 ? 4 : 3;
  const int64_t rb = rb0 + blockIdx.y;
  const uint16_t* srow = src + rb * R * ld;
  uint32_t* drb = dst + rb * int64_t(chunks_per_rb) * 4;
  // Chunks of this block: a permutation of [base, base + 1024). With 8-row
  // atoms consecutive lanes take consecutive chunks, so one wave reads 8 rows
  // x 128 contiguous bytes and writes contiguous 16-byte chunks. With 16-row
  // atoms that order would read 16 rows x 64 bytes per instruction; instead a
  // wave takes 8 rows x 4 atoms x 2 halves (k = 16) or 8 rows x 8 atoms
  // (k = 8), and the other 8 rows come from the unrolled iterations.
  const int32_t base = blockIdx.x * (kPackThreads * kPackUnroll);
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  int32_t cs[kPackUnroll];
#pragma unroll
  for (int u = 0; u < kPackUnroll; ++u) {
    int32_t c_local;
    if (R == 8) {
      c_local = threadIdx.x + u * kPackThreads;
    } else if (KA == 16) {  // c = (kr * 16 + i) * 2 + h
      const int h = l & 1, i = ((l >> 1) & 7) | ((u & 1) << 3);
      const int kr = ((l >> 4) & 3) | ((u >> 1) << 2) | (w << 3);
      c_local = (kr * 16 + i) * 2 + h;
    } else {  // c = kr * 16 + i
      const int i = (l & 7) | ((u & 1) << 3);
      const int kr = ((l >> 3) & 7) | ((u >> 1) << 3) | (w << 4);
      c_local = kr * 16 + i;
    }
    cs[u] = base + c_local;
  }
  u32x4 v[kPackUnroll];
#pragma unroll
  for (int u = 0; u < kPackUnroll; ++u) {
    const int32_t c = cs[u];
    if (c < chunks_per_rb) {
      // chunk c: K atom, row in atom, half (k = 16) or K atom, row (k = 8)
      const int32_t i = KA == 16 ? (c >> 1) & (R - 1) : c & (R - 1);
      const int32_t k8 = KA == 16 ? 2 * (c >> (kLog2R + 1)) + (c & 1) : c >> kLog2R;
      v[u] = load16_nt(reinterpret_cast<const uint32_t*>(srow + i * ld + 8 * k8));
    }
  }
#pragma unroll
  for (int u = 0; u < kPackUnroll; ++u) {
    const int32_t c = cs[u];
    if (c < chunks_per_rb)
      __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4*>(drb + int64_t(c) * 4));
  }
}

// ---- operands up to 128 MiB: staged through LDS ----
constexpr int kStagedThreads = 512;
constexpr int kStagedUnroll = 4;
constexpr int kSpan = kStagedThreads * kStagedUnroll;  // output chunks (16 B) per workgroup
constexpr int kLog2Span = 11;
static_assert(kSpan == 1 << kLog2Span, "span is a power of two");

template <int R, int KA>
__global__ __launch_bounds__(kStagedThreads) void pack_staged_kernel(
    uint32_t* __restrict__ dst, const uint16_t* __restrict__ src, int64_t rb0,
    int32_t chunks_per_rb, int64_t ld) {
  // One workgroup: row block rb and the kSpan output chunks (32 KB) of one K
  // span of 8 * kSpan / R values. Its source is R row pieces of 32 KB / R
  // each, so consecutive lanes read consecutive 16 bytes of one row; every
  // chunk goes to its output position in LDS, and the span is written out
  // contiguously.
  constexpr int kLog2R = R == 16 ? 4 : 3;
  constexpr int kRowChunks = kSpan / R;               // source chunks per row of the span
  constexpr int kLog2RowChunks = kLog2Span - kLog2R;
  constexpr int kShift = KA == 16 ? kLog2R + 1 : kLog2R;  // log2(chunks per K atom)
  constexpr int kMask = kShift >= 4 ? 15 : (1 << kShift) - 1;
  __shared__ __attribute__((aligned(16))) u32x4 lds[kSpan];
  // LDS slot of output chunk o: its low bits XORed with the K atom above them,
  // so that the strided writes below spread over the banks (a bijection: only
  // bits below kShift change, as a function of the bits from kShift up).
  auto slot = [](int o) { return o ^ ((o >> kShift) & kMask); };

  const int64_t rb = rb0 + blockIdx.y;
  const int32_t span0 = blockIdx.x * kSpan;           // first output chunk of the span
  const int32_t n_out = chunks_per_rb - span0 < kSpan ? chunks_per_rb - span0 : kSpan;
  const int64_t k0 = int64_t(blockIdx.x) * (8 * kRowChunks);  // first K value of the span
  const int64_t K = int64_t(chunks_per_rb) * 8 / R;
  const uint16_t* srow = src + rb * R * ld + k0;
#pragma unroll
  for (int u = 0; u < kStagedUnroll; ++u) {
    const int q = u * kStagedThreads + threadIdx.x;   // source chunk: row i, piece kc
    const int i = q >> kLog2RowChunks, kc = q & (kRowChunks - 1);
    if (k0 + 8 * kc < K) {
      const u32x4 v = load16_nt(reinterpret_cast<const uint32_t*>(srow + i * ld + 8 * kc));
      // output chunk: K atom, row in atom, half (k = 16) or K atom, row (k = 8)
      const int o = KA == 16 ? (((kc >> 1) << kLog2R) + i) * 2 + (kc & 1) : (kc << kLog2R) + i;
      lds[slot(o)] = v;
    }
  }
  __syncthreads();
  uint32_t* dspan = dst + (rb * int64_t(chunks_per_rb) + span0) * 4;
#pragma unroll
  for (int u = 0; u < kStagedUnroll; ++u) {
    const int o = u * kStagedThreads + threadIdx.x;
    if (o < n_out) *reinterpret_cast<u32x4*>(dspan + int64_t(o) * 4) = lds[slot(o)];
  }
}

// ---- K-major sources ----
// The source holds the transpose: element (row, k) at src[b, k, row], rows
// contiguous. One workgroup turns a tile of kKmTileRows rows x 64 K values
// around through LDS: lanes read 16-byte pieces of source rows (consecutive
// lanes along one k, so each k contributes a run of 2 * kKmTileRows bytes), a
// barrier, then each lane gathers the 8 consecutive K values of one row from
// the tile and stores them as one 16-byte packed chunk, the chunks of the tile
// in destination order (runs of one row block's 64 K values). The chunk is
// half a row of a 16-deep atom, or a whole row of an 8-deep one (KA = 8).
// Outputs up to 128 MiB are stored through the caches, as by the staged row-
// major packer (8192^2 bf16: each K-major pack 17% faster, and the multiply
// after it 3%); larger ones with non-temporal stores. Measured at 8192^2 in
// one process: plain source loads 2-5% faster than non-temporal ones; tiles
// of 128 or 256 rows 4% and 70% slower than 64; taking the K tiles first, or
// groups of 8 row tiles with the K tiles first, 5-14% and 0-10% slower.
constexpr int kKmTileK = 64;
constexpr int kKmTileRows = 64;
constexpr int kKmThreads = 256;

template <int R, int KA, bool kCachedStore>
__global__ __launch_bounds__(kKmThreads) void pack_kmajor_kernel(uint32_t* __restrict__ dst,
                                                                 const uint16_t* __restrict__ src,
                                                                 int64_t rows, int64_t K,
                                                                 int64_t ld) {
  constexpr int kPitch = kKmTileRows + 8;                         // u16 per LDS row (16-byte aligned)
  constexpr int kRowChunks = kKmTileRows / 8;                     // 16-byte pieces per k
  constexpr int kPerLane = kKmTileK * kRowChunks / kKmThreads;    // chunks per lane, each phase
  __shared__ __attribute__((aligned(16))) uint16_t tile[kKmTileK][kPitch];
  const int tid = threadIdx.x;
  const int64_t row0 = int64_t(blockIdx.x) * kKmTileRows, k0 = int64_t(blockIdx.y) * kKmTileK;
  const int64_t b = blockIdx.z;
  const uint16_t* sb = src + b * K * ld;
  u32x4 v[kPerLane];
#pragma unroll
  for (int u = 0; u < kPerLane; ++u) {
    const int c = tid + kKmThreads * u;
    const int kk = c / kRowChunks, rc = (c % kRowChunks) * 8;
    v[u] = u32x4{0u, 0u, 0u, 0u};
    if (k0 + kk < K && row0 + rc < rows)
      v[u] = load16(reinterpret_cast<const uint32_t*>(sb + (k0 + kk) * ld + row0 + rc));
  }
#pragma unroll
  for (int u = 0; u < kPerLane; ++u) {
    const int c = tid + kKmThreads * u;
    *reinterpret_cast<u32x4*>(&tile[c / kRowChunks][(c % kRowChunks) * 8]) = v[u];
  }
  __syncthreads();
  constexpr int kLog2R = R == 16 ? 4 : 3;
  const int64_t rows_rep = rows / R, K_rep = K / KA;
#pragma unroll
  for (int u = 0; u < kPerLane; ++u) {
    const int c = tid + kKmThreads * u;
    // chunk c of the tile: row block c / (8R), then K atom, row in atom, and
    // (KA = 16) half of the atom row
    const int rb = c >> (kLog2R + 3), rem = c & (8 * R - 1);
    const int kr = KA == 16 ? rem >> (kLog2R + 1) : rem >> kLog2R;
    const int i = KA == 16 ? (rem >> 1) & (R - 1) : rem & (R - 1);
    const int h = KA == 16 ? rem & 1 : 0;
    const int row_l = rb * R + i, k_l = kr * KA + h * 8;
    if (row0 + row_l >= rows || k0 + k_l >= K) continue;
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = uint32_t(tile[k_l + 2 * e][row_l]) | (uint32_t(tile[k_l + 2 * e + 1][row_l]) << 16);
    const int64_t off = (((b * rows_rep + row0 / R + rb) * K_rep + k0 / KA + kr) * R + i) *
                            (KA / 2) + 4 * h;
    if constexpr (kCachedStore)
      *reinterpret_cast<u32x4*>(dst + off) = w;
    else
      __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(dst + off));
  }
}

}  // namespace

hipError_t launch_pack_kmajor(uint32_t* dst, const uint16_t* src, int64_t batch, int64_t rows,
                              int64_t K, int64_t ld, int R, int atom_k, hipStream_t s) {
  const dim3 grid(unsigned((rows + kKmTileRows - 1) / kKmTileRows),
                  unsigned((K + kKmTileK - 1) / kKmTileK), unsigned(batch));
  const bool cached = batch * rows * K * 2 <= kCachedPackBytes;
  auto kern = cached ? (R == 16 ? (atom_k == 16 ? pack_kmajor_kernel<16, 16, true> : pack_kmajor_kernel<16, 8, true>)
                                : (atom_k == 16 ? pack_kmajor_kernel<8, 16, true> : pack_kmajor_kernel<8, 8, true>))
                     : (R == 16 ? (atom_k == 16 ? pack_kmajor_kernel<16, 16, false> : pack_kmajor_kernel<16, 8, false>)
                                : (atom_k == 16 ? pack_kmajor_kernel<8, 16, false> : pack_kmajor_kernel<8, 8, false>));
  hipLaunchKernelGGL(kern, grid, dim3(kKmThreads), 0, s, dst, src, rows, K, ld);
  return hipGetLastError();
}

hipError_t launch_pack(uint32_t* dst, const uint16_t* src, int64_t batch, int64_t rows,
                       int64_t K, int64_t ld, int R, int atom_k, hipStream_t s) {
  const int64_t n_rb = batch * (rows / R);
  const int32_t chunks = int32_t(R * (K / 8));  // 16-byte chunks per row block
  const bool staged = batch * rows * K * 2 <= kCachedPackBytes;
  const int per_block = staged ? kSpan : kPackThreads * kPackUnroll;
  const unsigned gx = unsigned((chunks + per_block - 1) / per_block);
  auto kern = staged ? (R == 16 ? (atom_k == 16 ? pack_staged_kernel<16, 16> : pack_staged_kernel<16, 8>)
                                : (atom_k == 16 ? pack_staged_kernel<8, 16> : pack_staged_kernel<8, 8>))
                     : (R == 16 ? (atom_k == 16 ? pack_kernel<16, 16> : pack_kernel<16, 8>)
                                : (atom_k == 16 ? pack_kernel<8, 16> : pack_kernel<8, 8>));
  const unsigned threads = staged ? kStagedThreads : kPackThreads;
  for (int64_t rb0 = 0; rb0 < n_rb; rb0 += 65535) {
    const unsigned gy = unsigned(n_rb - rb0 < 65535 ? n_rb - rb0 : 65535);
    hipLaunchKernelGGL(kern, dim3(gx, gy), dim3(threads), 0, s, dst, src, rb0, chunks, ld);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bmm
