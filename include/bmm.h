/*
 * bmm.h — C ABI of the MI355X (gfx950) tiled f16/bf16 multiply-accumulate
 * D = A * B^T + C with float32 accumulation, over the packed operand layouts
 * of the Apache TVM "tirx" mma.sync tile-op page.
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; the
 *     library keeps no reference to it after the call returns.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and return once the kernels are enqueued.
 *   - Arguments are validated on the host, once per call, before any HIP
 *     call (the cp.async.bulk.tensor page, "Example: two explicit 8x16
 *     boxes": descriptor set-up is host work, not repeated per box). On a
 *     failed check nothing is launched and nothing is written.
 *   - Invalid fields are rejected, never promoted, folded, transposed or
 *     reinterpreted (cp.async.bulk.tensor page, "Operands and descriptor
 *     fields"; mma.sync page introduction: no implicit type change, K-atom
 *     choice or transpose).
 *   - Return value: BMM_OK (0) or a negative status; bmm_last_error()
 *     returns a message for the last failure on the calling thread.
 *   - The library allocates no device memory. Scratch space (the split-K
 *     partial sums) is a caller-owned workspace, except in
 *     bmm_mma_tile_splitk_noalloc, which uses a fixed static array per device.
 *   - Destination first (mma.sync page, "Operand coordinates and
 *     ownership": the call takes D, A, B, C).
 */
#ifndef BMM_H
#define BMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { BMM_F16 = 0, BMM_BF16 = 1 } bmm_dtype;

enum {
  BMM_OK = 0,
  BMM_EINVAL = -1,   /* bad extent, dtype, field value or null pointer */
  BMM_EALIGN = -2,   /* pointer or stride not aligned as required */
  BMM_EOVERLAP = -3, /* destination overlaps a source (other than D == C) */
  BMM_ERANGE = -4,   /* a box image larger than the staging limit */
  BMM_EHIP = -5      /* the HIP runtime reported an error at launch */
};

/* Kernel selection for bmm_mma_tile_with. AUTO picks by shape (TILED with
 * more than 128 256 x 256 tiles, ragged ones counted, else TILED_256x128 with
 * more than 128 256 x 128 tiles, else TILED_128 with at least 128 128 x 128
 * tiles, else SKINNY, else DIRECT if a grid limit rules the others out); the
 * others force one kernel (every kernel accepts every valid shape within its
 * launch-grid limits). All three tiled kernels give identical results. */
typedef enum {
  BMM_KERNEL_AUTO = 0,
  BMM_KERNEL_DIRECT = 1, /* one wave per 16x16 output block, operands straight from HBM */
  BMM_KERNEL_TILED = 2,  /* LDS-staged 256x256 macro tiles for large M and N */
  BMM_KERNEL_SKINNY = 3, /* few output tiles: K split across the waves of a workgroup, B streamed */
  BMM_KERNEL_TILED_128 = 4, /* LDS-staged 128x128 macro tiles, two workgroups per CU */
  BMM_KERNEL_TILED_256x128 = 5 /* LDS-staged 256 (M) x 128 (N) macro tiles, one per CU */
} bmm_kernel;

/*
 * bmm_pack_operand — row-major halves to packed b32 atoms.
 *
 * Defined by the mma.sync page, "Operand coordinates and ownership" (A is
 * (M_repeat, K_repeat, 16, k/2) and B is (N_repeat, K_repeat, 8, k/2) b32
 * words, each word two adjacent K values) and the worked example's host
 * code (row-major halves reshaped, transposed and viewed as uint32, so the
 * even K value is the low 16 bits). Atom K is k = 16.
 *
 *   dst[b, r, kr, i, w] = src[b, R*r+i, 16*kr+2*w] | src[b, R*r+i, 16*kr+2*w+1] << 16
 *
 * dst       (batch, rows/R, K/16, R, 8) uint32, contiguous, 16-byte aligned.
 * src       (batch, rows, ld_src) 16-bit values (f16 or bf16 bits; the bits are
 *           moved, never converted), batch stride rows*ld_src elements,
 *           16-byte aligned.
 * rows      multiple of atom_rows; K multiple of 16; ld_src >= K and a
 *           multiple of 8 (16-byte row starts). Zero batch, rows or K is a
 *           no-op.
 * atom_rows R: 16 for an A operand, 8 for a B operand.
 * Errors: BMM_EINVAL (extents, atom_rows), BMM_EALIGN, BMM_EOVERLAP (dst and
 * src overlap), BMM_EHIP.
 */
int bmm_pack_operand(uint32_t* dst, const uint16_t* src, int64_t batch, int64_t rows,
                     int64_t K, int64_t ld_src, int32_t atom_rows, void* stream);

/*
 * bmm_pack_operand_k8 — row-major halves to packed atoms with an atom K of 8.
 *
 * The mma.sync page's introduction names the m16n8k8 form beside m16n8k16,
 * and its table of shapes gives k = 8 for f16/bf16 inputs. With k = 8 the
 * layouts of "Operand coordinates and ownership" hold k/2 = 4 words per atom
 * row: A is (M_repeat, K_repeat, 16, 4) and B is (N_repeat, K_repeat, 8, 4)
 * words, K_repeat = K/8:
 *
 *   dst[b, r, kr, i, w] = src[b, R*r+i, 8*kr+2*w] | src[b, R*r+i, 8*kr+2*w+1] << 16
 *
 * dst  (batch, rows/R, K/8, R, 4) uint32, contiguous, 16-byte aligned.
 * K    a multiple of 8. Every other argument, and the errors, as
 *      bmm_pack_operand.
 * The result feeds bmm_mma_tile_opts with atom_k = 8.
 */
int bmm_pack_operand_k8(uint32_t* dst, const uint16_t* src, int64_t batch, int64_t rows,
                        int64_t K, int64_t ld_src, int32_t atom_rows, void* stream);

/*
 * bmm_pack_operand_kmajor — packing from a K-major (transposed) source.
 *
 * The mma.sync page ("Accumulation, transpose and alpha/beta") leaves a
 * logical transpose to explicit preparation: a view cannot move values
 * between lanes, so an operand whose K values are not contiguous must be
 * rewritten. This is that preparation for the packed layouts: the source
 * holds element (row, k) of the logical operand at src[b, k, row] (rows
 * contiguous), and the result is exactly what bmm_pack_operand gives for the
 * row-major matrix:
 *
 *   dst[b, r, kr, i, w] = src[b, 16*kr+2*w, R*r+i] | src[b, 16*kr+2*w+1, R*r+i] << 16
 *
 * dst       (batch, rows/R, K/16, R, 8) uint32, contiguous, 16-byte aligned.
 * src       (batch, K, ld_src) 16-bit values, batch stride K*ld_src, 16-byte aligned.
 * rows      multiple of atom_rows; K multiple of 16 and below 2^22; ld_src >= rows and
 *           a multiple of 8; batch at most 65535; rows below 2^36. Zero batch, rows or K is a
 *           no-op.
 * Errors: as bmm_pack_operand.
 */
int bmm_pack_operand_kmajor(uint32_t* dst, const uint16_t* src, int64_t batch, int64_t rows,
                            int64_t K, int64_t ld_src, int32_t atom_rows, void* stream);

/*
 * bmm_pack_operand_kmajor_k8 — K-major source to the m16n8k8 layout.
 *
 * The two preparations above together: a K-major (transposed) source, as for
 * bmm_pack_operand_kmajor, packed into atoms with an atom K of 8, as for
 * bmm_pack_operand_k8 (mma.sync page: "Accumulation, transpose and
 * alpha/beta"; the m16n8k8 form of the introduction and the table of shapes).
 * The result is exactly what bmm_pack_operand_k8 gives for the row-major
 * matrix:
 *
 *   dst[b, r, kr, i, w] = src[b, 8*kr+2*w, R*r+i] | src[b, 8*kr+2*w+1, R*r+i] << 16
 *
 * dst  (batch, rows/R, K/8, R, 4) uint32, contiguous, 16-byte aligned.
 * K    a multiple of 8 and below 2^22. Every other argument, and the errors, as
 *      bmm_pack_operand_kmajor.
 */
int bmm_pack_operand_kmajor_k8(uint32_t* dst, const uint16_t* src, int64_t batch, int64_t rows,
                               int64_t K, int64_t ld_src, int32_t atom_rows, void* stream);

/*
 * bmm_box_copy — a rectangular global box through an LDS image.
 *
 * The role of the TMA tile-mode box load on the cp.async.bulk.tensor page
 * ("Operands and descriptor fields", "Example: two explicit 8x16 boxes"):
 * for each repeat t the box at coords + t*coord_step is staged into a
 * shared-memory (LDS) image, laid out with the requested swizzle, and the
 * image is written out compact and unswizzled:
 *
 *   dst_image[t, j_0..j_{rank-1}] = src[coords + t*coord_step + j] if every
 *                                   coordinate is inside dims, else 0.
 *
 * desc fields (outer-to-inner order, as on the page):
 *   rank        1..5
 *   elem_bytes  1, 2, 4 or 8 (the storage type; never reinterpreted)
 *   dims        global extents, each >= 1
 *   strides     byte strides; strides[rank-1] == elem_bytes; outer strides
 *               multiples of 16 ("suitably aligned outer byte strides")
 *   box         1..256 per dimension
 *   coords      start coordinates; may lie partly or wholly outside dims
 *   n_repeat    >= 1 repeats (the leading image axis)
 *   coord_step  per-repeat coordinate increment
 *   swizzle     0..3: none / 32-byte / 64-byte / 128-byte XOR swizzle of
 *               the LDS image (internal; the exported image is unswizzled)
 *   oob_fill    0 (zero fill, the page's default) is the only value accepted
 * dst_image    (n_repeat, box...) compact, 16-byte aligned; must not overlap src.
 * src          16-byte aligned base of the global tensor.
 * bytes_moved  nullable host pointer; receives n_repeat * prod(box) * elem_bytes.
 * One repeat's image may hold at most 65536 bytes (else BMM_ERANGE).
 * Errors: BMM_EINVAL, BMM_EALIGN, BMM_EOVERLAP, BMM_ERANGE, BMM_EHIP.
 */
typedef struct {
  int32_t rank;
  int32_t elem_bytes;
  int64_t dims[5];
  int64_t strides[5];
  int32_t box[5];
  int64_t coords[5];
  int32_t n_repeat;
  int64_t coord_step[5];
  int32_t swizzle;
  int32_t oob_fill;
} bmm_box_desc;

int bmm_box_copy(void* dst_image, const void* src, const bmm_box_desc* desc,
                 int64_t* bytes_moved, void* stream);

/*
 * bmm_box_store — a compact image written into a rectangular global box.
 *
 * The store direction of the cp.async.bulk.tensor page ("Stores, reductions,
 * and completion": the load's coordinate/box contract, global destination
 * first). Each repeat's image is staged through an LDS image (with the
 * requested swizzle) and written out:
 *
 *   dst[coords + t*coord_step + j] = src_image[t, j_0..j_{rank-1}]
 *                                    for every coordinate inside dims;
 *   elements outside dims are not written.
 *
 * Repeats are applied in ascending t: where the boxes of two repeats
 * overlap, the later repeat's values stand.
 * desc         as bmm_box_copy; additionally the destination view must not
 *              overlap itself (each outer stride at least the byte extent of
 *              the dimensions inside it), else BMM_EINVAL.
 * src_image    (n_repeat, box...) compact, 16-byte aligned, not overlapping dst.
 * bytes_moved  nullable; receives n_repeat * prod(box) * elem_bytes (image bytes read).
 * Errors: BMM_EINVAL, BMM_EALIGN, BMM_EOVERLAP, BMM_ERANGE, BMM_EHIP.
 */
int bmm_box_store(void* dst, const void* src_image, const bmm_box_desc* desc,
                  int64_t* bytes_moved, void* stream);

/* Element types of bmm_box_reduce_add; each must match desc->elem_bytes. */
typedef enum {
  BMM_ELEM_F32 = 1,  /* 4 bytes */
  BMM_ELEM_F16 = 2,  /* 2 bytes, IEEE binary16 */
  BMM_ELEM_BF16 = 3, /* 2 bytes, bfloat16 */
  BMM_ELEM_I32 = 4,  /* 4 bytes, wraps modulo 2^32 (signed or unsigned alike) */
  BMM_ELEM_I64 = 5   /* 8 bytes, wraps modulo 2^64 */
} bmm_elem_type;

/*
 * bmm_box_reduce_add — add a compact image into a rectangular global box.
 *
 * The add reduction of the cp.async.bulk.tensor page ("Stores, reductions,
 * and completion"); the destination holds its starting value beforehand.
 *
 *   dst[coords + t*coord_step + j] = dst[...] + src_image[t, j]
 *
 * for every coordinate inside dims, repeats in ascending t, one rounding per
 * add in the element type (round to nearest even; f16 and bf16 sums are
 * correctly rounded). Arguments, ordering and errors as bmm_box_store, plus
 * BMM_EINVAL for an elem_type that is not a bmm_elem_type or does not match
 * elem_bytes. NaN payloads of float results are unspecified.
 */
int bmm_box_reduce_add(void* dst, const void* src_image, const bmm_box_desc* desc,
                       int32_t elem_type, int64_t* bytes_moved, void* stream);

/*
 * bmm_mma_tile — D = A * B^T + C over packed operands.
 *
 * Defined by the mma.sync page: "Operand coordinates and ownership" (the
 * layouts below; A and B share one input dtype, the accumulator is float32)
 * and "Accumulation, transpose and alpha/beta" (repeat order batch, M, N,
 * then K; C is a matching tensor or a scalar broadcast; only the first K
 * step reads C, later steps read D).
 *
 * D  (batch, M_rep, N_rep, 16, 8) float32, written.
 * A  (batch, M_rep, K_rep, 16, 8) uint32 words (two halves per word, even K low).
 * B  (batch, N_rep, K_rep, 8, 8)  uint32 words; B's logical axes are (N, K).
 * C  (batch, M_rep, N_rep, 16, 8) float32, or NULL to use c_scalar for every
 *    element. C == D (in place) is allowed: each output is read before it is
 *    written by the same thread. Any other overlap of D with A, B or C is
 *    rejected.
 * Every pointer is 16-byte aligned. Extents are >= 0; a zero batch, M_rep or
 * N_rep is a no-op; K_rep = 0 gives D = C (the empty sum).
 * Summation order inside the hardware's 32-deep MFMA step is the hardware's;
 * between steps K is taken in ascending order from C.
 * This entry point takes no workspace and so never splits K: for shapes with
 * few output tiles and a long K, bmm_splitk_suggested says when
 * bmm_mma_tile_splitk is faster, and with how many splits.
 * Errors: BMM_EINVAL, BMM_EALIGN, BMM_EOVERLAP, BMM_EHIP.
 */
int bmm_mma_tile(float* D, const uint32_t* A, const uint32_t* B, const float* C,
                 float c_scalar, int64_t batch, int64_t M_rep, int64_t N_rep, int64_t K_rep,
                 bmm_dtype dtype, void* stream);

/* bmm_mma_tile with an explicit kernel choice (bmm_kernel); same contract. */
int bmm_mma_tile_with(float* D, const uint32_t* A, const uint32_t* B, const float* C,
                      float c_scalar, int64_t batch, int64_t M_rep, int64_t N_rep,
                      int64_t K_rep, bmm_dtype dtype, int32_t kernel, void* stream);

/*
 * bmm_mma_tile_scaled — D = alpha * (A * B^T) + beta * C, scaling at the call site.
 *
 * The mma.sync page ("Accumulation, transpose and alpha/beta") puts alpha/beta
 * scaling before or after the MMA at the call site, with the intended
 * rounding order; this entry point fixes that order: the product is
 * accumulated from zero (K ascending between 32-deep hardware steps), then
 *   D = fma(alpha, acc, fl(beta * C))
 * with one rounding for the final multiply-add (the fma page: a*b+c is one
 * fused operation). C (or c_scalar when C is NULL) is read once, in the
 * epilogue; D == C in place is allowed. Operands, layouts, kernel choice and
 * errors as bmm_mma_tile_with. alpha = beta = 1 differs from bmm_mma_tile
 * only in where C enters the sum (it is added last here, first there).
 */
int bmm_mma_tile_scaled(float* D, const uint32_t* A, const uint32_t* B, const float* C,
                        float c_scalar, float alpha, float beta, int64_t batch, int64_t M_rep,
                        int64_t N_rep, int64_t K_rep, bmm_dtype dtype, int32_t kernel,
                        void* stream);

/*
 * bmm_mma_tile_opts — every form of the multiply-accumulate behind one call.
 *
 * The options select what the other mma entry points fix:
 *   atom_k  16: operands in the k = 16 layout (bmm_pack_operand), K_rep
 *           counts 16-deep atoms; 8: the m16n8k8 layout (bmm_pack_operand_k8,
 *           the mma.sync page's introduction and table of shapes), A is
 *           (batch, M_rep, K_rep, 16, 4) and B (batch, N_rep, K_rep, 8, 4)
 *           words and K_rep counts 8-deep atoms. The sum is the same
 *           function of the logical operands in both layouts; the hardware
 *           step stays 32 K values deep.
 *   kernel  a bmm_kernel value.
 *   scaled  0: the C-then-D recurrence of bmm_mma_tile; 1: the alpha/beta
 *           form of bmm_mma_tile_scaled with these alpha and beta (ignored
 *           when scaled = 0).
 * opts = NULL means {16, BMM_KERNEL_AUTO, 0, 1, 1}, i.e. bmm_mma_tile.
 * D, A, B, C, c_scalar, extents, dtype: as bmm_mma_tile.
 * Errors: as bmm_mma_tile_with; BMM_EINVAL also for atom_k not 16 or 8 and
 * scaled not 0 or 1.
 */
typedef struct {
  int32_t atom_k;
  int32_t kernel;
  int32_t scaled;
  float alpha;
  float beta;
} bmm_mma_opts;

int bmm_mma_tile_opts(float* D, const uint32_t* A, const uint32_t* B, const float* C,
                      float c_scalar, int64_t batch, int64_t M_rep, int64_t N_rep, int64_t K_rep,
                      bmm_dtype dtype, const bmm_mma_opts* opts, void* stream);

/*
 * bmm_mma_tile_splitk — the multiply-accumulate with K split across workgroups.
 *
 * For shapes with few output tiles and a long K. The K axis is cut at
 * multiples of 32 values into S = min(splits, ceil(K / 32)) balanced ranges
 * of whole 32-value steps: split s takes steps [s*n/S, (s+1)*n/S) of the
 * n = ceil(K / 32). Each split's partial sum P_s starts from zero; then the
 * partial sums are add-reduced into a destination that starts at C (the
 * cp.async.bulk.tensor page, "Stores, reductions, and completion": the
 * reduction destination is initialised to the intended starting value):
 *
 *   D = (((C + P_0) + P_1) + ...) + P_{S-1}      (fp32, in this order)
 *
 * so the result is the same on every run and for every schedule. K = 0
 * gives D = C.
 * D, A, B, C, c_scalar, extents, dtype: as bmm_mma_tile (in place D == C
 * allowed); atom_k 16 or 8 as in bmm_mma_tile_opts; K < 2^22 values.
 * splits     1..65535 (bmm_splitk_default suggests one).
 * workspace  device memory of at least bmm_mma_splitk_workspace_bytes(...)
 *            bytes (S * batch * M_rep * N_rep * 512), 16-byte aligned, not
 *            overlapping D, A, B or C; owned by the caller, clobbered.
 * Errors: as bmm_mma_tile_with; BMM_EINVAL also for splits, K and a missing
 * or short workspace, BMM_EOVERLAP for an overlapping workspace.
 */
int bmm_mma_tile_splitk(float* D, const uint32_t* A, const uint32_t* B, const float* C,
                        float c_scalar, int64_t batch, int64_t M_rep, int64_t N_rep,
                        int64_t K_rep, bmm_dtype dtype, int32_t atom_k, int32_t splits,
                        float* workspace, int64_t workspace_bytes, void* stream);

/*
 * bmm_mma_tile_splitk_noalloc — bmm_mma_tile_splitk without a workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. It calls no
 * allocating routine.
 *
 * The partial sums go to a static device array of BMM_NOALLOC_SCRATCH_BYTES
 * (64 MiB) per device, set up on the first call on that device (the device
 * of `stream`; the current device for the null stream) and held until the
 * process ends. Same arguments, arithmetic, bits and errors as bmm_mma_tile_splitk,
 * minus the workspace; a request whose partial sums
 * (bmm_mma_splitk_workspace_bytes) exceed the array returns BMM_ERANGE and
 * launches nothing. Every call on one device shares that device's array, so
 * calls that overlap on one device (other streams, other threads) race and
 * must be serialised by the caller. Nothing in the array needs clearing: each
 * split writes its whole partial sum before the reduce reads it.
 */
#define BMM_NOALLOC_SCRATCH_BYTES (64LL << 20)
int bmm_mma_tile_splitk_noalloc(float* D, const uint32_t* A, const uint32_t* B, const float* C,
                                float c_scalar, int64_t batch, int64_t M_rep, int64_t N_rep,
                                int64_t K_rep, bmm_dtype dtype, int32_t atom_k, int32_t splits,
                                void* stream);

/* Workspace bytes bmm_mma_tile_splitk needs (0 when K = 0), or < 0. */
int64_t bmm_mma_splitk_workspace_bytes(int64_t batch, int64_t M_rep, int64_t N_rep,
                                       int64_t K_rep, int32_t atom_k, int32_t splits);

/* A split count for bmm_mma_tile_splitk: enough tiles x splits for every CU,
 * each split at least 1024 K values deep, at most 32; 1 when splitting does
 * not pay. (The split-K form uses 256 x 256 tiles when there are at least
 * 128 of them, or from K = 16384 values when there are at least 8 of them,
 * and 128 x 128 tiles otherwise.) */
int bmm_splitk_default(int64_t batch, int64_t M_rep, int64_t N_rep, int64_t K_rep,
                       int32_t atom_k);

/* Whether to call bmm_mma_tile_splitk instead of bmm_mma_tile for this
 * shape: the split count to use when the split-K form is expected to be the
 * faster of the two (shapes with few output tiles and a long K, e.g.
 * 1024 x 1024 x 65536: 123 against 335 us on MI355X), 1 when the plain entry
 * point is expected to be at least as fast, or < 0 for invalid extents. The
 * plain entry point never splits K itself, since it takes no workspace. */
int bmm_splitk_suggested(int64_t batch, int64_t M_rep, int64_t N_rep, int64_t K_rep,
                         int32_t atom_k);

/* Which kernel AUTO would run for this shape (K_rep in 16-deep atoms; a
 * bmm_kernel value), or < 0. */
int bmm_select_kernel(int64_t batch, int64_t M_rep, int64_t N_rep, int64_t K_rep);

/* Message for the last failed call on this thread ("" if none). */
const char* bmm_last_error(void);

/* ABI version: 1. */
int bmm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BMM_H */
