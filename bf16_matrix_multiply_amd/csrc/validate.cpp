#include "validate.h"

#include <cstdio>
#include <string>

namespace bmm {
namespace {

// Extents are capped so that every byte count below fits in int64 without
// overflow checks at each product.
constexpr int64_t kMaxExtent = int64_t(1) << 40;
constexpr int64_t kMaxBytes = int64_t(1) << 50;

Status fail(int code, const char* fmt, long long a = 0, long long b = 0) {
  Status s;
  s.code = code;
  char buf[256];
  std::snprintf(buf, sizeof buf, fmt, a, b);
  s.msg = buf;
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, int64_t an, const void* b, int64_t bn) {
  if (an <= 0 || bn <= 0) return false;
  uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + uintptr_t(bn) && b0 < a0 + uintptr_t(an);
}

// product of non-negative extents, or -1 when it exceeds kMaxBytes
int64_t mul_capped(std::initializer_list<int64_t> xs) {
  __int128 p = 1;
  for (int64_t x : xs) {
    p *= x;
    if (p > kMaxBytes) return -1;
  }
  return int64_t(p);
}

}  // namespace

Status check_pack(const uint32_t* dst, const uint16_t* src, int64_t batch, int64_t rows,
                  int64_t K, int64_t ld_src, int32_t atom_rows, int32_t atom_k) {
  if (atom_rows != 16 && atom_rows != 8)
    return fail(BMM_EINVAL, "pack_operand: atom_rows must be 16 (A) or 8 (B), got %lld",
                atom_rows);
  if (batch < 0 || rows < 0 || K < 0)
    return fail(BMM_EINVAL, "pack_operand: negative extent");
  if (batch > kMaxExtent || rows > kMaxExtent || K > (int64_t(1) << 26))
    return fail(BMM_EINVAL, "pack_operand: extent too large");
  if (rows % atom_rows)
    return fail(BMM_EINVAL, "pack_operand: rows (%lld) is not a multiple of atom_rows (%lld)",
                rows, atom_rows);
  if (K % atom_k)
    return fail(BMM_EINVAL, "pack_operand: K (%lld) is not a multiple of %lld", K, atom_k);
  if (ld_src < K) return fail(BMM_EINVAL, "pack_operand: ld_src (%lld) < K (%lld)", ld_src, K);
  if (ld_src > (int64_t(1) << 32)) return fail(BMM_EINVAL, "pack_operand: ld_src too large");
  if (batch == 0 || rows == 0 || K == 0) return Status{};
  if (!dst || !src) return fail(BMM_EINVAL, "pack_operand: null pointer");
  if (ld_src % 8)
    return fail(BMM_EALIGN, "pack_operand: ld_src (%lld) must be a multiple of 8 elements",
                ld_src);
  if (!aligned16(dst) || !aligned16(src))
    return fail(BMM_EALIGN, "pack_operand: dst and src must be 16-byte aligned");
  int64_t dst_bytes = mul_capped({batch, rows, K, 2});
  int64_t src_bytes = mul_capped({batch * rows - 1, ld_src, 2});
  if (dst_bytes < 0 || src_bytes < 0) return fail(BMM_EINVAL, "pack_operand: too large");
  src_bytes += K * 2;
  if (overlaps(dst, dst_bytes, src, src_bytes))
    return fail(BMM_EOVERLAP, "pack_operand: dst overlaps src");
  return Status{};
}

Status check_pack_kmajor(const uint32_t* dst, const uint16_t* src, int64_t batch, int64_t rows,
                         int64_t K, int64_t ld_src, int32_t atom_rows, int32_t atom_k) {
  if (atom_rows != 16 && atom_rows != 8)
    return fail(BMM_EINVAL, "pack_operand_kmajor: atom_rows must be 16 (A) or 8 (B), got %lld",
                atom_rows);
  if (batch < 0 || rows < 0 || K < 0)
    return fail(BMM_EINVAL, "pack_operand_kmajor: negative extent");
  // one workgroup per 64 x 64 tile: K / 64 and batch index grid dimensions
  if (batch > 65535 || rows >= (int64_t(1) << 36) || K >= (int64_t(1) << 22))
    return fail(BMM_EINVAL,
                "pack_operand_kmajor: extent too large (batch <= 65535, rows < 2^36, K < 2^22)");
  if (rows % atom_rows)
    return fail(BMM_EINVAL,
                "pack_operand_kmajor: rows (%lld) is not a multiple of atom_rows (%lld)", rows,
                atom_rows);
  if (K % atom_k)
    return fail(BMM_EINVAL, "pack_operand_kmajor: K (%lld) is not a multiple of %lld", K, atom_k);
  if (ld_src < rows)
    return fail(BMM_EINVAL, "pack_operand_kmajor: ld_src (%lld) < rows (%lld)", ld_src, rows);
  if (ld_src > (int64_t(1) << 32)) return fail(BMM_EINVAL, "pack_operand_kmajor: ld_src too large");
  if (batch == 0 || rows == 0 || K == 0) return Status{};
  if (!dst || !src) return fail(BMM_EINVAL, "pack_operand_kmajor: null pointer");
  if (ld_src % 8)
    return fail(BMM_EALIGN, "pack_operand_kmajor: ld_src (%lld) must be a multiple of 8 elements",
                ld_src);
  if (!aligned16(dst) || !aligned16(src))
    return fail(BMM_EALIGN, "pack_operand_kmajor: dst and src must be 16-byte aligned");
  int64_t dst_bytes = mul_capped({batch, rows, K, 2});
  int64_t src_bytes = mul_capped({batch * K - 1, ld_src, 2});
  if (dst_bytes < 0 || src_bytes < 0) return fail(BMM_EINVAL, "pack_operand_kmajor: too large");
  src_bytes += rows * 2;
  if (overlaps(dst, dst_bytes, src, src_bytes))
    return fail(BMM_EOVERLAP, "pack_operand_kmajor: dst overlaps src");
  return Status{};
}

// Descriptor fields shared by the load, the store and the add reduction.
// On success *span is the byte extent of the global view (from its base) and
// *image the bytes of one repeat's image.
Status check_box_desc(const bmm_box_desc* d, const char* what, int64_t* span_out,
                      int64_t* image_out) {
  auto failw = [what](int code, const char* fmt, long long a = 0, long long b = 0) {
    Status s = fail(code, fmt, a, b);
    s.msg = std::string(what) + ": " + s.msg;
    return s;
  };
  if (!d) return failw(BMM_EINVAL, "null descriptor");
  if (d->rank < 1 || d->rank > 5) return failw(BMM_EINVAL, "rank %lld not in 1..5", d->rank);
  const int eb = d->elem_bytes;
  if (eb != 1 && eb != 2 && eb != 4 && eb != 8)
    return failw(BMM_EINVAL, "elem_bytes %lld not 1, 2, 4 or 8", eb);
  if (d->swizzle < 0 || d->swizzle > 3)
    return failw(BMM_EINVAL, "swizzle %lld not in 0..3", d->swizzle);
  if (d->oob_fill != 0)
    return failw(BMM_EINVAL, "oob_fill %lld unsupported (only 0 = zero fill)", d->oob_fill);
  if (d->n_repeat < 1) return failw(BMM_EINVAL, "n_repeat %lld < 1", d->n_repeat);
  int64_t box_elems = 1, span = 0;
  for (int i = 0; i < d->rank; ++i) {
    if (d->box[i] < 1 || d->box[i] > 256)
      return failw(BMM_EINVAL, "box[%lld] = %lld not in 1..256", i, d->box[i]);
    if (d->dims[i] < 1 || d->dims[i] > kMaxExtent)
      return failw(BMM_EINVAL, "dims[%lld] = %lld out of range", i, d->dims[i]);
    const int64_t c = d->coords[i], st = d->coord_step[i];
    if (c < -kMaxExtent || c > kMaxExtent || st < -kMaxExtent || st > kMaxExtent)
      return failw(BMM_EINVAL, "coords/coord_step[%lld] out of range", i);
    box_elems *= d->box[i];
    if (i == d->rank - 1) {
      if (d->strides[i] != eb)
        return failw(BMM_EINVAL, "innermost stride %lld must equal elem_bytes %lld",
                     d->strides[i], eb);
    } else {
      if (d->strides[i] <= 0 || d->strides[i] > kMaxBytes)
        return failw(BMM_EINVAL, "stride[%lld] = %lld must be positive", i, d->strides[i]);
      if (d->strides[i] % 16)
        return failw(BMM_EALIGN, "outer stride[%lld] = %lld not a multiple of 16", i,
                     d->strides[i]);
    }
    int64_t s = mul_capped({d->dims[i] - 1, d->strides[i]});
    if (s < 0 || span + s > kMaxBytes) return failw(BMM_EINVAL, "tensor too large");
    span += s;
  }
  span += eb;
  const int64_t image = box_elems * eb;
  if (image > kBoxImageLimit)
    return failw(BMM_ERANGE, "one repeat's image is %lld bytes, limit %lld", image,
                 kBoxImageLimit);
  *span_out = span;
  *image_out = image;
  return Status{};
}

Status check_box(const void* dst, const void* src, const bmm_box_desc* d) {
  int64_t span = 0, image = 0;
  Status st = check_box_desc(d, "box_copy", &span, &image);
  if (!st.ok()) return st;
  if (!dst || !src) return fail(BMM_EINVAL, "box_copy: null pointer");
  if (!aligned16(dst) || !aligned16(src))
    return fail(BMM_EALIGN, "box_copy: dst_image and src must be 16-byte aligned");
  const int64_t total = mul_capped({image, d->n_repeat});
  if (total < 0) return fail(BMM_EINVAL, "box_copy: image too large");
  if (overlaps(dst, total, src, span)) return fail(BMM_EOVERLAP, "box_copy: dst overlaps src");
  return Status{};
}

Status check_box_store(const void* dst, const void* img, const bmm_box_desc* d,
                       int32_t elem_type, const char* what) {
  int64_t span = 0, image = 0;
  Status st = check_box_desc(d, what, &span, &image);
  if (!st.ok()) return st;
  auto failw = [what](int code, const char* fmt, long long a = 0, long long b = 0) {
    Status s = fail(code, fmt, a, b);
    s.msg = std::string(what) + ": " + s.msg;
    return s;
  };
  if (elem_type != 0) {
    static const int kTypeBytes[6] = {0, 4, 2, 2, 4, 8};
    if (elem_type < BMM_ELEM_F32 || elem_type > BMM_ELEM_I64)
      return failw(BMM_EINVAL, "elem_type %lld is not a bmm_elem_type", elem_type);
    if (kTypeBytes[elem_type] != d->elem_bytes)
      return failw(BMM_EINVAL, "elem_type %lld does not match elem_bytes %lld", elem_type,
                   d->elem_bytes);
  }
  // Every global element of the view must have its own address: each outer
  // stride covers the whole extent of the dimensions inside it.
  int64_t inner = d->elem_bytes;
  for (int i = d->rank - 1; i >= 0; --i) {
    if (i < d->rank - 1 && d->dims[i] > 1 && d->strides[i] < inner)
      return failw(BMM_EINVAL, "stride[%lld] = %lld makes the destination view overlap itself",
                   i, d->strides[i]);
    inner = (d->dims[i] - 1) * d->strides[i] + inner;
  }
  if (!dst || !img) return failw(BMM_EINVAL, "null pointer");
  if (!aligned16(dst) || !aligned16(img))
    return failw(BMM_EALIGN, "dst and src_image must be 16-byte aligned");
  const int64_t total = mul_capped({image, d->n_repeat});
  if (total < 0) return failw(BMM_EINVAL, "image too large");
  if (overlaps(dst, span, img, total)) return failw(BMM_EOVERLAP, "dst overlaps src_image");
  return Status{};
}

Status check_mma(const float* D, const uint32_t* A, const uint32_t* B, const float* C,
                 int64_t batch, int64_t M_rep, int64_t N_rep, int64_t K_rep, int32_t dtype,
                 int32_t kernel, int32_t atom_k) {
  if (atom_k != 16 && atom_k != 8)
    return fail(BMM_EINVAL, "mma_tile: atom_k must be 16 or 8, got %lld", atom_k);
  if (dtype != BMM_F16 && dtype != BMM_BF16)
    return fail(BMM_EINVAL, "mma_tile: dtype %lld is neither BMM_F16 nor BMM_BF16", dtype);
  if (kernel < BMM_KERNEL_AUTO || kernel > BMM_KERNEL_TILED_256x128)
    return fail(BMM_EINVAL, "mma_tile: unknown kernel %lld", kernel);
  if (batch < 0 || M_rep < 0 || N_rep < 0 || K_rep < 0)
    return fail(BMM_EINVAL, "mma_tile: negative extent");
  if (batch > kMaxExtent || M_rep > kMaxExtent || N_rep > kMaxExtent || K_rep > (1 << 26))
    return fail(BMM_EINVAL, "mma_tile: extent too large");
  const int64_t d_bytes = mul_capped({batch, M_rep, N_rep, 512});
  // one atom: 16 (A) or 8 (B) rows of atom_k / 2 words
  const int64_t a_bytes = mul_capped({batch, M_rep, K_rep, 32 * atom_k});
  const int64_t b_bytes = mul_capped({batch, N_rep, K_rep, 16 * atom_k});
  if (d_bytes < 0 || a_bytes < 0 || b_bytes < 0) return fail(BMM_EINVAL, "mma_tile: too large");
  if (d_bytes == 0) return Status{};
  if (!D) return fail(BMM_EINVAL, "mma_tile: D is null");
  if (K_rep > 0 && (!A || !B)) return fail(BMM_EINVAL, "mma_tile: A or B is null");
  if (!aligned16(D) || !aligned16(A) || !aligned16(B) || !aligned16(C))
    return fail(BMM_EALIGN, "mma_tile: D, A, B and C must be 16-byte aligned");
  if (overlaps(D, d_bytes, A, a_bytes)) return fail(BMM_EOVERLAP, "mma_tile: D overlaps A");
  if (overlaps(D, d_bytes, B, b_bytes)) return fail(BMM_EOVERLAP, "mma_tile: D overlaps B");
  if (C && C != D && overlaps(D, d_bytes, C, d_bytes))
    return fail(BMM_EOVERLAP, "mma_tile: D partially overlaps C (only D == C is allowed)");
  return Status{};
}

int64_t splitk_effective(int64_t K_rep, int32_t atom_k, int32_t splits) {
  const int64_t steps = (K_rep * atom_k + 31) / 32;
  return splits < steps ? splits : steps;
}

Status check_splitk(const float* D, const uint32_t* A, const uint32_t* B, const float* C,
                    int64_t batch, int64_t M_rep, int64_t N_rep, int64_t K_rep, int32_t dtype,
                    int32_t atom_k, int32_t splits, const void* workspace,
                    int64_t workspace_bytes) {
  Status st = check_mma(D, A, B, C, batch, M_rep, N_rep, K_rep, dtype, BMM_KERNEL_TILED, atom_k);
  if (!st.ok()) {
    st.msg = "mma_tile_splitk: " + st.msg;
    return st;
  }
  if (splits < 1 || splits > 65535)
    return fail(BMM_EINVAL, "mma_tile_splitk: splits %lld not in 1..65535", splits);
  if (K_rep * atom_k >= (int64_t(1) << 22))
    return fail(BMM_EINVAL, "mma_tile_splitk: K = %lld values, the tiled kernel takes K < 2^22",
                K_rep * atom_k);
  const int64_t d_bytes = mul_capped({batch, M_rep, N_rep, 512});
  if (d_bytes == 0) return Status{};
  const int64_t need = mul_capped({splitk_effective(K_rep, atom_k, splits), d_bytes});
  if (need < 0) return fail(BMM_EINVAL, "mma_tile_splitk: workspace too large");
  if (workspace_bytes < need)
    return fail(BMM_EINVAL, "mma_tile_splitk: workspace_bytes %lld < %lld needed",
                workspace_bytes, need);
  if (need > 0) {
    if (!workspace) return fail(BMM_EINVAL, "mma_tile_splitk: workspace is null");
    if (!aligned16(workspace))
      return fail(BMM_EALIGN, "mma_tile_splitk: workspace must be 16-byte aligned");
    const int64_t a_bytes = mul_capped({batch, M_rep, K_rep, 32 * atom_k});
    const int64_t b_bytes = mul_capped({batch, N_rep, K_rep, 16 * atom_k});
    if (overlaps(workspace, need, D, d_bytes) || overlaps(workspace, need, A, a_bytes) ||
        overlaps(workspace, need, B, b_bytes) || (C && overlaps(workspace, need, C, d_bytes)))
      return fail(BMM_EOVERLAP, "mma_tile_splitk: workspace overlaps D, A, B or C");
  }
  return Status{};
}

}  // namespace bmm
