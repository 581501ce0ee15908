#include "validate.h"

#include <cstdio>

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
                         int64_t K, int64_t ld_src, int32_t atom_rows) {
  if (atom_rows != 16 && atom_rows != 8)
    return fail(BMM_EINVAL, "pack_operand_kmajor: atom_rows must be 16 (A) or 8 (B), got %lld",
                atom_rows);
  if (batch < 0 || rows < 0 || K < 0)
    return fail(BMM_EINVAL, "pack_operand_kmajor: negative extent");
  if (batch > 65535 || rows > kMaxExtent || K > (int64_t(1) << 22))
    return fail(BMM_EINVAL, "pack_operand_kmajor: extent too large (batch <= 65535, K <= 2^22)");
  if (rows % atom_rows)
    return fail(BMM_EINVAL,
                "pack_operand_kmajor: rows (%lld) is not a multiple of atom_rows (%lld)", rows,
                atom_rows);
  if (K % 16) return fail(BMM_EINVAL, "pack_operand_kmajor: K (%lld) is not a multiple of 16", K);
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

Status check_box(const void* dst, const void* src, const bmm_box_desc* d) {
  if (!d) return fail(BMM_EINVAL, "box_copy: null descriptor");
  if (d->rank < 1 || d->rank > 5) return fail(BMM_EINVAL, "box_copy: rank %lld not in 1..5", d->rank);
  const int eb = d->elem_bytes;
  if (eb != 1 && eb != 2 && eb != 4 && eb != 8)
    return fail(BMM_EINVAL, "box_copy: elem_bytes %lld not 1, 2, 4 or 8", eb);
  if (d->swizzle < 0 || d->swizzle > 3)
    return fail(BMM_EINVAL, "box_copy: swizzle %lld not in 0..3", d->swizzle);
  if (d->oob_fill != 0)
    return fail(BMM_EINVAL, "box_copy: oob_fill %lld unsupported (only 0 = zero fill)",
                d->oob_fill);
  if (d->n_repeat < 1) return fail(BMM_EINVAL, "box_copy: n_repeat %lld < 1", d->n_repeat);
  int64_t box_elems = 1, span = 0;
  for (int i = 0; i < d->rank; ++i) {
    if (d->box[i] < 1 || d->box[i] > 256)
      return fail(BMM_EINVAL, "box_copy: box[%lld] = %lld not in 1..256", i, d->box[i]);
    if (d->dims[i] < 1 || d->dims[i] > kMaxExtent)
      return fail(BMM_EINVAL, "box_copy: dims[%lld] = %lld out of range", i, d->dims[i]);
    const int64_t c = d->coords[i], st = d->coord_step[i];
    if (c < -kMaxExtent || c > kMaxExtent || st < -kMaxExtent || st > kMaxExtent)
      return fail(BMM_EINVAL, "box_copy: coords/coord_step[%lld] out of range", i);
    box_elems *= d->box[i];
    if (i == d->rank - 1) {
      if (d->strides[i] != eb)
        return fail(BMM_EINVAL, "box_copy: innermost stride %lld must equal elem_bytes %lld",
                    d->strides[i], eb);
    } else {
      if (d->strides[i] <= 0 || d->strides[i] > kMaxBytes)
        return fail(BMM_EINVAL, "box_copy: stride[%lld] = %lld must be positive", i,
                    d->strides[i]);
      if (d->strides[i] % 16)
        return fail(BMM_EALIGN, "box_copy: outer stride[%lld] = %lld not a multiple of 16", i,
                    d->strides[i]);
    }
    int64_t s = mul_capped({d->dims[i] - 1, d->strides[i]});
    if (s < 0 || span + s > kMaxBytes) return fail(BMM_EINVAL, "box_copy: tensor too large");
    span += s;
  }
  span += eb;
  const int64_t image = box_elems * eb;
  if (image > kBoxImageLimit)
    return fail(BMM_ERANGE, "box_copy: one repeat's image is %lld bytes, limit %lld", image,
                kBoxImageLimit);
  if (!dst || !src) return fail(BMM_EINVAL, "box_copy: null pointer");
  if (!aligned16(dst) || !aligned16(src))
    return fail(BMM_EALIGN, "box_copy: dst_image and src must be 16-byte aligned");
  const int64_t total = mul_capped({image, d->n_repeat});
  if (total < 0) return fail(BMM_EINVAL, "box_copy: image too large");
  if (overlaps(dst, total, src, span)) return fail(BMM_EOVERLAP, "box_copy: dst overlaps src");
  return Status{};
}

Status check_mma(const float* D, const uint32_t* A, const uint32_t* B, const float* C,
                 int64_t batch, int64_t M_rep, int64_t N_rep, int64_t K_rep, int32_t dtype,
                 int32_t kernel, int32_t atom_k) {
  if (atom_k != 16 && atom_k != 8)
    return fail(BMM_EINVAL, "mma_tile: atom_k must be 16 or 8, got %lld", atom_k);
  if (dtype != BMM_F16 && dtype != BMM_BF16)
    return fail(BMM_EINVAL, "mma_tile: dtype %lld is neither BMM_F16 nor BMM_BF16", dtype);
  if (kernel < BMM_KERNEL_AUTO || kernel > BMM_KERNEL_SKINNY)
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

}  // namespace bmm
