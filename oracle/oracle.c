/*
 * CPU oracle for the tiled f16/bf16 multiply-accumulate D = A * B^T + C.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. The HIP product path
 * neither links nor calls it, and this file shares no code, header, table or
 * helper with that path.
 *
 * Plain, slow, obviously correct: every function is the definition from the
 * pages written out as loops, with no blocking or reordering. Sources (Apache
 * TVM "tirx" tile-op documentation):
 *   - mma.sync page, "Operand coordinates and ownership" (shapes table): the
 *     packed A (M_repeat, K_repeat, 16, k/2), B (N_repeat, K_repeat, 8, k/2)
 *     and D / tensor C (M_repeat, N_repeat, 16, 8) float32 layouts; k = 16.
 *   - mma.sync page, "Example: a 16x8 result with two K16 issues": the host
 *     packing (reshape + transpose + view as uint32), hence the even K value
 *     sits in the low 16 bits of a word on a little-endian host.
 *   - mma.sync page, "Accumulation, transpose and alpha/beta": repeat order
 *     batch, M, N, then K; C is a tensor or a scalar broadcast; only the first
 *     K issue reads C, later issues read D.
 *   - fma page, "Operand specification": a*b+c is a single rounding.
 *   - cp.async.bulk.tensor page, "Operands and descriptor fields" and
 *     "Example: two explicit 8x16 boxes": box / coords / coord_steps, the
 *     compact (repeat, box...) image, out-of-bounds fill defaulting to zero.
 *   - cp.async.bulk.tensor page, "Stores, reductions, and completion": the
 *     store and the add reduction take the same box contract with the global
 *     tensor as destination; a reduction destination holds its starting
 *     value before the first reduction (the split-K form's C).
 *   - mma.sync page introduction and shapes table: the m16n8k8 form (k = 8
 *     atoms, k/2 = 4 words per atom row).
 *
 * Readings where the pages leave a step open:
 *   - within one hardware issue the summation order is not stated; the oracle
 *     sums k in ascending order, one fp32 rounding per step (the accumulator
 *     is float32 on the pages). Each product of two f16 (11-bit significand)
 *     or two bf16 (8-bit) values is exact in fp32, so acc + a*b is one
 *     rounding, the same as a fused multiply-add.
 *   - a leading batch axis on A, B, C and D; batches are independent, and the
 *     scalar C broadcasts over all of them.
 *   - K_repeat = 0 leaves the empty sum: D = C.
 *
 * Pins (all in the CPU test suite): the page's own packing recipe and an
 * arange closed form for the packer; round trip over all 65536 bit patterns;
 * numpy/torch half decoders for h2f; int64 exact arithmetic for quarter-
 * integer inputs (the page's worked example is one); float64 numpy matmul
 * within the fp32 error bound for normal inputs; the page's two-box example
 * for the box copy and store; brute-force padding for out-of-bounds boxes;
 * numpy float32/float16, torch bfloat16 and wrap-around integer additions for
 * the add reduction; single-rounding cases that fix the split-K boundaries
 * and the order in which partial sums meet C.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F16 = 0, ORACLE_BF16 = 1 };

int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---- half-precision decode (IEEE-754 binary16; bfloat16 = top half of binary32) ---- */

float oracle_h2f(uint16_t h, int dtype) {
  if (dtype == ORACLE_BF16) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
  }
  /* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
  int sign = (h >> 15) & 1;
  int expo = (h >> 10) & 0x1f;
  int frac = h & 0x3ff;
  float v;
  if (expo == 0)
    v = ldexpf((float)frac, -24);                /* zero / subnormal: frac * 2^-24 */
  else if (expo == 31)
    v = frac ? NAN : INFINITY;
  else
    v = ldexpf((float)(frac + 1024), expo - 25); /* (1 + frac/1024) * 2^(expo-15) */
  return sign ? -v : v;
}

void oracle_h2f_array(float* out, const uint16_t* in, int64_t n, int dtype) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_h2f(in[i], dtype);
}

/* ---- packing: row-major halves -> packed b32 atoms ----
 * X is (batch, rows, K) with row stride ld (elements), batch stride rows*ld.
 * P is (batch, rows/R, K/16, R, 8) words, R = 16 for A and 8 for B:
 *   P[b, r, kr, i, w] = X[b, R*r+i, 16*kr+2*w] | X[b, R*r+i, 16*kr+2*w+1] << 16
 */
int oracle_pack(uint32_t* P, const uint16_t* X, int64_t batch, int64_t rows, int64_t K,
                int64_t ld, int64_t R) {
  if ((R != 16 && R != 8) || rows % R || K % 16 || ld < K) return -1;
  const int64_t rows_rep = rows / R, K_rep = K / 16;
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t r = 0; r < rows_rep; ++r)
      for (int64_t kr = 0; kr < K_rep; ++kr)
        for (int64_t i = 0; i < R; ++i)
          for (int64_t w = 0; w < 8; ++w) {
            const uint16_t* row = X + b * rows * ld + (R * r + i) * ld;
            uint32_t lo = row[16 * kr + 2 * w];
            uint32_t hi = row[16 * kr + 2 * w + 1];
            P[(((b * rows_rep + r) * K_rep + kr) * R + i) * 8 + w] = lo | (hi << 16);
          }
  return 0;
}

/* Packing from a K-major source: X is (batch, K, ld) with X[b, k, row] the
 * logical element (row, k) (the transpose of the row-major case), batch
 * stride K*ld. Same packed result as oracle_pack of the logical matrix:
 *   P[b, r, kr, i, w] = X[b, 16*kr+2*w, R*r+i] | X[b, 16*kr+2*w+1, R*r+i] << 16
 */
int oracle_pack_kmajor(uint32_t* P, const uint16_t* X, int64_t batch, int64_t rows, int64_t K,
                       int64_t ld, int64_t R) {
  if ((R != 16 && R != 8) || rows % R || K % 16 || ld < rows) return -1;
  const int64_t rows_rep = rows / R, K_rep = K / 16;
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t r = 0; r < rows_rep; ++r)
      for (int64_t kr = 0; kr < K_rep; ++kr)
        for (int64_t i = 0; i < R; ++i)
          for (int64_t w = 0; w < 8; ++w) {
            const uint16_t* col = X + b * K * ld + (R * r + i);
            uint32_t lo = col[(16 * kr + 2 * w) * ld];
            uint32_t hi = col[(16 * kr + 2 * w + 1) * ld];
            P[(((b * rows_rep + r) * K_rep + kr) * R + i) * 8 + w] = lo | (hi << 16);
          }
  return 0;
}

/* Packing with an atom K of 8 (the m16n8k8 form of the mma.sync page's
 * introduction; shapes table with k = 8): A is (rows/16, K/8, 16, 4) words,
 * B (rows/8, K/8, 8, 4):
 *   P[b, r, kr, i, w] = X[b, R*r+i, 8*kr+2*w] | X[b, R*r+i, 8*kr+2*w+1] << 16, w < 4
 */
int oracle_pack_k8(uint32_t* P, const uint16_t* X, int64_t batch, int64_t rows, int64_t K,
                   int64_t ld, int64_t R) {
  if ((R != 16 && R != 8) || rows % R || K % 8 || ld < K) return -1;
  const int64_t rows_rep = rows / R, K_rep = K / 8;
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t r = 0; r < rows_rep; ++r)
      for (int64_t kr = 0; kr < K_rep; ++kr)
        for (int64_t i = 0; i < R; ++i)
          for (int64_t w = 0; w < 4; ++w) {
            const uint16_t* src_row = X + b * rows * ld + (R * r + i) * ld;
            uint32_t lo = src_row[8 * kr + 2 * w];
            uint32_t hi = src_row[8 * kr + 2 * w + 1];
            P[(((b * rows_rep + r) * K_rep + kr) * R + i) * 4 + w] = lo | (hi << 16);
          }
  return 0;
}

/* Inverse of oracle_pack into a dense (batch, rows, K) array. */
int oracle_unpack(uint16_t* X, const uint32_t* P, int64_t batch, int64_t rows, int64_t K,
                  int64_t R) {
  if ((R != 16 && R != 8) || rows % R || K % 16) return -1;
  const int64_t rows_rep = rows / R, K_rep = K / 16;
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t row = 0; row < rows; ++row)
      for (int64_t k = 0; k < K; ++k) {
        uint32_t word =
            P[(((b * rows_rep + row / R) * K_rep + k / 16) * R + row % R) * 8 + (k % 16) / 2];
        X[(b * rows + row) * K + k] = (uint16_t)((word >> (16 * (k % 2))) & 0xFFFFu);
      }
  return 0;
}

/* ---- multiply-accumulate ---- */

/* Logical element (row, k) of a packed operand with atom height R and atom
 * K ka (16, or 8 for the m16n8k8 form): atom (row/R, k/ka), atom row row%R,
 * word (k%ka)/2, half k%2. */
static float packed_elem(const uint32_t* P, int64_t b, int64_t row, int64_t k, int64_t R,
                         int64_t rows_rep, int64_t K_rep, int64_t ka, int dtype) {
  uint32_t word =
      P[(((b * rows_rep + row / R) * K_rep + k / ka) * R + row % R) * (ka / 2) + (k % ka) / 2];
  return oracle_h2f((uint16_t)((word >> (16 * (k % 2))) & 0xFFFFu), dtype);
}

/* Offset of logical output (m, n) in the (batch, M_repeat, N_repeat, 16, 8) layout. */
static int64_t acc_offset(int64_t b, int64_t m, int64_t n, int64_t M_rep, int64_t N_rep) {
  return (((b * M_rep + m / 16) * N_rep + n / 8) * 16 + m % 16) * 8 + n % 8;
}

/* One output element: acc starts at C (read once), then every k in order. */
static float one_output(const uint32_t* A, const uint32_t* B, const float* C, float c,
                        int64_t b, int64_t m, int64_t n, int64_t M_rep, int64_t N_rep,
                        int64_t K_rep, int64_t ka, int dtype) {
  float acc = C ? C[acc_offset(b, m, n, M_rep, N_rep)] : c;
  for (int64_t k = 0; k < ka * K_rep; ++k) {
    float a = packed_elem(A, b, m, k, 16, M_rep, K_rep, ka, dtype);
    float x = packed_elem(B, b, n, k, 8, N_rep, K_rep, ka, dtype);
    acc = acc + a * x;
  }
  return acc;
}

/* D = A * B^T + C over the whole problem. C == NULL selects the scalar c;
 * ka is the atom K (16, or 8 for the m16n8k8 layout). */
int oracle_mma_k(float* D, const uint32_t* A, const uint32_t* B, const float* C, float c,
                 int64_t batch, int64_t M_rep, int64_t N_rep, int64_t K_rep, int64_t ka,
                 int dtype) {
  if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
  if (ka != 16 && ka != 8) return -1;
  const int64_t rows = batch * 16 * M_rep;
#pragma omp parallel for schedule(dynamic)
  for (int64_t bm = 0; bm < rows; ++bm) {
    const int64_t b = bm / (16 * M_rep), m = bm % (16 * M_rep);
    for (int64_t n = 0; n < 8 * N_rep; ++n)
      D[acc_offset(b, m, n, M_rep, N_rep)] =
          one_output(A, B, C, c, b, m, n, M_rep, N_rep, K_rep, ka, dtype);
  }
  return 0;
}

int oracle_mma(float* D, const uint32_t* A, const uint32_t* B, const float* C, float c,
               int64_t batch, int64_t M_rep, int64_t N_rep, int64_t K_rep, int dtype) {
  return oracle_mma_k(D, A, B, C, c, batch, M_rep, N_rep, K_rep, 16, dtype);
}

/* alpha/beta form, with the scaling at the call site (mma.sync page,
 * "Accumulation, transpose and alpha/beta"): the product is accumulated from
 * zero, k ascending, then D = fma(alpha, acc, fl(beta * C)) -- one rounding
 * for the final multiply-add (fma page, "Operand specification"). */
static float one_output_scaled(const uint32_t* A, const uint32_t* B, const float* C, float c,
                               float alpha, float beta, int64_t b, int64_t m, int64_t n,
                               int64_t M_rep, int64_t N_rep, int64_t K_rep, int dtype) {
  float acc = 0.0f;
  for (int64_t k = 0; k < 16 * K_rep; ++k) {
    float a = packed_elem(A, b, m, k, 16, M_rep, K_rep, 16, dtype);
    float x = packed_elem(B, b, n, k, 8, N_rep, K_rep, 16, dtype);
    acc = acc + a * x;
  }
  const float cv = C ? C[acc_offset(b, m, n, M_rep, N_rep)] : c;
  const float t = beta * cv;
  return fmaf(alpha, acc, t);
}

int oracle_mma_scaled(float* D, const uint32_t* A, const uint32_t* B, const float* C, float c,
                      float alpha, float beta, int64_t batch, int64_t M_rep, int64_t N_rep,
                      int64_t K_rep, int dtype) {
  if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
  const int64_t rows = batch * 16 * M_rep;
#pragma omp parallel for schedule(dynamic)
  for (int64_t bm = 0; bm < rows; ++bm) {
    const int64_t b = bm / (16 * M_rep), m = bm % (16 * M_rep);
    for (int64_t n = 0; n < 8 * N_rep; ++n)
      D[acc_offset(b, m, n, M_rep, N_rep)] =
          one_output_scaled(A, B, C, c, alpha, beta, b, m, n, M_rep, N_rep, K_rep, dtype);
  }
  return 0;
}

/* Split-K form: the K axis is cut at multiples of 32 values into S_eff =
 * min(splits, n) contiguous ranges of whole 32-value steps (n = ceil(K/32));
 * split s takes steps [s*n/S_eff, (s+1)*n/S_eff) (integer division), so every
 * range is non-empty. Each range is summed from zero, k ascending. The result
 * starts at C and the partial sums are added to it one at a time, s
 * ascending: the add reduction of the cp.async.bulk.tensor page ("Stores,
 * reductions, and completion"), whose destination holds the intended starting
 * value before the first reduction. K = 0 leaves D = C. */
static float one_output_splitk(const uint32_t* A, const uint32_t* B, const float* C, float c,
                               int64_t b, int64_t m, int64_t n, int64_t M_rep, int64_t N_rep,
                               int64_t K_rep, int64_t ka, int64_t splits, int dtype) {
  const int64_t K = ka * K_rep, steps = (K + 31) / 32;
  const int64_t S = splits < steps ? splits : steps;
  float d = C ? C[acc_offset(b, m, n, M_rep, N_rep)] : c;
  for (int64_t s = 0; s < S; ++s) {
    const int64_t lo = 32 * (s * steps / S);
    int64_t hi = 32 * ((s + 1) * steps / S);
    if (hi > K) hi = K;
    float part = 0.0f;
    for (int64_t k = lo; k < hi; ++k) {
      float a = packed_elem(A, b, m, k, 16, M_rep, K_rep, ka, dtype);
      float x = packed_elem(B, b, n, k, 8, N_rep, K_rep, ka, dtype);
      part = part + a * x;
    }
    d = d + part;
  }
  return d;
}

int oracle_mma_splitk(float* D, const uint32_t* A, const uint32_t* B, const float* C, float c,
                      int64_t batch, int64_t M_rep, int64_t N_rep, int64_t K_rep, int64_t ka,
                      int64_t splits, int dtype) {
  if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
  if ((ka != 16 && ka != 8) || splits < 1) return -1;
  const int64_t rows = batch * 16 * M_rep;
#pragma omp parallel for schedule(dynamic)
  for (int64_t bm = 0; bm < rows; ++bm) {
    const int64_t b = bm / (16 * M_rep), m = bm % (16 * M_rep);
    for (int64_t n = 0; n < 8 * N_rep; ++n)
      D[acc_offset(b, m, n, M_rep, N_rep)] =
          one_output_splitk(A, B, C, c, b, m, n, M_rep, N_rep, K_rep, ka, splits, dtype);
  }
  return 0;
}

int oracle_mma_splitk_sampled(float* out, const int64_t* idx, int64_t count, const uint32_t* A,
                              const uint32_t* B, const float* C, float c, int64_t batch,
                              int64_t M_rep, int64_t N_rep, int64_t K_rep, int64_t ka,
                              int64_t splits, int dtype) {
  if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
  if ((ka != 16 && ka != 8) || splits < 1) return -1;
  for (int64_t i = 0; i < count; ++i) {
    const int64_t *t = idx + 3 * i;
    if (t[0] < 0 || t[0] >= batch || t[1] < 0 || t[1] >= 16 * M_rep || t[2] < 0 ||
        t[2] >= 8 * N_rep)
      return -1;
  }
#pragma omp parallel for schedule(dynamic)
  for (int64_t i = 0; i < count; ++i)
    out[i] = one_output_splitk(A, B, C, c, idx[3 * i], idx[3 * i + 1], idx[3 * i + 2], M_rep,
                               N_rep, K_rep, ka, splits, dtype);
  return 0;
}

/* Selected outputs only: idx holds count triples (b, m, n); out[i] gets D[b, m, n]. */
int oracle_mma_sampled_k(float* out, const int64_t* idx, int64_t count, const uint32_t* A,
                         const uint32_t* B, const float* C, float c, int64_t batch,
                         int64_t M_rep, int64_t N_rep, int64_t K_rep, int64_t ka, int dtype) {
  if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
  if (ka != 16 && ka != 8) return -1;
  for (int64_t i = 0; i < count; ++i) {
    const int64_t *t = idx + 3 * i;
    if (t[0] < 0 || t[0] >= batch || t[1] < 0 || t[1] >= 16 * M_rep || t[2] < 0 ||
        t[2] >= 8 * N_rep)
      return -1;
  }
#pragma omp parallel for schedule(dynamic)
  for (int64_t i = 0; i < count; ++i)
    out[i] = one_output(A, B, C, c, idx[3 * i], idx[3 * i + 1], idx[3 * i + 2], M_rep, N_rep,
                        K_rep, ka, dtype);
  return 0;
}

int oracle_mma_sampled(float* out, const int64_t* idx, int64_t count, const uint32_t* A,
                       const uint32_t* B, const float* C, float c, int64_t batch,
                       int64_t M_rep, int64_t N_rep, int64_t K_rep, int dtype) {
  return oracle_mma_sampled_k(out, idx, count, A, B, C, c, batch, M_rep, N_rep, K_rep, 16, dtype);
}

/* ---- box copy (global tensor region -> compact image) ----
 * img[t, j_0, ..., j_{rank-1}] = G[coords + t*coord_step + j] when every
 * coordinate lies inside dims, else zero (the default out-of-bounds fill).
 * Strides are in bytes; the innermost stride equals the element size.
 * Returns the image bytes written (n_repeat * prod(box) * elem_bytes), the
 * quantity the page's example counts per barrier phase, or -1.
 */
int64_t oracle_box_copy(uint8_t* img, const uint8_t* G, int32_t rank, int32_t elem_bytes,
                        const int64_t* dims, const int64_t* strides, const int32_t* box,
                        const int64_t* coords, int32_t n_repeat, const int64_t* coord_step) {
  if (rank < 1 || rank > 5 || n_repeat < 1) return -1;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8) return -1;
  int64_t box_elems = 1;
  for (int d = 0; d < rank; ++d) {
    if (box[d] < 1 || box[d] > 256 || dims[d] < 1) return -1;
    box_elems *= box[d];
  }
  if (strides[rank - 1] != elem_bytes) return -1;
  for (int32_t t = 0; t < n_repeat; ++t) {
    for (int64_t e = 0; e < box_elems; ++e) {
      /* split e into box coordinates, innermost fastest */
      int64_t j[5], rem = e;
      for (int d = rank - 1; d >= 0; --d) {
        j[d] = rem % box[d];
        rem /= box[d];
      }
      int inside = 1;
      int64_t off = 0;
      for (int d = 0; d < rank; ++d) {
        int64_t g = coords[d] + (int64_t)t * coord_step[d] + j[d];
        if (g < 0 || g >= dims[d]) inside = 0;
        off += g * strides[d];
      }
      uint8_t* out = img + ((int64_t)t * box_elems + e) * elem_bytes;
      if (inside)
        memcpy(out, G + off, (size_t)elem_bytes);
      else
        memset(out, 0, (size_t)elem_bytes);
    }
  }
  return (int64_t)n_repeat * box_elems * elem_bytes;
}

/* ---- box store and add reduction (compact image -> global tensor region) ----
 * cp.async.bulk.tensor page, "Stores, reductions, and completion": the load's
 * coordinate/box contract with the global tensor as destination. For each
 * repeat t (ascending) and box element j (innermost fastest) whose global
 * coordinate coords + t*coord_step + j lies inside dims in every dimension:
 *   op 0 (store):  G[...] = img[t, j]
 *   op 1 (add):    G[...] = G[...] + img[t, j], one rounding per add in the
 *                  element type (1 f32, 2 f16, 3 bf16, 4 i32, 5 i64; integer
 *                  adds wrap modulo 2^32 / 2^64).
 * Elements outside dims are not written. Returns the image bytes consumed
 * (n_repeat * prod(box) * elem_bytes) or -1.
 */

/* x rounded to the nearest value with p significand bits, exponents in
 * [emin, emax] (gradual underflow below 2^emin), ties to even; beyond the
 * largest finite value it becomes infinity (IEEE-754 round to nearest). */
static double round_to_format(double x, int p, int emin, int emax) {
  if (x == 0.0 || !isfinite(x)) return x;
  int e;
  frexp(x, &e); /* |x| in [2^(e-1), 2^e) */
  int lead = e - 1;
  if (lead < emin) lead = emin;
  const double q = ldexp(1.0, lead - (p - 1)); /* spacing of representable values near x */
  const double r = nearbyint(x / q) * q;       /* default rounding mode: ties to even */
  const double max_finite = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
  if (fabs(r) > max_finite) return copysign(INFINITY, x);
  return r;
}

/* IEEE binary16 encoding of a value that binary16 represents exactly. */
static uint16_t f16_encode(double r) {
  if (isnan(r)) return 0x7e00u;
  const uint16_t sign = signbit(r) ? 0x8000u : 0u;
  const double a = fabs(r);
  if (isinf(a)) return (uint16_t)(sign | 0x7c00u);
  if (a < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)(a / ldexp(1.0, -24)));
  int e;
  const double f = frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
  return (uint16_t)(sign | (uint16_t)((e - 1 + 15) << 10) | (uint16_t)((2.0 * f - 1.0) * 1024.0));
}

/* bfloat16 encoding (top half of binary32) of a value bfloat16 represents exactly. */
static uint16_t bf16_encode(double r) {
  if (isnan(r)) return 0x7fc0u;
  const float f = (float)r;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static void add_into(uint8_t* g, const uint8_t* v, int elem_type) {
  if (elem_type == 1) {
    float x, y;
    memcpy(&x, g, 4);
    memcpy(&y, v, 4);
    const float z = x + y;
    memcpy(g, &z, 4);
  } else if (elem_type == 2 || elem_type == 3) {
    uint16_t x, y;
    memcpy(&x, g, 2);
    memcpy(&y, v, 2);
    const int dt = elem_type == 2 ? ORACLE_F16 : ORACLE_BF16;
    const double sum = (double)oracle_h2f(x, dt) + (double)oracle_h2f(y, dt);
    const uint16_t z = elem_type == 2 ? f16_encode(round_to_format(sum, 11, -14, 15))
                                      : bf16_encode(round_to_format(sum, 8, -126, 127));
    memcpy(g, &z, 2);
  } else if (elem_type == 4) {
    uint32_t x, y;
    memcpy(&x, g, 4);
    memcpy(&y, v, 4);
    const uint32_t z = x + y;
    memcpy(g, &z, 4);
  } else {
    uint64_t x, y;
    memcpy(&x, g, 8);
    memcpy(&y, v, 8);
    const uint64_t z = x + y;
    memcpy(g, &z, 8);
  }
}

int64_t oracle_box_store(uint8_t* G, const uint8_t* img, int32_t rank, int32_t elem_bytes,
                         const int64_t* dims, const int64_t* strides, const int32_t* box,
                         const int64_t* coords, int32_t n_repeat, const int64_t* coord_step,
                         int32_t op, int32_t elem_type) {
  if (rank < 1 || rank > 5 || n_repeat < 1 || (op != 0 && op != 1)) return -1;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8) return -1;
  if (op == 1) {
    static const int type_bytes[6] = {0, 4, 2, 2, 4, 8};
    if (elem_type < 1 || elem_type > 5 || type_bytes[elem_type] != elem_bytes) return -1;
  }
  int64_t box_elems = 1;
  for (int d = 0; d < rank; ++d) {
    if (box[d] < 1 || box[d] > 256 || dims[d] < 1) return -1;
    box_elems *= box[d];
  }
  if (strides[rank - 1] != elem_bytes) return -1;
  for (int32_t t = 0; t < n_repeat; ++t) {
    for (int64_t e = 0; e < box_elems; ++e) {
      int64_t j[5], rem = e;
      for (int d = rank - 1; d >= 0; --d) {
        j[d] = rem % box[d];
        rem /= box[d];
      }
      int inside = 1;
      int64_t off = 0;
      for (int d = 0; d < rank; ++d) {
        const int64_t g = coords[d] + coord_step[d] * (int64_t)t + j[d];
        if (g < 0 || g >= dims[d]) inside = 0;
        off += g * strides[d];
      }
      if (!inside) continue;
      const uint8_t* in = img + (e + (int64_t)t * box_elems) * elem_bytes;
      if (op == 0)
        memcpy(G + off, in, (size_t)elem_bytes);
      else
        add_into(G + off, in, elem_type);
    }
  }
  return (int64_t)n_repeat * box_elems * elem_bytes;
}
