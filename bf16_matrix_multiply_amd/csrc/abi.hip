// extern "C" entry points declared in include/bmm.h: validate on the host,
// then enqueue the kernels on the caller's stream.
#include <cstring>
#include <string>

#include "launch.h"
#include "validate.h"

namespace {

thread_local std::string g_last_error;

int report(const bmm::Status& st) {
  g_last_error = st.msg;
  return st.code;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) {
    g_last_error.clear();
    return BMM_OK;
  }
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return BMM_EHIP;
}

// Launch-grid limits of the kernels (one workgroup per 256 x 256 tile; the
// skinny kernel's grid is (N/64, M groups, batch); the direct kernel has one
// wave per 16 x 16 block, four per workgroup).
bool tiled_fits(int64_t batch, int64_t M_rep, int64_t N_rep, int64_t K, int tile = 256,
                int tile_n = 0) {
  const int64_t ma = tile / 16, na = (tile_n ? tile_n : tile) / 8;  // M and N atoms per tile
  return K < bmm::kTiledMaxK && batch * ((M_rep + ma - 1) / ma) * ((N_rep + na - 1) / na) <= 0x7fffffff;
}
bool skinny_fits(int64_t batch, int64_t M_rep, int64_t N_rep) {
  return batch <= 65535 && (M_rep + 3) / 4 <= 65535 && (N_rep + 7) / 8 <= 0x7fffffff;
}
bool direct_fits(int64_t batch, int64_t M_rep, int64_t N_rep) {
  return (batch * M_rep * ((N_rep + 1) / 2) + 3) / 4 <= 0x7fffffff;
}

// Shape rule of BMM_KERNEL_AUTO (K counted in values), from a sweep of the
// kernels over shapes from 16 x 1024 x 1024 to 8192^3 on MI355X (bf16, normal
// operands, 4-wave tiles):
// - 256 x 256 LDS tiles when there are more than 128 (3072^3, 144 tiles:
//   59.0 us against 66.8 with 128 x 128 tiles and 73.6 with 256 x 128). With
//   128 or fewer the large tiles leave half the CUs idle (8192 x 1024 x 8192,
//   128 tiles: 136.4 us);
// - 256 x 128 LDS tiles (one workgroup per CU) when there are more than 128
//   of them (8192 x 1024 x 8192, 256 tiles: 102.3 against 111.0 us with
//   128 x 128 tiles; 2304 x 2304 x 4096, 162 tiles: 46.8 against 50.3; 2560^3,
//   200 tiles: 34.7 against 36.1). With 128 of them the 128 x 128 tile wins
//   (2048 x 2048 x 8192: 87.2 against 70.7 us; 1024 x 4096 x 4096: 44.8
//   against 39.0);
// - 128 x 128 LDS tiles when there are at least 128 full ones (2048^3: 22.8
//   us against 26.8 with 256 x 128 and 38.6 with 256 x 256; 1536^3: 18.4
//   against 21.3 and 31.4);
// - otherwise the K-splitting, B-streaming kernel, fastest or tied for every
//   shape with fewer tiles (1024 x 1024 x 8192: 41.0 against 66.6 us;
//   256 x 4096 x 4096: 23.9 against 36.0 us);
// - the direct kernel where the others' launch grids would overflow.
int choose_kernel(int64_t batch, int64_t M_rep, int64_t N_rep, int64_t K) {
  const int64_t tiles256 = batch * ((M_rep + 15) / 16) * ((N_rep + 31) / 32);
  const int64_t tiles128 = batch * ((M_rep + 7) / 8) * ((N_rep + 15) / 16);
  const int64_t tiles256x128 = batch * ((M_rep + 15) / 16) * ((N_rep + 15) / 16);
  if (M_rep >= 16 && N_rep >= 32 && tiles256 > 128 && tiled_fits(batch, M_rep, N_rep, K))
    return BMM_KERNEL_TILED;
  if (M_rep >= 16 && N_rep >= 16 && tiles256x128 > 128 &&
      tiled_fits(batch, M_rep, N_rep, K, 256, 128))
    return BMM_KERNEL_TILED_256x128;
  if (M_rep >= 8 && N_rep >= 16 && tiles128 >= 128 && tiled_fits(batch, M_rep, N_rep, K, 128))
    return BMM_KERNEL_TILED_128;
  if (skinny_fits(batch, M_rep, N_rep)) return BMM_KERNEL_SKINNY;
  if (direct_fits(batch, M_rep, N_rep)) return BMM_KERNEL_DIRECT;
  if (tiled_fits(batch, M_rep, N_rep, K, 128)) return BMM_KERNEL_TILED_128;
  return BMM_KERNEL_DIRECT;  // rejected below with a message
}

// Repeats t < u touch disjoint global boxes when some dimension steps by at
// least the box extent (then every later repeat is further away still).
bool repeats_disjoint(const bmm_box_desc& d) {
  if (d.n_repeat == 1) return true;
  for (int i = 0; i < d.rank; ++i) {
    const int64_t st = d.coord_step[i] < 0 ? -d.coord_step[i] : d.coord_step[i];
    if (st >= d.box[i]) return true;
  }
  return false;
}

int box_store_common(void* dst, const void* img, const bmm_box_desc& d, int elem_type,
                     int64_t* bytes_moved, void* stream, const char* what) {
  int64_t elems = 1;
  for (int i = 0; i < d.rank; ++i) elems *= d.box[i];
  const int rc = hip_status(bmm::launch_box_store(dst, img, d, elem_type, repeats_disjoint(d),
                                                  static_cast<hipStream_t>(stream)),
                            what);
  if (rc == BMM_OK && bytes_moved) *bytes_moved = elems * d.elem_bytes * d.n_repeat;
  return rc;
}

}  // namespace

namespace bmm {
void set_last_error(const std::string& msg) { g_last_error = msg; }
}  // namespace bmm

extern "C" {

int bmm_abi_version(void) { return 1; }

const char* bmm_last_error(void) { return g_last_error.c_str(); }

int bmm_pack_operand(uint32_t* dst, const uint16_t* src, int64_t batch, int64_t rows,
                     int64_t K, int64_t ld_src, int32_t atom_rows, void* stream) {
  bmm::Status st = bmm::check_pack(dst, src, batch, rows, K, ld_src, atom_rows, 16);
  if (!st.ok()) return report(st);
  if (batch == 0 || rows == 0 || K == 0) return report(st);
  return hip_status(bmm::launch_pack(dst, src, batch, rows, K, ld_src, atom_rows, 16,
                                     static_cast<hipStream_t>(stream)),
                    "pack_operand launch");
}

int bmm_pack_operand_k8(uint32_t* dst, const uint16_t* src, int64_t batch, int64_t rows,
                        int64_t K, int64_t ld_src, int32_t atom_rows, void* stream) {
  bmm::Status st = bmm::check_pack(dst, src, batch, rows, K, ld_src, atom_rows, 8);
  if (!st.ok()) return report(st);
  if (batch == 0 || rows == 0 || K == 0) return report(st);
  return hip_status(bmm::launch_pack(dst, src, batch, rows, K, ld_src, atom_rows, 8,
                                     static_cast<hipStream_t>(stream)),
                    "pack_operand_k8 launch");
}

int bmm_pack_operand_kmajor(uint32_t* dst, const uint16_t* src, int64_t batch, int64_t rows,
                            int64_t K, int64_t ld_src, int32_t atom_rows, void* stream) {
  bmm::Status st = bmm::check_pack_kmajor(dst, src, batch, rows, K, ld_src, atom_rows, 16);
  if (!st.ok()) return report(st);
  if (batch == 0 || rows == 0 || K == 0) return report(st);
  return hip_status(bmm::launch_pack_kmajor(dst, src, batch, rows, K, ld_src, atom_rows, 16,
                                            static_cast<hipStream_t>(stream)),
                    "pack_operand_kmajor launch");
}

int bmm_pack_operand_kmajor_k8(uint32_t* dst, const uint16_t* src, int64_t batch, int64_t rows,
                               int64_t K, int64_t ld_src, int32_t atom_rows, void* stream) {
  bmm::Status st = bmm::check_pack_kmajor(dst, src, batch, rows, K, ld_src, atom_rows, 8);
  if (!st.ok()) return report(st);
  if (batch == 0 || rows == 0 || K == 0) return report(st);
  return hip_status(bmm::launch_pack_kmajor(dst, src, batch, rows, K, ld_src, atom_rows, 8,
                                            static_cast<hipStream_t>(stream)),
                    "pack_operand_kmajor_k8 launch");
}

int bmm_box_copy(void* dst_image, const void* src, const bmm_box_desc* desc,
                 int64_t* bytes_moved, void* stream) {
  bmm::Status st = bmm::check_box(dst_image, src, desc);
  if (!st.ok()) return report(st);
  int64_t elems = 1;
  for (int i = 0; i < desc->rank; ++i) elems *= desc->box[i];
  const int rc = hip_status(bmm::launch_box(dst_image, src, *desc, static_cast<hipStream_t>(stream)),
                            "box_copy launch");
  if (rc == BMM_OK && bytes_moved) *bytes_moved = elems * desc->elem_bytes * desc->n_repeat;
  return rc;
}

int bmm_box_store(void* dst, const void* src_image, const bmm_box_desc* desc,
                  int64_t* bytes_moved, void* stream) {
  bmm::Status st = bmm::check_box_store(dst, src_image, desc, 0, "box_store");
  if (!st.ok()) return report(st);
  return box_store_common(dst, src_image, *desc, 0, bytes_moved, stream, "box_store launch");
}

int bmm_box_reduce_add(void* dst, const void* src_image, const bmm_box_desc* desc,
                       int32_t elem_type, int64_t* bytes_moved, void* stream) {
  if (elem_type < BMM_ELEM_F32 || elem_type > BMM_ELEM_I64) {
    g_last_error = "box_reduce_add: elem_type " + std::to_string(elem_type) +
                   " is not a bmm_elem_type";
    return BMM_EINVAL;
  }
  bmm::Status st = bmm::check_box_store(dst, src_image, desc, elem_type, "box_reduce_add");
  if (!st.ok()) return report(st);
  return box_store_common(dst, src_image, *desc, elem_type, bytes_moved, stream,
                          "box_reduce_add launch");
}

int bmm_select_kernel(int64_t batch, int64_t M_rep, int64_t N_rep, int64_t K_rep) {
  if (batch < 0 || M_rep < 0 || N_rep < 0 || K_rep < 0) return BMM_EINVAL;
  if (K_rep > (int64_t(1) << 26)) return BMM_EINVAL;
  return choose_kernel(batch, M_rep, N_rep, 16 * K_rep);
}

namespace {

int mma_common(const bmm::MmaArgs& a0, int32_t kernel, void* stream) {
  bmm::Status st = bmm::check_mma(a0.D, a0.A, a0.B, a0.C, a0.batch, a0.M_rep, a0.N_rep,
                                  a0.K_rep, a0.dtype, kernel, a0.atom_k);
  if (!st.ok()) return report(st);
  if (a0.batch == 0 || a0.M_rep == 0 || a0.N_rep == 0) return report(st);
  const int64_t K = a0.K_rep * a0.atom_k;
  if (kernel == BMM_KERNEL_AUTO) kernel = choose_kernel(a0.batch, a0.M_rep, a0.N_rep, K);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (kernel) {
    case BMM_KERNEL_DIRECT:
      if (!direct_fits(a0.batch, a0.M_rep, a0.N_rep)) {
        g_last_error = "mma_tile: too many 16 x 16 blocks for one direct-kernel launch";
        return BMM_EINVAL;
      }
      return hip_status(bmm::launch_mma_direct(a0, s), "mma_tile direct launch");
    case BMM_KERNEL_TILED:
    case BMM_KERNEL_TILED_256x128:
    case BMM_KERNEL_TILED_128: {
      const int tile = kernel == BMM_KERNEL_TILED_128 ? 128 : 256;
      const int tile_n = kernel == BMM_KERNEL_TILED_256x128 ? 128 : 0;
      if (K >= bmm::kTiledMaxK) {
        g_last_error = "mma_tile: the tiled kernel takes K < 4194304 values";
        return BMM_EINVAL;
      }
      if (!tiled_fits(a0.batch, a0.M_rep, a0.N_rep, K, tile, tile_n)) {
        g_last_error = "mma_tile: too many macro tiles for one tiled-kernel launch";
        return BMM_EINVAL;
      }
      bmm::MmaArgs a = a0;
      a.tile = tile;
      a.tile_n = tile_n;
      return hip_status(bmm::launch_mma_tiled(a, s), "mma_tile tiled launch");
    }
    default:
      if (!skinny_fits(a0.batch, a0.M_rep, a0.N_rep)) {
        g_last_error = "mma_tile: the skinny kernel takes batch <= 65535 and M_rep <= 262140";
        return BMM_EINVAL;
      }
      return hip_status(bmm::launch_mma_skinny(a0, s), "mma_tile skinny launch");
  }
}

}  // namespace

int bmm_mma_tile_with(float* D, const uint32_t* A, const uint32_t* B, const float* C,
                      float c_scalar, int64_t batch, int64_t M_rep, int64_t N_rep,
                      int64_t K_rep, bmm_dtype dtype, int32_t kernel, void* stream) {
  const bmm::MmaArgs a{D, A, B, C, c_scalar, batch, M_rep, N_rep, K_rep, int(dtype), 0, 1.f, 1.f, 16};
  return mma_common(a, kernel, stream);
}

int bmm_mma_tile_scaled(float* D, const uint32_t* A, const uint32_t* B, const float* C,
                        float c_scalar, float alpha, float beta, int64_t batch, int64_t M_rep,
                        int64_t N_rep, int64_t K_rep, bmm_dtype dtype, int32_t kernel,
                        void* stream) {
  const bmm::MmaArgs a{D, A, B, C, c_scalar, batch, M_rep, N_rep, K_rep, int(dtype), 1, alpha, beta, 16};
  return mma_common(a, kernel, stream);
}

int bmm_mma_tile_opts(float* D, const uint32_t* A, const uint32_t* B, const float* C,
                      float c_scalar, int64_t batch, int64_t M_rep, int64_t N_rep, int64_t K_rep,
                      bmm_dtype dtype, const bmm_mma_opts* opts, void* stream) {
  const bmm_mma_opts o = opts ? *opts : bmm_mma_opts{16, BMM_KERNEL_AUTO, 0, 1.f, 1.f};
  if (o.scaled != 0 && o.scaled != 1) {
    g_last_error = "mma_tile_opts: scaled must be 0 or 1";
    return BMM_EINVAL;
  }
  const bmm::MmaArgs a{D, A, B, C, c_scalar, batch, M_rep, N_rep, K_rep, int(dtype),
                       o.scaled, o.scaled ? o.alpha : 1.f, o.scaled ? o.beta : 1.f, o.atom_k};
  return mma_common(a, o.kernel, stream);
}

}  // extern "C"

namespace {

// Macro tile of the split-K form: 256 x 256 when there are at least 128 such
// tiles (then the default count makes tiles x splits fill the chip one
// workgroup per CU), or from 16384 K values when at most 32 splits of them
// still fill it (8 tiles or more); 128 x 128 otherwise. Measured
// best-over-splits (us, 256 / 128 tiles): 1024 x 1024 x 8192 36.2 / 31.6,
// 64 x 8192 x 8192 33.9 / 27.5, 2048 x 2048 x 8192 74.0 / 75.1, 8192 x 1024
// x 8192 121.3 (2 splits) / 132.5, 3072 x 3072 x 8192 144.5 / 161.2,
// 2048 x 2048 x 16384 118.5 / 131.2, 1024 x 1024 x 65536 121.0 / 139.2,
// 512 x 512 x 65536 (4 large tiles) 57.1 / 47.1.
int splitk_tile(int64_t batch, int64_t M_rep, int64_t N_rep, int64_t K) {
  const int64_t tiles256 = batch * ((M_rep + 15) / 16) * ((N_rep + 31) / 32);
  return tiles256 >= 128 || (K >= 16384 && tiles256 >= 8) ? 256 : 128;
}

}  // namespace

extern "C" {

int64_t bmm_mma_splitk_workspace_bytes(int64_t batch, int64_t M_rep, int64_t N_rep,
                                       int64_t K_rep, int32_t atom_k, int32_t splits) {
  if (batch < 0 || M_rep < 0 || N_rep < 0 || K_rep < 0 || K_rep > (int64_t(1) << 26) ||
      (atom_k != 16 && atom_k != 8) || splits < 1 || batch > (int64_t(1) << 40) ||
      M_rep > (int64_t(1) << 40) || N_rep > (int64_t(1) << 40))
    return BMM_EINVAL;
  const __int128 bytes = __int128(bmm::splitk_effective(K_rep, atom_k, splits)) * batch * M_rep *
                         N_rep * 512;
  if (bytes > (__int128(1) << 50)) return BMM_EINVAL;
  return int64_t(bytes);
}

int bmm_splitk_default(int64_t batch, int64_t M_rep, int64_t N_rep, int64_t K_rep,
                       int32_t atom_k) {
  if (batch < 0 || M_rep < 0 || N_rep < 0 || K_rep < 0 || K_rep > (int64_t(1) << 26) ||
      (atom_k != 16 && atom_k != 8))
    return BMM_EINVAL;
  // Enough tiles x splits (tiles of the size splitk_tile picks) to give every
  // CU a workgroup, with each split at least 32 steps (1024 K values) deep so
  // that its partial-sum traffic stays small against its MFMA time (measured
  // best or within 10% of best at 1024 x 1024 x 8192, 64 x 8192 x 8192,
  // 2048 x 2048 x 8192, 1024 x 1024 x 65536 and 512 x 512 x 65536).
  const int64_t steps = (K_rep * atom_k + 31) / 32;
  const int tile = splitk_tile(batch, M_rep, N_rep, K_rep * atom_k);
  const int64_t ta = tile / 16, tb = tile / 8;
  const int64_t tiles = batch * ((M_rep + ta - 1) / ta) * ((N_rep + tb - 1) / tb);
  // (rounded down: 144 tiles stay whole, as two splits would leave a second
  // partial wave of workgroups)
  int64_t s = tiles > 0 ? 256 / tiles : 1;
  if (s > steps / 32) s = steps / 32;
  // at most 32 partial sums: at 512 x 512 x 65536, 32 splits took 66 us and
  // 64 splits 82 us (the reduce reads every partial once)
  if (s > 32) s = 32;
  if (s > 65535) s = 65535;
  return int(s < 1 ? 1 : s);
}

// Whether the split-K form beats the plain entry point for a shape, from a
// sweep of both over 28 shapes (bf16, normal operands; MI355X). Splitting won
// exactly where K >= 4096, M >= 32, AUTO would run the skinny or the 128 x 128
// kernel and the default split count is above one: 1024 x 1024 x 8192 (30.1
// against 41.0 us), 2048 x 1024 x 4096 (30.1 / 36.5), 256 x 4096 x 4096
// (22.4 / 23.9), 64 x 8192 x 8192 (27.5 / 44.1), 32 x 16384 x 4096 (26.4 /
// 28.9), 1024 x 1024 x 65536 (113.6 / 337.1), 512 x 512 x 65536 (48.7 /
// 270.4). It lost with K = 2048 (512 x 2048 x 2048: 20.3 / 13.3), with M = 16
// (16 x 16384 x 16384, where the skinny kernel streams B once: 105.7 / 87.0)
// and on the 256 x 128 tile (8192 x 1024 x 8192: 113.9 / 102.3).
int bmm_splitk_suggested(int64_t batch, int64_t M_rep, int64_t N_rep, int64_t K_rep,
                         int32_t atom_k) {
  const int s = bmm_splitk_default(batch, M_rep, N_rep, K_rep, atom_k);
  if (s <= 1) return s;
  const int64_t K = K_rep * atom_k;
  const int k = choose_kernel(batch, M_rep, N_rep, K);
  return K >= 4096 && M_rep >= 2 && (k == BMM_KERNEL_SKINNY || k == BMM_KERNEL_TILED_128) ? s
                                                                                        : 1;
}

int bmm_mma_tile_splitk(float* D, const uint32_t* A, const uint32_t* B, const float* C,
                        float c_scalar, int64_t batch, int64_t M_rep, int64_t N_rep,
                        int64_t K_rep, bmm_dtype dtype, int32_t atom_k, int32_t splits,
                        float* workspace, int64_t workspace_bytes, void* stream) {
  bmm::Status st = bmm::check_splitk(D, A, B, C, batch, M_rep, N_rep, K_rep, int(dtype), atom_k,
                                     splits, workspace, workspace_bytes);
  if (!st.ok()) return report(st);
  if (batch == 0 || M_rep == 0 || N_rep == 0) return report(st);
  const int tile = splitk_tile(batch, M_rep, N_rep, K_rep * atom_k);
  if (!tiled_fits(batch, M_rep, N_rep, K_rep * atom_k, tile)) {
    g_last_error = "mma_tile_splitk: too many macro tiles for one launch";
    return BMM_EINVAL;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t S = bmm::splitk_effective(K_rep, atom_k, splits);
  const int64_t d_floats = batch * M_rep * N_rep * 128;
  if (S > 0) {
    // partial sums from zero, one per split, into the workspace
    bmm::MmaArgs a{workspace, A, B, nullptr, 0.f, batch, M_rep, N_rep, K_rep, int(dtype), 0,
                   1.f, 1.f, atom_k};
    a.splits = int(S);
    a.steps = (K_rep * atom_k + 31) / 32;
    a.part_floats = d_floats;
    a.tile = tile;
    const int rc = hip_status(bmm::launch_mma_tiled(a, s), "mma_tile_splitk tiled launch");
    if (rc != BMM_OK) return rc;
  }
  return hip_status(bmm::launch_splitk_reduce(D, C, c_scalar, workspace, int(S), d_floats,
                                              d_floats / 4, s),
                    "mma_tile_splitk reduce launch");
}

int bmm_mma_tile(float* D, const uint32_t* A, const uint32_t* B, const float* C,
                 float c_scalar, int64_t batch, int64_t M_rep, int64_t N_rep, int64_t K_rep,
                 bmm_dtype dtype, void* stream) {
  return bmm_mma_tile_with(D, A, B, C, c_scalar, batch, M_rep, N_rep, K_rep, dtype,
                           BMM_KERNEL_AUTO, stream);
}

}  // extern "C"
