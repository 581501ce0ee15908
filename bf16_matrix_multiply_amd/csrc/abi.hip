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

// Shape rule of BMM_KERNEL_AUTO (K counted in values): the LDS-staged kernel
// once there are enough 256 x 256 macro tiles to occupy the 256 CUs; the
// B-streaming kernel when D has at most 64 rows and B is large (at least 16 MB
// per batch); otherwise one wave per 16 x 16 block.
int choose_kernel(int64_t batch, int64_t M_rep, int64_t N_rep, int64_t K) {
  const int64_t macro_tiles = batch * ((M_rep + 15) / 16) * ((N_rep + 31) / 32);
  if (macro_tiles >= 128 && K < bmm::kTiledMaxK) return BMM_KERNEL_TILED;
  if (M_rep <= 4 && N_rep * K >= 16 * 65536) return BMM_KERNEL_SKINNY;
  return BMM_KERNEL_DIRECT;
}

}  // namespace

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
  bmm::Status st = bmm::check_pack_kmajor(dst, src, batch, rows, K, ld_src, atom_rows);
  if (!st.ok()) return report(st);
  if (batch == 0 || rows == 0 || K == 0) return report(st);
  return hip_status(bmm::launch_pack_kmajor(dst, src, batch, rows, K, ld_src, atom_rows,
                                            static_cast<hipStream_t>(stream)),
                    "pack_operand_kmajor launch");
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
    case BMM_KERNEL_DIRECT: return hip_status(bmm::launch_mma_direct(a0, s), "mma_tile direct launch");
    case BMM_KERNEL_TILED:
      if (K >= bmm::kTiledMaxK) {
        g_last_error = "mma_tile: the tiled kernel takes K < 4194304 values";
        return BMM_EINVAL;
      }
      return hip_status(bmm::launch_mma_tiled(a0, s), "mma_tile tiled launch");
    default: return hip_status(bmm::launch_mma_skinny(a0, s), "mma_tile skinny launch");
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

int bmm_mma_tile(float* D, const uint32_t* A, const uint32_t* B, const float* C,
                 float c_scalar, int64_t batch, int64_t M_rep, int64_t N_rep, int64_t K_rep,
                 bmm_dtype dtype, void* stream) {
  return bmm_mma_tile_with(D, A, B, C, c_scalar, batch, M_rep, N_rep, K_rep, dtype,
                           BMM_KERNEL_AUTO, stream);
}

}  // extern "C"
