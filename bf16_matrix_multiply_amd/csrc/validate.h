// Host-side argument checks for every entry point. Pure C++ (no HIP calls),
// so each rejection path runs without a GPU.
#pragma once

#include <stdint.h>
#include <string>

#include "../../include/bmm.h"

namespace bmm {

struct Status {
  int code = BMM_OK;
  std::string msg;
  bool ok() const { return code == BMM_OK; }
};

// Sets the message bmm_last_error returns on this thread (defined with the
// entry points).
void set_last_error(const std::string& msg);

Status check_pack(const uint32_t* dst, const uint16_t* src, int64_t batch, int64_t rows,
                  int64_t K, int64_t ld_src, int32_t atom_rows, int32_t atom_k);

Status check_pack_kmajor(const uint32_t* dst, const uint16_t* src, int64_t batch, int64_t rows,
                         int64_t K, int64_t ld_src, int32_t atom_rows,
                         int32_t atom_k);

Status check_box(const void* dst, const void* src, const bmm_box_desc* d);

// Store (elem_type 0) or add reduction (a bmm_elem_type) into a global box;
// `what` prefixes the messages.
Status check_box_store(const void* dst, const void* img, const bmm_box_desc* d,
                       int32_t elem_type, const char* what);

Status check_mma(const float* D, const uint32_t* A, const uint32_t* B, const float* C,
                 int64_t batch, int64_t M_rep, int64_t N_rep, int64_t K_rep, int32_t dtype,
                 int32_t kernel, int32_t atom_k);

// Split count actually used: min(splits, number of 32-value K steps).
int64_t splitk_effective(int64_t K_rep, int32_t atom_k, int32_t splits);

Status check_splitk(const float* D, const uint32_t* A, const uint32_t* B, const float* C,
                    int64_t batch, int64_t M_rep, int64_t N_rep, int64_t K_rep, int32_t dtype,
                    int32_t atom_k, int32_t splits, const void* workspace,
                    int64_t workspace_bytes);

// Largest image (bytes) one box repeat may stage through LDS.
constexpr int64_t kBoxImageLimit = 65536;

}  // namespace bmm
