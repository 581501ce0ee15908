// Internal launchers (host side). Arguments are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bmm.h"

namespace bmm {

struct MmaArgs {
  float* D;
  const uint32_t* A;
  const uint32_t* B;
  const float* C;  // null -> c_scalar
  float c_scalar;
  int64_t batch, M_rep, N_rep, K_rep;
  int dtype;
  // alpha/beta form: accumulate the product from zero, then
  // D = fma(alpha, acc, beta * C) (C or c_scalar) in the epilogue.
  int scaled;
  float alpha, beta;
};

hipError_t launch_pack(uint32_t* dst, const uint16_t* src, int64_t batch, int64_t rows,
                       int64_t K, int64_t ld, int R, hipStream_t s);
hipError_t launch_pack_kmajor(uint32_t* dst, const uint16_t* src, int64_t batch, int64_t rows,
                              int64_t K, int64_t ld, int R, hipStream_t s);
hipError_t launch_box(void* dst, const void* src, const bmm_box_desc& d, hipStream_t s);
hipError_t launch_mma_direct(const MmaArgs& a, hipStream_t s);
// The tiled kernel addresses one tile's operands with 32-bit buffer offsets:
// it takes K_rep < 2^18 (K < 4M).
constexpr int64_t kTiledMaxKRep = int64_t(1) << 18;
hipError_t launch_mma_tiled(const MmaArgs& a, hipStream_t s);
hipError_t launch_mma_skinny(const MmaArgs& a, hipStream_t s);

}  // namespace bmm
