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
  // atom K of the packed operands: 16 (m16n8k16 layout) or 8 (m16n8k8)
  int atom_k;
  // split-K (tiled kernel only): splits > 1 cuts the `steps` 32-value K steps
  // into that many ranges, partial sums from zero to D + s * part_floats
  int splits;
  int64_t steps, part_floats;
  // tiled kernel macro tile: tile rows 256 (default, also for 0) or 128;
  // tile_n columns: 0 for as many as rows, or 128 with 256 rows
  int tile;
  int tile_n;
};

// In 8-value K chunks, one 32-deep MFMA step spans the same bytes in either
// layout (A: 64 words per chunk per 16-row atom block, B: 32 words per 8-row
// block); only a lane's offset inside the step differs. Lane group g takes
// chunk g of the step: atom g/2, half g%2 for k = 16; atom g for k = 8.
__host__ __device__ inline int64_t k_chunks(const MmaArgs& a) { return a.K_rep * (a.atom_k / 8); }
__device__ inline int a_lane_words(int atom_k, int row, int g) {
  return atom_k == 16 ? (g >> 1) * 128 + row * 8 + (g & 1) * 4 : g * 64 + row * 4;
}
__device__ inline int b_lane_words(int atom_k, int row, int g) {
  return atom_k == 16 ? (g >> 1) * 64 + row * 8 + (g & 1) * 4 : g * 32 + row * 4;
}

hipError_t launch_pack(uint32_t* dst, const uint16_t* src, int64_t batch, int64_t rows,
                       int64_t K, int64_t ld, int R, int atom_k, hipStream_t s);
hipError_t launch_pack_kmajor(uint32_t* dst, const uint16_t* src, int64_t batch, int64_t rows,
                              int64_t K, int64_t ld, int R, int atom_k, hipStream_t s);
hipError_t launch_box(void* dst, const void* src, const bmm_box_desc& d, hipStream_t s);
// Store (elem_type 0) or add reduction of a compact image into a global box.
hipError_t launch_box_store(void* dst, const void* img, const bmm_box_desc& d, int elem_type,
                            bool repeats_disjoint, hipStream_t s);
hipError_t launch_mma_direct(const MmaArgs& a, hipStream_t s);
// The tiled kernel addresses one tile's operands with 32-bit buffer offsets:
// it takes K < 2^22.
constexpr int64_t kTiledMaxK = int64_t(1) << 22;
hipError_t launch_mma_tiled(const MmaArgs& a, hipStream_t s);
hipError_t launch_mma_skinny(const MmaArgs& a, hipStream_t s);
// D = C (or c) + part[0] + part[1] + ... + part[splits-1], added in that order;
// n4 = floats of D / 4, part s at parts + s * part_floats.
hipError_t launch_splitk_reduce(float* D, const float* C, float c, const float* parts,
                                int splits, int64_t part_floats, int64_t n4, hipStream_t s);

}  // namespace bmm
