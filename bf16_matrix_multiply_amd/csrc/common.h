// Device-side vocabulary shared by the gfx950 kernels: vector types, 16-byte
// global/LDS moves and the MFMA wrapper. CDNA4 only (64-lane wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bmm {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

enum : int { kF16 = 0, kBF16 = 1 };

constexpr int kWave = 64;

// Floats per accumulator atom (16 rows x 8 columns).
constexpr int kAtomFloats = 128;

// One v_mfma_f32_16x16x32_{f16,bf16}: acc[i][j] += sum_k x[i][k] * y[k][j].
// Lane l supplies row (l % 16) of x and column (l % 16) of y, each with the
// eight k values of its lane group (l / 16); it receives acc rows
// 4*(l/16) .. 4*(l/16)+3 of column l % 16. The products are exact and the
// k order within the step is the hardware's.
template <int DT>
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 x, u32x4 y, f32x4 acc) {
  if constexpr (DT == kBF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x),
                                                   __builtin_bit_cast(bf16x8, y), acc, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, x),
                                                  __builtin_bit_cast(f16x8, y), acc, 0, 0, 0);
  }
}

__device__ __forceinline__ u32x4 load16(const uint32_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Streaming (non-temporal) 16-byte load: data read once should not evict
// data that is reused.
__device__ __forceinline__ u32x4 load16_nt(const uint32_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ f32x4 load16f(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}

__device__ __forceinline__ void store16f(float* p, f32x4 v) {
  *reinterpret_cast<f32x4*>(p) = v;
}

// Streaming forms for data touched once (C read, D written): non-temporal,
// so they do not push the operand tiles other workgroups still need out of
// the caches.
__device__ __forceinline__ f32x4 load16f_nt(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}

__device__ __forceinline__ void store16f_nt(float* p, f32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}

}  // namespace bmm
