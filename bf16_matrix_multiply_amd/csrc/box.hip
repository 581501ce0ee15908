// Box transfers through an LDS image. The load: the role of the TMA tile-mode box load of the
// cp.async.bulk.tensor page ("Operands and descriptor fields", "Example: two
// explicit 8x16 boxes"), done the CDNA4 way. One workgroup stages one repeat:
// its lanes read the box from global memory with consecutive lanes on
// consecutive innermost elements (coalesced), substitute zero outside the
// tensor, and write the LDS image in the requested XOR-swizzled layout; after a
// barrier they read the image back through the same swizzle and store it
// compact and unswizzled.
#include "common.h"
#include "launch.h"

namespace bmm {
namespace {

constexpr int kBoxThreads = 256;

// Swizzle of an LDS byte offset: mode s in 1..3 XORs the 16-byte chunk bits
// [4, 4+s) with the 128-byte row bits [7, 7+s); mode 0 is the identity. Each
// offset stays inside its own 128-byte row, and the map is an involution.
__device__ __forceinline__ uint32_t swizzle_offset(uint32_t off, int mode) {
  const uint32_t mask = (1u << mode) - 1u;
  return off ^ (((off >> 7) & mask) << 4);
}

struct BoxParams {
  int32_t rank, eb, swizzle, pad;
  int64_t dims[5], strides[5], coords[5], step[5];
  int32_t box[5];
  int32_t box_elems;
};

template <typename T>
__device__ __forceinline__ void copy_in(const char* src, char* lds, const BoxParams& p,
                                        int64_t t) {
  for (int32_t e = threadIdx.x; e < p.box_elems; e += kBoxThreads) {
    int32_t rem = e;
    bool inside = true;
    int64_t off = 0;
    for (int d = p.rank - 1; d >= 0; --d) {
      const int32_t j = rem % p.box[d];
      rem /= p.box[d];
      const int64_t g = p.coords[d] + t * p.step[d] + j;
      inside = inside && g >= 0 && g < p.dims[d];
      off += g * p.strides[d];
    }
    const T v = inside ? *reinterpret_cast<const T*>(src + off) : T(0);
    *reinterpret_cast<T*>(lds + swizzle_offset(uint32_t(e) * sizeof(T), p.swizzle)) = v;
  }
}

template <typename T>
__device__ __forceinline__ void copy_out(char* dst, const char* lds, const BoxParams& p,
                                         int64_t t) {
  T* out = reinterpret_cast<T*>(dst) + t * p.box_elems;
  for (int32_t e = threadIdx.x; e < p.box_elems; e += kBoxThreads)
    out[e] = *reinterpret_cast<const T*>(lds + swizzle_offset(uint32_t(e) * sizeof(T), p.swizzle));
}

__global__ __launch_bounds__(kBoxThreads) void box_kernel(char* __restrict__ dst,
                                                          const char* __restrict__ src,
                                                          BoxParams p) {
  extern __shared__ __attribute__((aligned(128))) char lds[];
  const int64_t t = blockIdx.x;
  switch (p.eb) {
    case 1: copy_in<uint8_t>(src, lds, p, t); break;
    case 2: copy_in<uint16_t>(src, lds, p, t); break;
    case 4: copy_in<uint32_t>(src, lds, p, t); break;
    default: copy_in<uint64_t>(src, lds, p, t); break;
  }
  __syncthreads();
  switch (p.eb) {
    case 1: copy_out<uint8_t>(dst, lds, p, t); break;
    case 2: copy_out<uint16_t>(dst, lds, p, t); break;
    case 4: copy_out<uint32_t>(dst, lds, p, t); break;
    default: copy_out<uint64_t>(dst, lds, p, t); break;
  }
}

// ---- store and add reduction: compact image -> LDS image -> global box ----
// The direction of the cp.async.bulk.tensor page's "Stores, reductions, and
// completion": the same box contract, global destination first. One
// workgroup takes one repeat: it stages the repeat's compact image into LDS
// (swizzled as requested; coalesced reads), then writes every element whose
// global coordinate lies inside the tensor, plain or added to what is there.
// Within one launch no two lanes touch the same global element: the host
// checks that the view does not overlap itself and launches repeats that
// overlap one another in separate, stream-ordered launches.

// f32 -> bf16 bits, round to nearest even (NaN kept quiet, overflow to inf).
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  return uint16_t((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float bf16_value(uint16_t h) {
  return __builtin_bit_cast(float, uint32_t(h) << 16);
}

// One rounding per add: f16 and bf16 sums are formed in f32 and rounded once
// more to the 16-bit format; f32 has at least 2p+2 significand bits for both
// formats, so the two roundings give the correctly rounded sum.
template <int ET>
__device__ __forceinline__ void add_elem(char* g, const char* v) {
  if constexpr (ET == BMM_ELEM_F32) {
    float* x = reinterpret_cast<float*>(g);
    *x = *x + *reinterpret_cast<const float*>(v);
  } else if constexpr (ET == BMM_ELEM_F16) {
    _Float16* x = reinterpret_cast<_Float16*>(g);
    *x = _Float16(float(*x) + float(*reinterpret_cast<const _Float16*>(v)));
  } else if constexpr (ET == BMM_ELEM_BF16) {
    uint16_t* x = reinterpret_cast<uint16_t*>(g);
    *x = bf16_rne(bf16_value(*x) + bf16_value(*reinterpret_cast<const uint16_t*>(v)));
  } else if constexpr (ET == BMM_ELEM_I32) {
    uint32_t* x = reinterpret_cast<uint32_t*>(g);
    *x = *x + *reinterpret_cast<const uint32_t*>(v);
  } else {
    uint64_t* x = reinterpret_cast<uint64_t*>(g);
    *x = *x + *reinterpret_cast<const uint64_t*>(v);
  }
}

// ET = 0: plain store of T-sized elements.
template <typename T, int ET>
__global__ __launch_bounds__(kBoxThreads) void box_store_kernel(char* __restrict__ dst,
                                                                const char* __restrict__ img,
                                                                BoxParams p, int64_t t0) {
  extern __shared__ __attribute__((aligned(128))) char lds[];
  const int64_t t = t0 + blockIdx.x;
  const T* in = reinterpret_cast<const T*>(img) + t * p.box_elems;
  for (int32_t e = threadIdx.x; e < p.box_elems; e += kBoxThreads)
    *reinterpret_cast<T*>(lds + swizzle_offset(uint32_t(e) * sizeof(T), p.swizzle)) = in[e];
  __syncthreads();
  for (int32_t e = threadIdx.x; e < p.box_elems; e += kBoxThreads) {
    int32_t rem = e;
    bool inside = true;
    int64_t off = 0;
    for (int d = p.rank - 1; d >= 0; --d) {
      const int32_t j = rem % p.box[d];
      rem /= p.box[d];
      const int64_t g = p.coords[d] + t * p.step[d] + j;
      inside = inside && g >= 0 && g < p.dims[d];
      off += g * p.strides[d];
    }
    if (!inside) continue;
    const char* v = lds + swizzle_offset(uint32_t(e) * sizeof(T), p.swizzle);
    if constexpr (ET == 0)
      *reinterpret_cast<T*>(dst + off) = *reinterpret_cast<const T*>(v);
    else
      add_elem<ET>(dst + off, v);
  }
}

BoxParams box_params(const bmm_box_desc& d) {
  BoxParams p{};
  p.rank = d.rank;
  p.eb = d.elem_bytes;
  p.swizzle = d.swizzle;
  int64_t elems = 1;
  for (int i = 0; i < d.rank; ++i) {
    p.dims[i] = d.dims[i];
    p.strides[i] = d.strides[i];
    p.coords[i] = d.coords[i];
    p.step[i] = d.coord_step[i];
    p.box[i] = d.box[i];
    elems *= d.box[i];
  }
  p.box_elems = int32_t(elems);
  return p;
}

}  // namespace

hipError_t launch_box_store(void* dst, const void* img, const bmm_box_desc& d, int elem_type,
                            bool repeats_disjoint, hipStream_t s) {
  const BoxParams p = box_params(d);
  const size_t lds_bytes = size_t((int64_t(p.box_elems) * d.elem_bytes + 127) / 128 * 128);
  void (*kern)(char*, const char*, BoxParams, int64_t) = nullptr;
  switch (elem_type) {
    case BMM_ELEM_F32: kern = box_store_kernel<float, BMM_ELEM_F32>; break;
    case BMM_ELEM_F16: kern = box_store_kernel<uint16_t, BMM_ELEM_F16>; break;
    case BMM_ELEM_BF16: kern = box_store_kernel<uint16_t, BMM_ELEM_BF16>; break;
    case BMM_ELEM_I32: kern = box_store_kernel<uint32_t, BMM_ELEM_I32>; break;
    case BMM_ELEM_I64: kern = box_store_kernel<uint64_t, BMM_ELEM_I64>; break;
    default:
      switch (d.elem_bytes) {
        case 1: kern = box_store_kernel<uint8_t, 0>; break;
        case 2: kern = box_store_kernel<uint16_t, 0>; break;
        case 4: kern = box_store_kernel<uint32_t, 0>; break;
        default: kern = box_store_kernel<uint64_t, 0>; break;
      }
  }
  char* out = static_cast<char*>(dst);
  const char* in = static_cast<const char*>(img);
  if (repeats_disjoint) {
    hipLaunchKernelGGL(kern, dim3(unsigned(d.n_repeat)), dim3(kBoxThreads), lds_bytes, s, out, in,
                       p, int64_t(0));
    return hipGetLastError();
  }
  // overlapping repeats: one launch each, in repeat order
  for (int64_t t = 0; t < d.n_repeat; ++t) {
    hipLaunchKernelGGL(kern, dim3(1), dim3(kBoxThreads), lds_bytes, s, out, in, p, t);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_box(void* dst, const void* src, const bmm_box_desc& d, hipStream_t s) {
  const BoxParams p = box_params(d);
  const int64_t elems = p.box_elems;
  // The swizzle keeps every offset inside its 128-byte row: round the image up.
  const size_t lds_bytes = size_t((elems * d.elem_bytes + 127) / 128 * 128);
  hipLaunchKernelGGL(box_kernel, dim3(unsigned(d.n_repeat)), dim3(kBoxThreads), lds_bytes, s,
                     static_cast<char*>(dst), static_cast<const char*>(src), p);
  return hipGetLastError();
}

}  // namespace bmm
