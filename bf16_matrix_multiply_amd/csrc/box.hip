// Box transfers through an LDS image. The load: the role of the TMA tile-mode box load of the
// cp.async.bulk.tensor page ("Operands and descriptor fields", "Example: two
// explicit 8x16 boxes"), done the CDNA4 way. One workgroup stages one repeat:
// its lanes read the box from global memory with consecutive lanes on
// consecutive innermost elements (coalesced), substitute zero outside the
// tensor, and write the LDS image in the requested XOR-swizzled layout; after a
// barrier they read the image back through the same swizzle and store it
// compact and unswizzled.
//
// Two paths. When every 16-byte chunk of the box is aligned and wholly inside
// or outside the tensor (box_chunk_path), each lane moves whole chunks, the
// swizzle permutes chunks, and the workgroup is sized to the box (up to 1024
// lanes, at most four chunks each: one round of loads in flight). Otherwise
// 256 lanes move one element at a time. Since the exported image is the
// unswizzled one, in both paths a lane reads back exactly the LDS slots it
// wrote; the swizzled image is the layout a consumer in the same workgroup
// would read.
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
  // 16-byte path (see box_chunk_path): chunks in the box, chunks per
  // innermost box row, elements per chunk
  int32_t box_chunks, inner_chunks, vlen, vec;
};

constexpr int kChunkUnroll = 4;        // 16-byte chunks a lane has in flight
constexpr int kChunkThreadsMax = 1024;  // 16-byte path: lanes per workgroup at most

// 16-byte path workgroup size: enough lanes that each has at most
// kChunkUnroll chunks of its box (one round of loads in flight), in whole
// wavefronts. A 64 KB box takes 1024 lanes; two such workgroups fill a CU's LDS.
inline int chunk_threads(int32_t box_chunks) {
  const int32_t per = (box_chunks + kChunkUnroll - 1) / kChunkUnroll;
  const int32_t t = (per + 63) / 64 * 64;
  return t < 64 ? 64 : (t > kChunkThreadsMax ? kChunkThreadsMax : t);
}

// Global byte offset of 16-byte chunk c of repeat t, and whether it lies
// inside the tensor (with the 16-byte path a chunk is wholly inside or
// wholly outside: see box_chunk_path).
__device__ __forceinline__ int64_t chunk_offset(const BoxParams& p, int64_t t, int32_t c,
                                                bool& inside) {
  const int in = p.rank - 1;
  int32_t row = c / p.inner_chunks;
  const int64_t gi = p.coords[in] + t * p.step[in] + int64_t(c - row * p.inner_chunks) * p.vlen;
  inside = gi >= 0 && gi < p.dims[in];
  int64_t off = gi * p.eb;
  for (int d = in - 1; d >= 0; --d) {
    const int32_t j = row % p.box[d];
    row /= p.box[d];
    const int64_t g = p.coords[d] + t * p.step[d] + j;
    inside = inside && g >= 0 && g < p.dims[d];
    off += g * p.strides[d];
  }
  return off;
}

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

// Box load, 16 bytes per lane: chunks read from global memory (zero outside
// the tensor), written to the swizzled LDS image, read back and stored compact.
// One round per lane, as in box_store_kernel_v.
__global__ __launch_bounds__(kChunkThreadsMax) void box_kernel_v(char* __restrict__ dst,
                                                                 const char* __restrict__ src,
                                                                 BoxParams p) {
  extern __shared__ __attribute__((aligned(128))) char lds[];
  const int64_t t = blockIdx.x;
  const int32_t n = p.box_chunks;
  const int32_t nt = blockDim.x;
  u32x4 v[kChunkUnroll];
#pragma unroll
  for (int u = 0; u < kChunkUnroll; ++u) {
    const int32_t c = int32_t(threadIdx.x) + u * nt;
    v[u] = u32x4{0u, 0u, 0u, 0u};
    if (c < n) {
      bool inside;
      const int64_t off = chunk_offset(p, t, c, inside);
      if (inside) v[u] = load16(reinterpret_cast<const uint32_t*>(src + off));
    }
  }
#pragma unroll
  for (int u = 0; u < kChunkUnroll; ++u) {
    const int32_t c = int32_t(threadIdx.x) + u * nt;
    if (c < n)
      *reinterpret_cast<u32x4*>(lds + swizzle_offset(uint32_t(c) * 16, p.swizzle)) = v[u];
  }
  __syncthreads();
  u32x4* out = reinterpret_cast<u32x4*>(dst + t * int64_t(n) * 16);
#pragma unroll
  for (int u = 0; u < kChunkUnroll; ++u) {
    const int32_t c = int32_t(threadIdx.x) + u * nt;
    if (c < n)
      out[c] = *reinterpret_cast<const u32x4*>(lds + swizzle_offset(uint32_t(c) * 16, p.swizzle));
  }
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

// Lane-wise add of a 16-byte chunk with the element semantics of add_elem.
template <int ET>
__device__ __forceinline__ u32x4 add_chunk(u32x4 g, u32x4 v) {
  // Whole-vector operations or scalar copies only: a bit cast applied to an element of an
  // ext_vector_type operand does not reliably read that element.
  u32x4 r = g;
  if constexpr (ET == BMM_ELEM_F32) {
    r = __builtin_bit_cast(u32x4, __builtin_bit_cast(f32x4, g) + __builtin_bit_cast(f32x4, v));
  } else if constexpr (ET == BMM_ELEM_I32) {
    r = g + v;
  } else if constexpr (ET == BMM_ELEM_I64) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint64_t a = uint64_t(g[2 * e]) | (uint64_t(g[2 * e + 1]) << 32);
      const uint64_t b = uint64_t(v[2 * e]) | (uint64_t(v[2 * e + 1]) << 32);
      const uint64_t s = a + b;
      r[2 * e] = uint32_t(s);
      r[2 * e + 1] = uint32_t(s >> 32);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint16_t lo, hi;
      const uint16_t glo = uint16_t(g[e]), ghi = uint16_t(g[e] >> 16);
      const uint16_t vlo = uint16_t(v[e]), vhi = uint16_t(v[e] >> 16);
      if constexpr (ET == BMM_ELEM_F16) {
        lo = __builtin_bit_cast(uint16_t, _Float16(float(__builtin_bit_cast(_Float16, glo)) +
                                                   float(__builtin_bit_cast(_Float16, vlo))));
        hi = __builtin_bit_cast(uint16_t, _Float16(float(__builtin_bit_cast(_Float16, ghi)) +
                                                   float(__builtin_bit_cast(_Float16, vhi))));
      } else {
        lo = bf16_rne(bf16_value(glo) + bf16_value(vlo));
        hi = bf16_rne(bf16_value(ghi) + bf16_value(vhi));
      }
      r[e] = uint32_t(lo) | (uint32_t(hi) << 16);
    }
  }
  return r;
}

// Box store (ET = 0) or add reduction, 16 bytes per lane. A box holds at most
// kChunkThreadsMax * kChunkUnroll chunks (64 KB), so each lane takes one round:
// its image chunks and, for the add, the destination chunks they land on are
// all requested before the barrier, and the adds and stores follow it.
template <int ET>
__global__ __launch_bounds__(kChunkThreadsMax) void box_store_kernel_v(char* __restrict__ dst,
                                                                       const char* __restrict__ img,
                                                                       BoxParams p, int64_t t0) {
  extern __shared__ __attribute__((aligned(128))) char lds[];
  const int64_t t = t0 + blockIdx.x;
  const int32_t n = p.box_chunks;
  const int32_t nt = blockDim.x;
  const u32x4* in = reinterpret_cast<const u32x4*>(img + t * int64_t(n) * 16);
  int64_t off[kChunkUnroll];
  bool ok[kChunkUnroll];
  u32x4 v[kChunkUnroll], g[kChunkUnroll];
#pragma unroll
  for (int u = 0; u < kChunkUnroll; ++u) {
    const int32_t c = int32_t(threadIdx.x) + u * nt;
    ok[u] = false;
    off[u] = 0;
    if (c < n) {
      v[u] = in[c];
      off[u] = chunk_offset(p, t, c, ok[u]);
      if constexpr (ET != 0) {
        if (ok[u]) g[u] = load16(reinterpret_cast<const uint32_t*>(dst + off[u]));
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kChunkUnroll; ++u) {
    const int32_t c = int32_t(threadIdx.x) + u * nt;
    if (c < n)
      *reinterpret_cast<u32x4*>(lds + swizzle_offset(uint32_t(c) * 16, p.swizzle)) = v[u];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kChunkUnroll; ++u) {
    if (!ok[u]) continue;
    const int32_t c = int32_t(threadIdx.x) + u * nt;
    const u32x4 x = *reinterpret_cast<const u32x4*>(lds + swizzle_offset(uint32_t(c) * 16, p.swizzle));
    if constexpr (ET == 0)
      *reinterpret_cast<u32x4*>(dst + off[u]) = x;
    else
      *reinterpret_cast<u32x4*>(dst + off[u]) = add_chunk<ET>(g[u], x);
  }
}

// The 16-byte path applies when every 16-byte chunk of every repeat is
// aligned in global memory and wholly inside or wholly outside the tensor:
// the innermost box row, start coordinate, coordinate step and tensor extent
// are all whole chunks (outer strides and base are 16-byte aligned by
// validation).
bool box_chunk_path(const bmm_box_desc& d) {
  const int in = d.rank - 1;
  const int64_t eb = d.elem_bytes;
  return (d.box[in] * eb) % 16 == 0 && (d.coords[in] * eb) % 16 == 0 &&
         (d.coord_step[in] * eb) % 16 == 0 && (d.dims[in] * eb) % 16 == 0;
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
  p.vec = box_chunk_path(d) ? 1 : 0;
  p.vlen = 16 / d.elem_bytes;
  p.box_chunks = int32_t(elems * d.elem_bytes / 16);
  p.inner_chunks = int32_t(int64_t(d.box[d.rank - 1]) * d.elem_bytes / 16);
  // the 16-byte kernels cover a box in one round of kChunkUnroll chunks per lane
  if (p.box_chunks > kChunkThreadsMax * kChunkUnroll) p.vec = 0;
  return p;
}

}  // namespace

hipError_t launch_box_store(void* dst, const void* img, const bmm_box_desc& d, int elem_type,
                            bool repeats_disjoint, hipStream_t s) {
  const BoxParams p = box_params(d);
  const size_t lds_bytes = size_t((int64_t(p.box_elems) * d.elem_bytes + 127) / 128 * 128);
  void (*kern)(char*, const char*, BoxParams, int64_t) = nullptr;
  if (p.vec) {
    switch (elem_type) {
      case BMM_ELEM_F32: kern = box_store_kernel_v<BMM_ELEM_F32>; break;
      case BMM_ELEM_F16: kern = box_store_kernel_v<BMM_ELEM_F16>; break;
      case BMM_ELEM_BF16: kern = box_store_kernel_v<BMM_ELEM_BF16>; break;
      case BMM_ELEM_I32: kern = box_store_kernel_v<BMM_ELEM_I32>; break;
      case BMM_ELEM_I64: kern = box_store_kernel_v<BMM_ELEM_I64>; break;
      default: kern = box_store_kernel_v<0>; break;
    }
  } else switch (elem_type) {
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
  const unsigned threads = unsigned(p.vec ? chunk_threads(p.box_chunks) : kBoxThreads);
  if (repeats_disjoint) {
    hipLaunchKernelGGL(kern, dim3(unsigned(d.n_repeat)), dim3(threads), lds_bytes, s, out, in, p,
                       int64_t(0));
    return hipGetLastError();
  }
  // overlapping repeats: one launch each, in repeat order
  for (int64_t t = 0; t < d.n_repeat; ++t) {
    hipLaunchKernelGGL(kern, dim3(1), dim3(threads), lds_bytes, s, out, in, p, t);
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
  const unsigned threads = unsigned(p.vec ? chunk_threads(p.box_chunks) : kBoxThreads);
  hipLaunchKernelGGL(p.vec ? box_kernel_v : box_kernel, dim3(unsigned(d.n_repeat)),
                     dim3(threads), lds_bytes, s, static_cast<char*>(dst),
                     static_cast<const char*>(src), p);
  return hipGetLastError();
}

}  // namespace bmm
