// Chip probes behind the kernel design choices (MI355X, gfx950):
//   1. MFMA issue rate: v_mfma_f32_16x16x32_bf16 vs v_mfma_f32_32x32x16_bf16,
//      one / two / four waves per SIMD, operands with few toggling bits (small
//      integers) vs full-entropy bf16 values; reports TFLOP/s and the shader
//      clock measured in-kernel (s_memtime against the 100 MHz s_memrealtime).
//   2. LDS read rate of ds_read_b128 for the access patterns the kernels use.
// Every access stays inside its buffer; every kernel runs a fixed trip count.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

#define CHECK(x)                                                              \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));            \
      std::exit(1);                                                           \
    }                                                                         \
  } while (0)

__device__ bf16x8 operand(int tid, int salt, bool random) {
  bf16x8 v;
  for (int i = 0; i < 8; ++i) {
    uint32_t h = (uint32_t(tid) * 2654435761u) ^ (uint32_t(i + salt) * 40503u) ^
                 (uint32_t(blockIdx.x) * 97u);
    h ^= h >> 13;
    h *= 0x5bd1e995u;
    h ^= h >> 15;
    const float r = float(int(h & 0xffff)) / 32768.0f - 1.0f;
    v[i] = __bf16(random ? r : float((tid + i + salt) & 3));
  }
  return v;
}

// SHAPE 16: 16 accumulators of 4 floats; SHAPE 32: 16 accumulators of 16.
template <int SHAPE>
__global__ __launch_bounds__(256) void mfma_rate(f32x4* out, unsigned long long* clk, int iters,
                                                 int random) {
  const int tid = threadIdx.x;
  const bf16x8 a = operand(tid, 0, random != 0), b = operand(tid, 3, random != 0);
  unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  f32x4 res = {0.f, 0.f, 0.f, 0.f};
  if constexpr (SHAPE == 16) {
    f32x4 acc[16];
    for (int i = 0; i < 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
    for (int i = 0; i < 16; ++i) res += acc[i];
  } else {
    f32x16 acc[8];
    for (int i = 0; i < 8; ++i) acc[i] = f32x16{};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
    for (int i = 0; i < 8; ++i) res += f32x4{acc[i][0], acc[i][5], acc[i][10], acc[i][15]};
  }
  unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  out[blockIdx.x * 256 + tid] = res;
  if (blockIdx.x == 0 && tid == 0) {
    clk[0] = t1 - t0;
    clk[1] = r1 - r0;
  }
}

// LDS read patterns (byte offset of lane l in a 1 KB fragment):
//   0 contiguous: 16 l
//   1 16x16 fragment, plain atoms: (g/2)*512 + m*32 + (g%2)*16, m = l%16, g = l/16
//   2 16x16 fragment, halves XOR-swapped by row bits 2 and 3
__global__ __launch_bounds__(256) void lds_rate(u32x4* out, int iters, int pattern) {
  __shared__ u32x4 buf[4096];  // 64 KB
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < 4096; i += 256) buf[i] = u32x4{uint32_t(i), 1u, 2u, 3u};
  __syncthreads();
  const int m = lane & 15, g = lane >> 4;
  int off = lane * 16;
  if (pattern == 1) off = (g >> 1) * 512 + m * 32 + 16 * (g & 1);
  if (pattern == 2) off = (g >> 1) * 512 + m * 32 + 16 * ((g & 1) ^ (((m >> 2) ^ (m >> 3)) & 1));
  // wave base 16 KB apart (mod 48 KB), 8 fragments 2 KB apart: max offset < 48 KB + 16 KB
  const __attribute__((address_space(3))) char* base =
      (const __attribute__((address_space(3))) char*)buf + off + (w * 16384) % 49152;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= *(const volatile lds_u32x4*)(base + j * 2048);
  out[blockIdx.x * 256 + tid] = acc;
}

static int cus() {
  hipDeviceProp_t p;
  CHECK(hipGetDeviceProperties(&p, 0));
  return p.multiProcessorCount;
}

template <int SHAPE>
static void run_mfma(int waves_per_simd, int random) {
  const int blocks = cus() * waves_per_simd;  // 4 waves per block = one per SIMD
  const int iters = SHAPE == 16 ? 20000 : 20000;
  f32x4* d;
  unsigned long long* c;
  CHECK(hipMalloc(&d, size_t(blocks) * 256 * sizeof(f32x4)));
  CHECK(hipMalloc(&c, 2 * sizeof(unsigned long long)));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  hipLaunchKernelGGL(mfma_rate<SHAPE>, dim3(blocks), dim3(256), 0, 0, d, c, 100, random);
  CHECK(hipEventRecord(e0));
  hipLaunchKernelGGL(mfma_rate<SHAPE>, dim3(blocks), dim3(256), 0, 0, d, c, iters, random);
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  float ms;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  unsigned long long h[2];
  CHECK(hipMemcpy(h, c, sizeof h, hipMemcpyDeviceToHost));
  const double per_wave_flops = double(iters) * (SHAPE == 16 ? 16 * 16384.0 : 8 * 32768.0);
  const double flops = double(blocks) * 4 * per_wave_flops;
  const double ghz = double(h[0]) / (double(h[1]) / 100e6) / 1e9;
  const int ops_per_iter = SHAPE == 16 ? 16 : 8;
  std::printf("mfma %-9s waves/SIMD=%d %-6s %8.1f TFLOP/s  clock %.3f GHz  %5.1f cycles per op per wave\n",
              SHAPE == 16 ? "16x16x32" : "32x32x16", waves_per_simd, random ? "random" : "small",
              flops / ms / 1e9, ghz, double(h[0]) / (double(iters) * ops_per_iter));
  CHECK(hipFree(d));
  CHECK(hipFree(c));
}

static void run_lds(int pattern) {
  const int blocks = cus() * 2, iters = 4096;
  u32x4* d;
  CHECK(hipMalloc(&d, size_t(blocks) * 256 * sizeof(u32x4)));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  hipLaunchKernelGGL(lds_rate, dim3(blocks), dim3(256), 0, 0, d, 16, pattern);
  CHECK(hipEventRecord(e0));
  hipLaunchKernelGGL(lds_rate, dim3(blocks), dim3(256), 0, 0, d, iters, pattern);
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  float ms;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  const double bytes = double(blocks) * 256 * 16 * 8 * iters;
  const char* names[] = {"contiguous", "16x16 fragment, plain atoms", "16x16 fragment, XOR half-swap"};
  std::printf("lds ds_read_b128 %-30s %8.1f GB/s chip  %6.1f B per CU per 2.2 GHz clock\n",
              names[pattern], bytes / ms / 1e6, bytes / (ms * 1e-3) / cus() / 2.2e9);
  CHECK(hipFree(d));
}

int main() {
  std::printf("compute units: %d\n", cus());
  for (int random = 0; random < 2; ++random)
    for (int w : {1, 2}) {
      run_mfma<16>(w, random);
      run_mfma<32>(w, random);
    }
  for (int pat = 0; pat < 3; ++pat) run_lds(pat);
  return 0;
}
