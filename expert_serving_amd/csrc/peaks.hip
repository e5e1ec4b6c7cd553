// Measured ceilings of the GPU the library runs on: sustained bf16 MFMA rate
// (16x16x32 and 32x32x16 forms, 1-2 waves per SIMD), LDS read bandwidth, and
// HBM read and copy bandwidth.  Standalone program: moe_peaks.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#define CK(x)                                                              \
  do {                                                                     \
    hipError_t e_ = (x);                                                   \
    if (e_ != hipSuccess) {                                                \
      printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      exit(1);                                                             \
    }                                                                      \
  } while (0)

// CH independent accumulator chains per wave
template <int CH>
__global__ __launch_bounds__(256) void k_mfma16(float* out, int iters) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(threadIdx.x * 0.001f + i);
    b[i] = (__bf16)(i * 0.5f);
  }
  f32x4 c[CH];
  for (int j = 0; j < CH; ++j) c[j] = f32x4{0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < CH; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
  }
  float s = 0;
  for (int j = 0; j < CH; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

template <int CH>
__global__ __launch_bounds__(256) void k_mfma32(float* out, int iters) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(threadIdx.x * 0.001f + i);
    b[i] = (__bf16)(i * 0.5f);
  }
  f32x16 c[CH];
  for (int j = 0; j < CH; ++j)
    for (int q = 0; q < 16; ++q) c[j][q] = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < CH; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
  }
  float s = 0;
  for (int j = 0; j < CH; ++j)
    for (int q = 0; q < 16; ++q) s += c[j][q];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// 16-byte LDS reads from a 32 KiB buffer; the address changes every iteration
__global__ __launch_bounds__(256) void k_lds(unsigned* out, int iters) {
  __shared__ __attribute__((aligned(16))) unsigned lds[8192];
  for (int i = threadIdx.x; i < 8192; i += 256) lds[i] = i * 2654435761u;
  __syncthreads();
  u32x4 acc = {0, 0, 0, 0};
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int idx = ((w * 8 + j) * 64 + lane + it * 64) & 2047;
      acc ^= *reinterpret_cast<const u32x4*>(lds + idx * 4);
    }
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// n is a multiple of 4 * gridDim.x * 256
__global__ __launch_bounds__(256) void k_copy4(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                               long n) {
  const long stride = (long)gridDim.x * blockDim.x * 4;
  for (long i = (long)blockIdx.x * blockDim.x * 4 + threadIdx.x; i < n; i += stride) {
    const u32x4 v0 = src[i], v1 = src[i + 256], v2 = src[i + 512], v3 = src[i + 768];
    dst[i] = v0;
    dst[i + 256] = v1;
    dst[i + 512] = v2;
    dst[i + 768] = v3;
  }
}

__global__ __launch_bounds__(256) void k_read4(const u32x4* __restrict__ src, unsigned* out, long n) {
  const long stride = (long)gridDim.x * blockDim.x * 4;
  u32x4 acc = {0, 0, 0, 0};
  for (long i = (long)blockIdx.x * blockDim.x * 4 + threadIdx.x; i < n; i += stride)
    acc ^= src[i] ^ src[i + 256] ^ src[i + 512] ^ src[i + 768];
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

template <typename F>
static float time_ms(F f) {
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  f();
  CK(hipEventRecord(e0));
  f();
  CK(hipEventRecord(e1));
  CK(hipEventSynchronize(e1));
  float ms;
  CK(hipEventElapsedTime(&ms, e0, e1));
  CK(hipEventDestroy(e0));
  CK(hipEventDestroy(e1));
  return ms;
}

int main() {
  hipDeviceProp_t p;
  CK(hipGetDeviceProperties(&p, 0));
  const int CUs = p.multiProcessorCount;
  printf("device %s, %d CUs, peak clock %d MHz, LDS per block %zu KiB\n", p.gcnArchName, CUs,
         p.clockRate / 1000, p.sharedMemPerBlock / 1024);
  float* o;
  CK(hipMalloc(&o, (size_t)CUs * 4 * 256 * sizeof(float)));
  const int iters = 20000;
  for (int bpc : {1, 2}) {
    const int grid = CUs * bpc;
    float ms = time_ms([&] { hipLaunchKernelGGL(k_mfma16<16>, dim3(grid), dim3(256), 0, 0, o, iters / 2); });
    printf("mfma bf16 16x16x32, %d wave(s)/SIMD, 16 chains: %.1f TFLOP/s\n", bpc,
           (double)grid * 4 * (iters / 2) * 16 * 16384.0 / ms / 1e9);
    ms = time_ms([&] { hipLaunchKernelGGL(k_mfma32<4>, dim3(grid), dim3(256), 0, 0, o, iters); });
    printf("mfma bf16 32x32x16, %d wave(s)/SIMD,  4 chains: %.1f TFLOP/s\n", bpc,
           (double)grid * 4 * iters * 4 * 32768.0 / ms / 1e9);
  }
  for (int bpc : {1, 4}) {
    const int grid = CUs * bpc;
    unsigned* ou;
    CK(hipMalloc(&ou, (size_t)grid * 256 * 4));
    const float ms = time_ms([&] { hipLaunchKernelGGL(k_lds, dim3(grid), dim3(256), 0, 0, ou, iters); });
    const double bytes = (double)grid * 256 * iters * 8 * 16.0;
    printf("lds 16-byte reads, %d block(s)/CU: %.0f bytes/clk/CU at the peak clock\n", bpc,
           bytes / (ms * 1e-3) / CUs / (p.clockRate * 1e3));
    CK(hipFree(ou));
  }
  const long n = (4L << 30) / 16;
  u32x4 *a, *b;
  CK(hipMalloc(&a, n * 16));
  CK(hipMalloc(&b, n * 16));
  CK(hipMemset(a, 1, n * 16));
  unsigned* ou;
  CK(hipMalloc(&ou, (size_t)CUs * 8 * 256 * 4));
  const int g = CUs * 8;
  float ms = time_ms([&] { hipLaunchKernelGGL(k_read4, dim3(g), dim3(256), 0, 0, a, ou, n); });
  printf("hbm read 4 GiB: %.0f GB/s\n", 1.0 * n * 16 / ms / 1e6);
  ms = time_ms([&] { hipLaunchKernelGGL(k_copy4, dim3(g), dim3(256), 0, 0, a, b, n); });
  printf("hbm copy 4 GiB: %.0f GB/s (read + write)\n", 2.0 * n * 16 / ms / 1e6);
  CK(hipFree(a));
  CK(hipFree(b));
  CK(hipFree(ou));
  CK(hipFree(o));
  return 0;
}
