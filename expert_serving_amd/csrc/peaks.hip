// Measured ceilings of the GPU the library runs on: sustained bf16 MFMA rate
// (16x16x32 and 32x32x16 forms, 1-2 waves per SIMD), LDS bandwidth (reads,
// the grouped GEMM's read and write shapes, and their mix), vector-memory
// load rate for the GEMM's two tile-row shapes, and HBM read and copy
// bandwidth.  Standalone program: moe_peaks.
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

// 32x32x16 with random operands, a different pair per chain, so consecutive
// MFMAs switch their inputs as a real GEMM's do (the power drawn, and so the
// clock the chip holds, depends on the operand bits)
__device__ __forceinline__ unsigned hash32(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}
__global__ __launch_bounds__(256) void k_mfma32_rand(float* out, int iters) {
  constexpr int CH = 4;
  bf16x8 a[CH], b[CH];
  for (int j = 0; j < CH; ++j)
    for (int i = 0; i < 8; ++i) {
      // bf16 values in about [-2, 2] with random mantissas
      const unsigned ha = hash32((blockIdx.x * 256 + threadIdx.x) * 64 + j * 8 + i);
      const unsigned hb = hash32(ha ^ 0x9e3779b9u);
      a[j][i] = (__bf16)(((int)(ha & 0xFFFF) - 32768) / 16384.0f);
      b[j][i] = (__bf16)(((int)(hb & 0xFFFF) - 32768) / 16384.0f);
    }
  f32x16 c[CH];
  for (int j = 0; j < CH; ++j)
    for (int q = 0; q < 16; ++q) c[j][q] = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < CH; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[j], c[j], 0, 0, 0);
  }
  float s = 0;
  for (int j = 0; j < CH; ++j) s += c[j][0] + c[j][5] + c[j][10] + c[j][15];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// 32x32x16 f16 with random operands (the down projection's form: fp16 h
// times bf16 weights widened to fp16, whose three low mantissa bits are zero
// when BF16W)
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
template <bool BF16W>
__global__ __launch_bounds__(256) void k_mfma32_f16_rand(float* out, int iters) {
  constexpr int CH = 4;
  f16x8 a[CH], b[CH];
  for (int j = 0; j < CH; ++j)
    for (int i = 0; i < 8; ++i) {
      const unsigned ha = hash32((blockIdx.x * 256 + threadIdx.x) * 64 + j * 8 + i);
      const unsigned hb = hash32(ha ^ 0x9e3779b9u);
      a[j][i] = (_Float16)(((int)(ha & 0xFFFF) - 32768) / 16384.0f);
      float bw = ((int)(hb & 0xFFFF) - 32768) / 16384.0f;
      if (BF16W) bw = __uint_as_float(__float_as_uint(bw) & 0xFFFF0000u);
      b[j][i] = (_Float16)bw;
    }
  f32x16 c[CH];
  for (int j = 0; j < CH; ++j)
    for (int q = 0; q < 16; ++q) c[j][q] = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < CH; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[j], b[j], c[j], 0, 0, 0);
  }
  float s = 0;
  for (int j = 0; j < CH; ++j) s += c[j][0] + c[j][5] + c[j][10] + c[j][15];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands and E8M0 block scales
// (the MXFP8 GEMM's instruction), CH independent chains; RAND: random codes
// (exponent field kept below 8, so no NaN) and random scales near 2^0, a
// different operand pair per chain
typedef int i32x8 __attribute__((ext_vector_type(8)));
template <bool RAND>
__global__ __launch_bounds__(256) void k_mfma_fp8(float* out, int iters) {
  constexpr int CH = 4;
  i32x8 a[CH], b[CH];
  int sa[CH], sb[CH];
  for (int j = 0; j < CH; ++j) {
    for (int i = 0; i < 8; ++i) {
      const unsigned ha = hash32((blockIdx.x * 256 + threadIdx.x) * 64 + j * 8 + i);
      const unsigned hb = hash32(ha ^ 0x9e3779b9u);
      a[j][i] = RAND ? (int)(ha & 0xBFBFBFBFu) : 0x38383838;
      b[j][i] = RAND ? (int)(hb & 0xBFBFBFBFu) : 0x30303030;
    }
    sa[j] = RAND ? 120 + (int)(hash32(j + 77 * threadIdx.x) & 7) : 127;
    sb[j] = RAND ? 120 + (int)(hash32(j + 91 * threadIdx.x) & 7) : 127;
  }
  f32x16 c[CH];
  for (int j = 0; j < CH; ++j)
    for (int q = 0; q < 16; ++q) c[j][q] = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < CH; ++j)
      c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[j], b[j], c[j], 0, 0, 0, sa[j], 0, sb[j]);
  }
  float s = 0;
  for (int j = 0; j < CH; ++j) s += c[j][0] + c[j][5] + c[j][10] + c[j][15];
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

// LDS traffic in the grouped GEMM's shapes, timed in shader clocks
// (s_memtime): 16-byte reads of 16 rows x 1 chunk per 16 lanes, 16-byte writes
// of 2 rows x 8 chunks, on 128-byte rows with chunk c of row r at
// c ^ ((r >> 1) & 7).  MODE 0: reads, 1: writes, 2: three reads per write.
template <int MODE>
__global__ __launch_bounds__(512) void k_lds_shapes(unsigned long long* cyc, unsigned* out, int iters) {
  extern __shared__ __attribute__((aligned(16))) unsigned short sm[];  // 512 rows x 64 elements
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 512 * 64 / 8; i += blockDim.x)
    reinterpret_cast<u32x4*>(sm)[i] = u32x4{1u, 2u, 3u, (unsigned)i};
  __syncthreads();
  u32x4 acc = {0, 0, 0, 0};
  const int fr = lane & 31, fk = lane >> 5;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (MODE == 0 || (MODE == 2 && (j & 3) != 3)) {
        const int r = ((wave * 8 + j) * 32 + fr + it * 64) & 511;
        const int c = (j * 2 + fk) & 7;
        acc ^= *reinterpret_cast<const u32x4*>(sm + r * 64 + ((c ^ ((r >> 1) & 7)) << 3));
      } else {
        const int r = ((wave * 8 + j) * 8 + (lane >> 3) + it * 64) & 511;
        const int c = lane & 7;
        *reinterpret_cast<u32x4*>(sm + r * 64 + ((c ^ ((r >> 1) & 7)) << 3)) =
            u32x4{(unsigned)it, 0u, 0u, (unsigned)j};
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) cyc[blockIdx.x] = t1 - t0;
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

// LDS fragment reads (as k_lds_shapes) alongside direct-to-LDS loads
// (global_load_lds_dwordx4, 8 rows x 128 bytes per wavefront load, from a
// 1 MiB L2-resident buffer) into a second 64 KiB region: 3 reads per load.
__global__ __launch_bounds__(512) void k_lds_with_dma(const u32x4* __restrict__ src,
                                                      unsigned long long* cyc, unsigned* out,
                                                      int iters) {
  extern __shared__ __attribute__((aligned(16))) unsigned short sm[];  // 2 x 512 rows x 64 elements
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 512 * 64 / 8; i += blockDim.x)
    reinterpret_cast<u32x4*>(sm)[i] = u32x4{1u, 2u, 3u, (unsigned)i};
  __syncthreads();
  u32x4 acc = {0, 0, 0, 0};
  const int fr = lane & 31, fk = lane >> 5;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int r = ((wave * 8 + j) * 32 + fr + it * 64) & 511;
      const int c = (j * 2 + fk) & 7;
      acc ^= *reinterpret_cast<const u32x4*>(sm + r * 64 + ((c ^ ((r >> 1) & 7)) << 3));
    }
    const int row = (wave * 8 + (lane >> 3) + it * 64) & 8191;
    unsigned short* dst = sm + 32768 + ((wave + 8 * it) & 63) * 512;
    __builtin_amdgcn_global_load_lds((gbl_ptr_t)(src + (size_t)row * 8 + (lane & 7)), (lds_ptr_t)dst,
                                     16, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) cyc[blockIdx.x] = t1 - t0;
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// Vector-memory load rate for 1 KiB-per-wavefront loads shaped as the GEMM's
// tile rows: LPR lanes per row, i.e. 16 rows x 64 bytes (LPR 4) or 8 rows x
// 128 bytes (LPR 8); rows 8 KiB apart in a 16 MiB (L2/MALL-resident) buffer.
template <int LPR>
__global__ __launch_bounds__(512) void k_rows(const u32x4* __restrict__ buf, unsigned* out, int iters) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane / LPR, chunk = lane % LPR;
  constexpr int kRowsPerLoad = 64 / LPR;
  u32x4 acc = {0, 0, 0, 0};
  int r0 = (blockIdx.x * 8 + wave) * 7;
  for (int it = 0; it < iters; ++it) {
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = (r0 + j * kRowsPerLoad + row) & 2047;
      v[j] = buf[(size_t)r * 512 + ((it * LPR + chunk) & 511)];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j];
    r0 += 8 * kRowsPerLoad;
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
    ms = time_ms([&] { hipLaunchKernelGGL(k_mfma32_rand, dim3(grid), dim3(256), 0, 0, o, iters); });
    printf("mfma bf16 32x32x16, %d wave(s)/SIMD,  4 chains, random operands: %.1f TFLOP/s\n", bpc,
           (double)grid * 4 * iters * 4 * 32768.0 / ms / 1e9);
    ms = time_ms([&] { hipLaunchKernelGGL(k_mfma32_f16_rand<false>, dim3(grid), dim3(256), 0, 0, o, iters); });
    printf("mfma f16 32x32x16, %d wave(s)/SIMD,  4 chains, random operands: %.1f TFLOP/s\n", bpc,
           (double)grid * 4 * iters * 4 * 32768.0 / ms / 1e9);
    ms = time_ms([&] { hipLaunchKernelGGL(k_mfma32_f16_rand<true>, dim3(grid), dim3(256), 0, 0, o, iters); });
    printf("mfma f16 32x32x16, %d wave(s)/SIMD,  4 chains, random fp16 x bf16-valued operands: %.1f TFLOP/s\n",
           bpc, (double)grid * 4 * iters * 4 * 32768.0 / ms / 1e9);
    ms = time_ms([&] { hipLaunchKernelGGL(k_mfma_fp8<false>, dim3(grid), dim3(256), 0, 0, o, iters / 2); });
    printf("mfma scaled fp8 32x32x64, %d wave(s)/SIMD,  4 chains: %.1f TFLOP/s\n", bpc,
           (double)grid * 4 * (iters / 2) * 4 * 131072.0 / ms / 1e9);
    ms = time_ms([&] { hipLaunchKernelGGL(k_mfma_fp8<true>, dim3(grid), dim3(256), 0, 0, o, iters / 2); });
    printf("mfma scaled fp8 32x32x64, %d wave(s)/SIMD,  4 chains, random operands: %.1f TFLOP/s\n", bpc,
           (double)grid * 4 * (iters / 2) * 4 * 131072.0 / ms / 1e9);
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
  {
    unsigned long long* cyc;
    unsigned* ou;
    CK(hipMalloc(&cyc, (size_t)CUs * sizeof(unsigned long long)));
    CK(hipMalloc(&ou, (size_t)CUs * 512 * 4));
    const int it_lds = 4000;
    for (int mode = 0; mode < 3; ++mode) {
      auto kern = mode == 0 ? k_lds_shapes<0> : (mode == 1 ? k_lds_shapes<1> : k_lds_shapes<2>);
      CK(hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                             hipFuncAttributeMaxDynamicSharedMemorySize, 65536));
      hipLaunchKernelGGL(kern, dim3(CUs), dim3(512), 65536, 0, cyc, ou, it_lds);
      CK(hipDeviceSynchronize());
      unsigned long long* h = (unsigned long long*)malloc((size_t)CUs * sizeof(unsigned long long));
      CK(hipMemcpy(h, cyc, (size_t)CUs * sizeof(unsigned long long), hipMemcpyDeviceToHost));
      double avg = 0;
      for (int i = 0; i < CUs; ++i) avg += (double)h[i];
      avg /= CUs;
      free(h);
      printf("lds %s, 8 waves/CU: %.0f bytes/clk/CU (shader clocks)\n",
             mode == 0 ? "GEMM fragment reads  " : (mode == 1 ? "GEMM row writes      " : "3 reads : 1 write mix"),
             512.0 * it_lds * 8 * 16 / avg);
    }
    {
      u32x4* src;
      CK(hipMalloc(&src, 1 << 20));
      CK(hipMemset(src, 1, 1 << 20));
      CK(hipFuncSetAttribute(reinterpret_cast<const void*>(k_lds_with_dma),
                             hipFuncAttributeMaxDynamicSharedMemorySize, 131072));
      hipLaunchKernelGGL(k_lds_with_dma, dim3(CUs), dim3(512), 131072, 0, src, cyc, ou, it_lds);
      CK(hipDeviceSynchronize());
      unsigned long long* h = (unsigned long long*)malloc((size_t)CUs * sizeof(unsigned long long));
      CK(hipMemcpy(h, cyc, (size_t)CUs * sizeof(unsigned long long), hipMemcpyDeviceToHost));
      double avg = 0;
      for (int i = 0; i < CUs; ++i) avg += (double)h[i];
      avg /= CUs;
      free(h);
      printf("lds 3 reads : 1 direct-to-LDS load, 8 waves/CU: %.0f bytes/clk/CU (shader clocks)\n",
             512.0 * it_lds * 4 * 16 / avg);
      CK(hipFree(src));
    }
    u32x4* buf;
    CK(hipMalloc(&buf, 16 << 20));
    CK(hipMemset(buf, 1, 16 << 20));
    const int it_rows = 2000;
    for (int lpr : {4, 8}) {
      const float ms = time_ms([&] {
        if (lpr == 4) hipLaunchKernelGGL(k_rows<4>, dim3(CUs), dim3(512), 0, 0, buf, ou, it_rows);
        else hipLaunchKernelGGL(k_rows<8>, dim3(CUs), dim3(512), 0, 0, buf, ou, it_rows);
      });
      const double bytes = (double)CUs * 512 * it_rows * 8 * 16.0;
      printf("vector-memory loads, %2d rows x %3d bytes per wavefront load: %.0f bytes/clk/CU at the peak clock\n",
             64 / lpr, lpr * 16, bytes / (ms * 1e-3) / CUs / (p.clockRate * 1e3));
    }
    CK(hipFree(buf));
    CK(hipFree(ou));
    CK(hipFree(cyc));
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
