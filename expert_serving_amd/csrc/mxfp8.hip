// MXFP8 quantisation of bf16 / fp32 rows for the 8-bit expert path.
//
// Format: OCP Microscaling Formats v1.0, MXFP8 with E4M3 elements -- blocks
// of 32 consecutive elements of a row share one E8M0 scale 2^s with
// s = floor(log2 amax) - 8 (8 being the exponent of E4M3's largest binade),
// clamped at -127; every element is v / 2^s rounded to nearest-even E4M3,
// saturated to +-448.  The pages serve FP8 experts and keep the router in
// higher precision ("LLM MoE Expert Parallel production practice",
// deployment examples; "Expert parallelism for MoE serving", FAQ) without
// fixing a scaling granularity; 32-element blocks are what CDNA4's scaled
// MFMA applies in hardware.
//
// Scale layout (chosen for the GEMM's loads): the scales of the four blocks
// of one 128-column group of a row form one 32-bit word, and the words are
// group-major: block b of row r is byte ((b / 4) * stride + r) * 4 + b % 4,
// stride >= rows.  A GEMM stage of 128 columns then reads one word per row,
// consecutive rows at consecutive addresses.
//
// One wavefront quantises 512 consecutive elements of a row (16 blocks, 4
// lanes of 8 elements per block): a 16-byte load per lane, the block's
// maximum over the 4 lanes by two xor shuffles, the scale from the
// exponent field of the maximum, and 8 hardware conversions to E4M3.
#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kQuantThreads = 256;

// E8M0 byte of a block with maximum magnitude amax (amax >= 0, finite):
// floor(log2 amax) - 8 + 127 = exponent field - 8, at least 0 (2^-127; also
// the byte of an all-zero block).
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
  const int e = (int)(__float_as_uint(amax) >> 23);
  return e > 8 ? (uint32_t)(e - 8) : 0u;
}

// four values, already divided by the block scale, to four E4M3 bytes
// (element 0 in the low byte); round to nearest even, saturate to +-448
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  c = fminf(fmaxf(c, -448.f), 448.f);
  d = fminf(fmaxf(d, -448.f), 448.f);
  int p = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  p = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, p, true);
  return (uint32_t)p;
}

// When row_of_slot is given, each scale byte is also written for every kept
// slot of the row (row r = token r, slots r * k .. r * k + k - 1) at its
// dispatch row in perm_scales (stride perm_stride): the grouped GEMM then
// reads the token scales of a row tile as consecutive words.
template <bool BF16>
__global__ __launch_bounds__(kQuantThreads) void k_quant_mxfp8(const void* __restrict__ src,
                                                               int rows, int cols, int stride,
                                                               uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales,
                                                               uint32_t* __restrict__ flags,
                                                               const int32_t* __restrict__ row_of_slot,
                                                               int k, uint8_t* __restrict__ perm_scales,
                                                               int perm_stride) {
  const int lane = threadIdx.x & 63;
  const long long seg = (long long)blockIdx.x * (kQuantThreads / 64) + (threadIdx.x >> 6);
  const int segs_per_row = (cols + 511) / 512;
  if (seg >= (long long)rows * segs_per_row) return;
  const int r = (int)(seg / segs_per_row);
  const int c0 = (int)(seg - (long long)r * segs_per_row) * 512;
  const int c = c0 + lane * 8;  // this lane's 8 elements
  const bool live = c < cols;   // cols is a multiple of 128: a block is all live or all not
  float v[8];
  if (live) {
    const size_t o = (size_t)r * cols + c;
    if constexpr (BF16) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + o);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else {
      const float* p = static_cast<const float*>(src) + o;
      const float4 a = *reinterpret_cast<const float4*>(p);
      const float4 b = *reinterpret_cast<const float4*>(p + 4);
      v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w;
      v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  if (!live) return;
  if (!(amax <= 3.402823466e38f)) {  // inf or NaN input
    if (flags && (lane & 3) == 0) atomicOr(flags, (uint32_t)MOE_FLAG_H_RANGE);
  }
  const uint32_t sb = mx_scale_byte(amax);
  const int sh = 127 - (int)sb;  // multiply by 2^-s, exactly
  u32x2 out;
  out[0] = e4m3x4(ldexpf(v[0], sh), ldexpf(v[1], sh), ldexpf(v[2], sh), ldexpf(v[3], sh));
  out[1] = e4m3x4(ldexpf(v[4], sh), ldexpf(v[5], sh), ldexpf(v[6], sh), ldexpf(v[7], sh));
  *reinterpret_cast<u32x2*>(codes + (size_t)r * cols + c) = out;
  if ((lane & 3) == 0) {
    const int b = c >> 5;
    scales[((size_t)(b >> 2) * stride + r) * 4 + (b & 3)] = (uint8_t)sb;
    if (row_of_slot) {
      for (int j = 0; j < k; ++j) {
        const int rr = row_of_slot[(size_t)r * k + j];
        if (rr >= 0) perm_scales[((size_t)(b >> 2) * perm_stride + rr) * 4 + (b & 3)] = (uint8_t)sb;
      }
    }
  }
}

}  // namespace

hipError_t launch_quant_mxfp8(int src_dtype, const void* src, int rows, int cols, int stride,
                              uint8_t* codes, uint8_t* scales, uint32_t* flags, hipStream_t st,
                              const int32_t* row_of_slot, int k, uint8_t* perm_scales,
                              int perm_stride) {
  const long long segs = (long long)rows * ((cols + 511) / 512);
  const long long blocks = (segs + kQuantThreads / 64 - 1) / (kQuantThreads / 64);
  if (blocks == 0) return hipSuccess;
  if (src_dtype == MOE_BF16)
    hipLaunchKernelGGL(k_quant_mxfp8<true>, dim3((unsigned)blocks), dim3(kQuantThreads), 0, st, src,
                       rows, cols, stride, codes, scales, flags, row_of_slot, k, perm_scales,
                       perm_stride);
  else
    hipLaunchKernelGGL(k_quant_mxfp8<false>, dim3((unsigned)blocks), dim3(kQuantThreads), 0, st, src,
                       rows, cols, stride, codes, scales, flags, row_of_slot, k, perm_scales,
                       perm_stride);
  return hipGetLastError();
}

}  // namespace moe
