// S10: combine -- the k_t expert outputs of a token, weighted by the router
// gates, summed back into the token's own row ("Expert Parallelism: MoE model
// parallel split", §1 weighted sum and §12 Q2: combine merges the k outputs
// back to the original position).  On one GPU this is the inverse of the
// dispatch permutation: a gather over row_of_slot, never a scatter with
// atomics, so the sum order (slot j ascending, then the shared expert) is
// fixed.
#include "moe_internal.h"

namespace moe {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b + (((b >> 16) & 1u) + 0x7FFFu)) >> 16;
}

// Four fp16 values (8 bytes) widened to fp32.
__device__ __forceinline__ f32x4 load_h4(const void* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  const auto lo = __builtin_bit_cast(_Float16 __attribute__((ext_vector_type(2))), w.x);
  const auto hi = __builtin_bit_cast(_Float16 __attribute__((ext_vector_type(2))), w.y);
  return f32x4{(float)lo[0], (float)lo[1], (float)hi[0], (float)hi[1]};
}

// One block per token (and column slice: a small batch splits the columns
// over gridDim.y blocks so that more compute units share the reads); thread
// i owns 4 consecutive columns per pass.  KM is
// a compile-time bound on k_max (2, 4, 8 or 16), so the loads of all of a
// token's rows are issued before the first multiply-add waits on them.  y may
// come in `parts` partial sums (a K-split down projection), each `part_stride`
// floats apart; they are added in part order before the gate multiplies.
// YH: y and y_shared hold fp16 values (one part), widened exactly to fp32.
template <bool OUT_BF16, int KM, bool YH>
__global__ __launch_bounds__(256) void k_combine(const void* __restrict__ yv, int parts,
                                                 long long part_stride,
                                                 const int32_t* __restrict__ row_of_slot,
                                                 const float* __restrict__ gates,
                                                 const void* __restrict__ ysv, int H,
                                                 int k_max, void* __restrict__ out) {
  const float* y = static_cast<const float*>(yv);
  const float* y_shared = static_cast<const float*>(ysv);
  const uint16_t* yh = static_cast<const uint16_t*>(yv);
  const uint16_t* ysh = static_cast<const uint16_t*>(ysv);
  const int t = blockIdx.x;
  __shared__ int s_row[KM];
  __shared__ float s_g[KM];
  if (threadIdx.x < KM) {
    const bool live = (int)threadIdx.x < k_max;
    s_row[threadIdx.x] = live ? row_of_slot[(size_t)t * k_max + threadIdx.x] : -1;
    s_g[threadIdx.x] = live ? gates[(size_t)t * k_max + threadIdx.x] : 0.f;
  }
  __syncthreads();
  for (int c = (blockIdx.y * blockDim.x + threadIdx.x) * 4; c < H; c += gridDim.y * blockDim.x * 4) {
    f32x4 v[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      const int r = s_row[j];
      v[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (r >= 0) {
        if constexpr (YH) {
          v[j] = load_h4(yh + (size_t)r * H + c);
        } else {
          v[j] = *reinterpret_cast<const f32x4*>(y + (size_t)r * H + c);
          for (int p = 1; p < parts; ++p)
            v[j] += *reinterpret_cast<const f32x4*>(y + p * part_stride + (size_t)r * H + c);
        }
      }
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (s_row[j] < 0) continue;
      const float g = s_g[j];
      acc[0] = fmaf(g, v[j][0], acc[0]);
      acc[1] = fmaf(g, v[j][1], acc[1]);
      acc[2] = fmaf(g, v[j][2], acc[2]);
      acc[3] = fmaf(g, v[j][3], acc[3]);
    }
    if (ysv) {
      if constexpr (YH) acc += load_h4(ysh + (size_t)t * H + c);
      else acc += *reinterpret_cast<const f32x4*>(y_shared + (size_t)t * H + c);
    }
    if constexpr (OUT_BF16) {
      uint2 pk;
      pk.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
      pk.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + (size_t)t * H + c) = pk;
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(out) + (size_t)t * H + c) = acc;
    }
  }
}

template <int KM, bool YH>
hipError_t launch_combine_k(const moe_shape& s, const void* y, int parts, long long part_stride,
                            const int32_t* row_of_slot, const float* gates, const void* y_shared,
                            void* out, hipStream_t st) {
  // fewer than 512 tokens: up to one block per 1024 columns of a token
  const int ysplit = s.num_tokens < 512 ? std::max(1, s.hidden / 1024) : 1;
  const dim3 grid(s.num_tokens, ysplit);
  if (s.out_dtype == MOE_BF16)
    hipLaunchKernelGGL((k_combine<true, KM, YH>), grid, dim3(256), 0, st, y, parts, part_stride, row_of_slot,
                       gates, y_shared, s.hidden, s.top_k, out);
  else
    hipLaunchKernelGGL((k_combine<false, KM, YH>), grid, dim3(256), 0, st, y, parts, part_stride, row_of_slot,
                       gates, y_shared, s.hidden, s.top_k, out);
  return hipGetLastError();
}

template <bool YH>
hipError_t launch_combine_y(const moe_shape& s, const void* y_perm, const int32_t* row_of_slot,
                            const float* gates, const void* y_shared, void* out, hipStream_t st, int parts,
                            long long part_stride) {
  if (s.top_k <= 2)
    return launch_combine_k<2, YH>(s, y_perm, parts, part_stride, row_of_slot, gates, y_shared, out, st);
  if (s.top_k <= 4)
    return launch_combine_k<4, YH>(s, y_perm, parts, part_stride, row_of_slot, gates, y_shared, out, st);
  if (s.top_k <= 8)
    return launch_combine_k<8, YH>(s, y_perm, parts, part_stride, row_of_slot, gates, y_shared, out, st);
  return launch_combine_k<kMaxTopK, YH>(s, y_perm, parts, part_stride, row_of_slot, gates, y_shared, out, st);
}

}  // namespace

hipError_t launch_combine(const moe_shape& s, const void* y_perm, const int32_t* row_of_slot,
                          const float* gates, const void* y_shared, void* out, hipStream_t st,
                          int parts, long long part_stride, bool y_half) {
  if (y_half) {
    if (parts != 1) return hipErrorInvalidValue;
    return launch_combine_y<true>(s, y_perm, row_of_slot, gates, y_shared, out, st, 1, 0);
  }
  return launch_combine_y<false>(s, y_perm, row_of_slot, gates, y_shared, out, st, parts, part_stride);
}

}  // namespace moe
