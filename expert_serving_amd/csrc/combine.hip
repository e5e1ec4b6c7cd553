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

// One block per token; thread i owns 4 consecutive columns per pass.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y,
                                                 const int32_t* __restrict__ row_of_slot,
                                                 const float* __restrict__ gates,
                                                 const float* __restrict__ y_shared, int H,
                                                 int k_max, void* __restrict__ out) {
  const int t = blockIdx.x;
  __shared__ int s_row[kMaxTopK];
  __shared__ float s_g[kMaxTopK];
  if (threadIdx.x < k_max) {
    s_row[threadIdx.x] = row_of_slot[(size_t)t * k_max + threadIdx.x];
    s_g[threadIdx.x] = gates[(size_t)t * k_max + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x * 4; c < H; c += blockDim.x * 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k_max; ++j) {
      const int r = s_row[j];
      if (r < 0) continue;
      const float g = s_g[j];
      const f32x4 v = *reinterpret_cast<const f32x4*>(y + (size_t)r * H + c);
      acc[0] = fmaf(g, v[0], acc[0]);
      acc[1] = fmaf(g, v[1], acc[1]);
      acc[2] = fmaf(g, v[2], acc[2]);
      acc[3] = fmaf(g, v[3], acc[3]);
    }
    if (y_shared) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(y_shared + (size_t)t * H + c);
      acc += v;
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

}  // namespace

hipError_t launch_combine(const moe_shape& s, const float* y_perm, const int32_t* row_of_slot,
                          const float* gates, const float* y_shared, void* out, hipStream_t st) {
  const dim3 grid(s.num_tokens);
  if (s.out_dtype == MOE_BF16)
    hipLaunchKernelGGL(k_combine<true>, grid, dim3(256), 0, st, y_perm, row_of_slot, gates,
                       y_shared, s.hidden, s.top_k, out);
  else
    hipLaunchKernelGGL(k_combine<false>, grid, dim3(256), 0, st, y_perm, row_of_slot, gates,
                       y_shared, s.hidden, s.top_k, out);
  return hipGetLastError();
}

}  // namespace moe
