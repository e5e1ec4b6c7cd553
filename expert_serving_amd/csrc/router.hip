// S1 for layers with few experts: router logits
//   logits[t][e] = sum_h x[t][h] * Wr[e][h] + b[e]   (fp32 accumulation)
// ("Expert parallelism for MoE serving", deep dive: a small linear router
// scores every expert for every token).
//
// With E <= 32 the product is a handful of dot products per token, far too
// narrow for 128-wide MFMA tiles, and the cost is reading x once.  Wider
// routers with few tokens (a 128-row MFMA tile per block would leave most
// compute units idle) take the same kernel over slices of EMAX experts
// (blockIdx.y), re-reading the few x rows from L2.  One block
// of 256 threads takes TPB tokens; thread i reads the 16-byte chunks
// i, i+256, ... of each token row (coalesced) and the same chunks of every
// router row (L2-resident), and keeps TPB*EMAX fp32 partial sums.  The
// partial sums are reduced across each wavefront with a transposing
// butterfly -- every exchange halves the values a lane holds, so N values
// need N-1+6-log2(N) shuffles instead of 6N -- and then across the four
// wavefronts through LDS in fixed order, so the result is deterministic.
#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRouterThreads = 256;

__device__ __forceinline__ void bf16x8_to_f32(const u32x4 v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
}

constexpr int ilog2(int n) { return n <= 1 ? 0 : 1 + ilog2(n / 2); }

// The first kernel of a layer call also clears its device flag word (when
// given), which saves a launch of its own.
template <int EMAX, int TPB>
__global__ __launch_bounds__(kRouterThreads) void k_router_skinny(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int T, int H, int E, float* __restrict__ logits,
    uint32_t* __restrict__ flags) {
  if (flags && blockIdx.x == 0 && threadIdx.x == 0) *flags = 0u;
  constexpr int N = EMAX * TPB;  // values per thread, index tok*EMAX + e
  constexpr int L = ilog2(N);
  static_assert((1 << L) == N && N <= 64, "N must be a power of two <= 64");
  constexpr int NWAVES = kRouterThreads / 64;
  __shared__ float s_part[NWAVES][N];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * TPB;
  const int e0 = blockIdx.y * EMAX;  // first expert of this block's slice
  const int chunks = H >> 3;

  float v[N];
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = 0.f;

  for (int c = tid; c < chunks; c += kRouterThreads) {
    // every load of the step is issued before the first use: x rows of the
    // block's tokens, then the router rows (rows e >= E repeat row E-1; their
    // sums are never stored)
    u32x4 xr[TPB], wrr[EMAX];
#pragma unroll
    for (int q = 0; q < TPB; ++q)
      xr[q] = *reinterpret_cast<const u32x4*>(x + (size_t)min(t0 + q, T - 1) * H + c * 8);
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
      wrr[e] = *reinterpret_cast<const u32x4*>(wr + (size_t)min(e0 + e, E - 1) * H + c * 8);
    float xf[TPB][8];
#pragma unroll
    for (int q = 0; q < TPB; ++q) bf16x8_to_f32(xr[q], xf[q]);
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      float wf[8];
      bf16x8_to_f32(wrr[e], wf);
#pragma unroll
      for (int q = 0; q < TPB; ++q)
#pragma unroll
        for (int j = 0; j < 8; ++j) v[q * EMAX + e] = fmaf(xf[q][j], wf[j], v[q * EMAX + e]);
    }
  }

  // transposing butterfly: after step s a lane keeps the half of its values
  // selected by lane bit (5 - s), summed with its partner's copy of that half
#pragma unroll
  for (int s = 0; s < L; ++s) {
    const int off = 32 >> s;
    const int half = N >> (s + 1);
    // bit-select masks, so the choice stays a per-lane select between two
    // registers rather than an indexed read of the array
    const uint32_t up = (lane & off) ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const uint32_t lo = __float_as_uint(v[i]), hi = __float_as_uint(v[i + half]);
      const float send = __uint_as_float((lo & up) | (hi & ~up));
      const float keep = __uint_as_float((hi & up) | (lo & ~up));
      v[i] = keep + __shfl_xor(send, off, 64);
    }
  }
  float r = v[0];
#pragma unroll
  for (int off = 32 >> L; off >= 1; off >>= 1) r += __shfl_xor(r, off, 64);
  // the lane's value index is given by its top L lane bits
  if ((lane & ((64 >> L) - 1)) == 0) s_part[wave][lane >> (6 - L)] = r;
  __syncthreads();
  if (tid < N) {
    float sum = s_part[0][tid];
#pragma unroll
    for (int w = 1; w < NWAVES; ++w) sum += s_part[w][tid];
    const int q = tid / EMAX, e = tid % EMAX, t = t0 + q;
    if (t < T && e0 + e < E) logits[(size_t)t * E + e0 + e] = sum + (bias ? bias[e0 + e] : 0.f);
  }
}

template <int EMAX, int TPB>
hipError_t launch_skinny(const void* x, const void* wr, const float* bias, int T, int H, int E,
                         float* logits, uint32_t* flags, hipStream_t st) {
  hipLaunchKernelGGL((k_router_skinny<EMAX, TPB>), dim3((T + TPB - 1) / TPB, (E + EMAX - 1) / EMAX),
                     dim3(kRouterThreads), 0, st, static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(wr), bias, T, H, E, logits, flags);
  return hipGetLastError();
}

}  // namespace

bool router_skinny_supported(const moe_shape& s) {
  return s.act_dtype == MOE_BF16 &&
         (s.num_experts <= kRouterSkinnyMaxExperts || s.num_tokens <= kRouterSlicedMaxTokens);
}

hipError_t launch_router_skinny(const moe_shape& s, const void* x, const void* w_router,
                                const float* bias, float* logits, uint32_t* flags, hipStream_t st) {
  const int T = s.num_tokens, H = s.hidden, E = s.num_experts;
  // several tokens per block share each router-row load; below 1024 tokens
  // one token per block keeps enough blocks in flight
  const bool wide = T >= 1024;
  // wide routers, few tokens: 8-expert slices, one token per block below 64
  // tokens, four above
  if (E > kRouterSkinnyMaxExperts)
    return T >= 64 ? launch_skinny<8, 4>(x, w_router, bias, T, H, E, logits, flags, st)
                   : launch_skinny<8, 1>(x, w_router, bias, T, H, E, logits, flags, st);
  if (E <= 8)
    return wide ? launch_skinny<8, 4>(x, w_router, bias, T, H, E, logits, flags, st)
                : launch_skinny<8, 1>(x, w_router, bias, T, H, E, logits, flags, st);
  if (E <= 16)
    return wide ? launch_skinny<16, 4>(x, w_router, bias, T, H, E, logits, flags, st)
                : launch_skinny<16, 1>(x, w_router, bias, T, H, E, logits, flags, st);
  return wide ? launch_skinny<32, 2>(x, w_router, bias, T, H, E, logits, flags, st)
              : launch_skinny<32, 1>(x, w_router, bias, T, H, E, logits, flags, st);
}

}  // namespace moe
