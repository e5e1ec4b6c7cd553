// S2: router scoring, optional group limit, top-k_t selection and gates.
//
// One 64-lane wavefront per token.  Lane l holds EPL consecutive logits
// (experts l*EPL .. l*EPL+EPL-1), so a selection round is a lane-local
// compare followed by a 6-step butterfly over the wavefront.
//
// Pages: a router picks the top-k experts per token ("Expert parallelism for
// MoE serving", deep dive and FAQ); node-limited routing bounds the groups a
// token's experts span (same page, deployment examples); the routing budget k
// may differ per request (MoE-Prism summary, §1 and §5).
#include <climits>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kMaxGroupTopn = 8;

// The fp32 logistic function used for group scores, as a fixed sequence of
// IEEE single-precision operations rounded to nearest even (no contraction):
// clamp to [-30, 30]; e^-x by Cody-Waite reduction n = rint(-x*log2e),
// r = -x - n*ln2 with ln2 split into a 17-bit head and an fp32 tail; a
// degree-7 Taylor polynomial of e^r (coefficients fp32(1/i!)) in Horner form
// with fused multiply-adds; ldexp by n; then 1/(1+e).
__device__ __forceinline__ float logistic_seq(float x) {
  x = x < -30.0f ? -30.0f : x;
  x = x > 30.0f ? 30.0f : x;
  const float z = -x;
  const float n = rintf(__fmul_rn(z, 0x1.715476p+0f));
  float r = __fmaf_rn(-n, 0x1.62e400p-1f, z);
  r = __fmaf_rn(-n, 0x1.7f7d1cp-20f, r);
  float p = 0x1.a01a02p-13f;
  p = __fmaf_rn(p, r, 0x1.6c16c2p-10f);
  p = __fmaf_rn(p, r, 0x1.111112p-7f);
  p = __fmaf_rn(p, r, 0x1.555556p-5f);
  p = __fmaf_rn(p, r, 0x1.555556p-3f);
  p = __fmaf_rn(p, r, 0x1.0p-1f);
  p = __fmaf_rn(p, r, 1.0f);
  p = __fmaf_rn(p, r, 1.0f);
  const float e = ldexpf(p, (int)n);
  return __fdiv_rn(1.0f, __fadd_rn(1.0f, e));
}

// (va, ia) ranks before (vb, ib): valid first, larger value, then lower index.
// (Bitwise operators, so the test compiles to mask arithmetic, not branches.)
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
  return (ia != INT_MAX) & ((ib == INT_MAX) | (va > vb) | ((va == vb) & (ia < ib)));
}

__device__ __forceinline__ void wave_argbest(float& v, int& i) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(v, off, 64);
    const int oi = __shfl_xor(i, off, 64);
    if (ranks_before(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

template <int EPL>
__global__ __launch_bounds__(256) void k_route_topk(const float* __restrict__ logits, int T, int E,
                                                    int k_max, const int32_t* __restrict__ kpt,
                                                    int score, int renorm, float scale, int G,
                                                    int topk_groups, int topn,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ gates,
                                                    uint32_t* __restrict__ flags, int parts,
                                                    long long part_stride, float* __restrict__ sum_out) {
  __shared__ float s_logit[kWavesPerBlock][kMaxExperts];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * kWavesPerBlock + wave;
  const bool active = t < T;

  float v[EPL];
  bool elig[EPL];
  int ec[EPL];  // the lane's experts, clamped to a valid address
  // logits in `parts` partial sums (a K-split router) are added in part
  // order, and the sums stored at sum_out.  Every load of a part is issued
  // before the first is used.
  const float* lt = logits + (size_t)(active ? t : 0) * E;
  int kt = k_max;
  if (active && kpt) kt = kpt[t];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane * EPL + i;
    elig[i] = active && e < E;
    ec[i] = elig[i] ? e : 0;
    v[i] = lt[ec[i]];
  }
  for (int p = 1; p < parts; ++p) {
    float w[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) w[i] = lt[p * part_stride + ec[i]];
#pragma unroll
    for (int i = 0; i < EPL; ++i) v[i] += w[i];
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    if (parts > 1 && sum_out && elig[i]) sum_out[(size_t)t * E + ec[i]] = v[i];
    v[i] = elig[i] ? v[i] : 0.0f;
  }
  const bool bad_k = active && (kt < 1 || kt > k_max);

  // ---- group limit: lane g ends with group g's score, the wave keeps the best groups ----
  if (G > 1) {
    const int gs = E / G;
    const int gl = gs / EPL;  // lanes of a group, when groups fall on whole lanes
    float gscore = 0.0f;
    int gidx = INT_MAX;
    if (gs % EPL == 0 && gl > 0 && (gl & (gl - 1)) == 0) {
      // Groups on whole, aligned runs of gl lanes: every lane scores its own
      // experts into a descending top-n list, and a butterfly over the
      // group's lanes merges the lists (each lane inserts its partner's), so
      // every lane of the group ends with the group's n largest scores.  The
      // score is their sum, largest first, as below.
      float top[kMaxGroupTopn];
#pragma unroll
      for (int q = 0; q < kMaxGroupTopn; ++q) top[q] = -1.0f;  // below any sigmoid value
      auto insert = [&](float sv) {
#pragma unroll
        for (int q = 0; q < kMaxGroupTopn; ++q) {
          if (q < topn && sv > top[q]) {
            const float tmp = top[q];
            top[q] = sv;
            sv = tmp;
          }
        }
      };
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane * EPL + i < E) insert(logistic_seq(v[i]));
      for (int m = 1; m < gl; m <<= 1) {
        float other[kMaxGroupTopn];
#pragma unroll
        for (int q = 0; q < kMaxGroupTopn; ++q) other[q] = __shfl_xor(top[q], m, 64);
#pragma unroll
        for (int q = 0; q < kMaxGroupTopn; ++q)
          if (q < topn) insert(other[q]);
      }
      float sum = top[0];
#pragma unroll
      for (int q = 1; q < kMaxGroupTopn; ++q)
        if (q < topn) sum = __fadd_rn(sum, top[q]);
      const float at_g = __shfl(sum, (lane < G ? lane : 0) * gl, 64);
      if (active && lane < G) {
        gscore = at_g;
        gidx = lane;
      }
    } else {
      // other group shapes: lane g scores group g serially
      if (active) {
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (elig[i]) s_logit[wave][lane * EPL + i] = v[i];
      }
      __syncthreads();
      if (active && lane < G) {
        float top[kMaxGroupTopn];
#pragma unroll
        for (int q = 0; q < kMaxGroupTopn; ++q) top[q] = -1.0f;  // below any sigmoid value
        for (int e = lane * gs; e < (lane + 1) * gs; ++e) {
          float s = logistic_seq(s_logit[wave][e]);
          // insert into the descending list top[0..topn)
#pragma unroll
          for (int q = 0; q < kMaxGroupTopn; ++q) {
            if (q < topn && s > top[q]) {
              const float tmp = top[q];
              top[q] = s;
              s = tmp;
            }
          }
        }
        float sum = top[0];
#pragma unroll
        for (int q = 1; q < kMaxGroupTopn; ++q)
          if (q < topn) sum = __fadd_rn(sum, top[q]);
        gscore = sum;
        gidx = lane;
      }
    }
    uint64_t kept = 0;
    for (int q = 0; q < topk_groups; ++q) {
      float bv = gscore;
      int bi = gidx;
      wave_argbest(bv, bi);
      if (bi != INT_MAX) {
        kept |= 1ull << bi;
        if (lane == bi) gidx = INT_MAX;  // taken
      }
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane * EPL + i;
      if (elig[i]) elig[i] = (kept >> (e / gs)) & 1ull;
    }
  }
  if (!active) return;

  int32_t* idt = ids + (size_t)t * k_max;
  float* gt = gates + (size_t)t * k_max;
  if (bad_k) {
    if (lane < k_max) {
      idt[lane] = -1;
      gt[lane] = 0.0f;
    }
    if (lane == 0) atomicOr(flags, (uint32_t)MOE_FLAG_BAD_K);
    return;
  }

  // ---- top-k_t: k_t rounds of (lane-local best, wave butterfly) ----
  int my_id = -1;
  float my_v = 0.0f, v0 = 0.0f;
  for (int j = 0; j < kt; ++j) {
    float bv = 0.0f;
    int bi = INT_MAX;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane * EPL + i;
      if (elig[i] && ranks_before(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
    wave_argbest(bv, bi);
    if (bi == INT_MAX) break;  // fewer eligible experts than k_t (rejected on the host)
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane * EPL + i == bi) elig[i] = false;
    if (j == 0) v0 = bv;
    if (lane == j) {
      my_id = bi;
      my_v = bv;
    }
  }

  // ---- gates ----
  const bool mine = lane < kt && my_id >= 0;
  float g = 0.0f;
  if (score == MOE_SCORE_SOFTMAX) {
    if (renorm) {
      // softmax over all E renormalised over the selected equals softmax over
      // the selected logits; subtract the largest selected logit
      const float e = mine ? expf(my_v - v0) : 0.0f;
      const float s = wave_sum(e);
      g = e / s;
    } else {
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane * EPL + i < E) m = fmaxf(m, v[i]);
      m = wave_max(m);
      float d = 0.0f;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane * EPL + i < E) d += expf(v[i] - m);
      d = wave_sum(d);
      g = mine ? expf(my_v - m) / d : 0.0f;
    }
  } else {
    const float sg = mine ? 1.0f / (1.0f + expf(-my_v)) : 0.0f;
    if (renorm) {
      const float s = wave_sum(sg);
      g = sg / s;
    } else {
      g = sg;
    }
  }
  g = g * scale;
  if (lane < k_max) {
    idt[lane] = mine ? my_id : -1;
    gt[lane] = mine ? g : 0.0f;
  }
}

__global__ __launch_bounds__(256) void k_logistic(const float* __restrict__ x,
                                                  float* __restrict__ y, long long n) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    y[i] = logistic_seq(x[i]);
}

}  // namespace

hipError_t launch_logistic(const float* x, float* y, long long n, hipStream_t st) {
  const long long blocks = (n + 255) / 256;
  const int grid = (int)(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL(k_logistic, dim3(grid), dim3(256), 0, st, x, y, n);
  return hipGetLastError();
}

hipError_t launch_route_topk(const moe_shape& s, const float* logits, const int32_t* k_per_token,
                             int32_t* ids, float* gates, uint32_t* flags, hipStream_t st, int parts,
                             long long part_stride, float* sum_out) {
  const int T = s.num_tokens, E = s.num_experts;
  const int grid = (T + kWavesPerBlock - 1) / kWavesPerBlock;
  const int G = s.num_groups > 1 ? s.num_groups : 1;
  const int topn = s.group_topn > 0 ? s.group_topn : 1;
#define MOE_ROUTE_LAUNCH(EPL)                                                                    \
  hipLaunchKernelGGL(k_route_topk<EPL>, dim3(grid), dim3(256), 0, st, logits, T, E, s.top_k,   \
                     k_per_token, s.score, s.renormalize, s.routed_scale, G, s.topk_groups,     \
                     topn, ids, gates, flags, parts, part_stride, sum_out)
  if (E <= 64) MOE_ROUTE_LAUNCH(1);
  else if (E <= 128) MOE_ROUTE_LAUNCH(2);
  else if (E <= 256) MOE_ROUTE_LAUNCH(4);
  else MOE_ROUTE_LAUNCH(8);
#undef MOE_ROUTE_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
