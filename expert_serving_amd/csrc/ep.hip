// The expert-parallel exchange on one GPU: the send layout of the dispatch
// exchange over G ranks, and the source's sum of the rows the ranks return.
//
// "Expert Parallelism: MoE model parallel split": with expert parallelism
// over G GPUs the experts form G contiguous blocks (§8, EP=8: 32 experts per
// GPU); each MoE layer exchanges twice -- dispatch sends a token's hidden
// state to the ranks of its experts, combine brings their outputs back (§3,
// §12 Q2); rows bound for one rank are grouped into one send (§7 and §12,
// token sorting).  "Expert parallelism for MoE serving", deployment
// examples: node-limited routing bounds the ranks a token's experts span, so
// a token travels once to each rank holding any of its experts; that rank
// runs all of the token's experts it holds on the one row and returns their
// gate-weighted sum as one row.
//
// Send layout: destination-major, tokens ascending within a destination, no
// padding rows.  Positions come from per-tile counts, a column scan and
// in-wave ballot ranks -- never from atomics -- so the layout is bitwise
// deterministic.
//   k_ep_count    per 64-token tile: rows per destination rank
//   k_ep_scan     per-tile bases, rank counts and offsets (one block)
//   k_ep_scatter  positions -> send_token, send_ids, send_gates, slot_send_pos
//   k_ep_combine  out[t] = sum of the token's returned rows, ascending rank
#include "moe_internal.h"

namespace moe {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kEpTileTokens = 64;  // one wavefront, one token per lane

// Bit d: token t has a routed slot (id in [0, E)) on rank d (experts
// d*epr .. d*epr + epr - 1).  Ids outside [-1, E) set `bad`.
__device__ __forceinline__ uint64_t rank_mask(const int32_t* __restrict__ ids, int t, int T, int k, int E,
                                              int epr, bool& bad) {
  uint64_t m = 0;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = ids[(size_t)t * k + j];
      if (e >= 0 && e < E) m |= 1ull << (e / epr);
      else if (e != -1) bad = true;
    }
  }
  return m;
}

// Four tiles per block, one per wavefront.
__global__ __launch_bounds__(256) void k_ep_count(const int32_t* __restrict__ ids, int T, int k, int E, int G,
                                                  int n_tiles, int32_t* __restrict__ tile_counts,
                                                  uint32_t* __restrict__ flags) {
  const int lane = threadIdx.x & 63;
  const int tile = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= n_tiles) return;  // whole wavefronts
  bool bad = false;
  const uint64_t m = rank_mask(ids, tile * kEpTileTokens + lane, T, k, E, E / G, bad);
  int mine = 0;
  for (int d = 0; d < G; ++d) {
    const int c = __popcll(__ballot((m >> d) & 1ull));
    if (lane == d) mine = c;
  }
  if (lane < G) tile_counts[(size_t)tile * G + lane] = mine;
  if (__ballot(bad) && lane == 0) atomicOr(flags, (uint32_t)MOE_FLAG_BAD_EXPERT);
}

// One block of 1024 threads.  Each rank's column of tile counts is cut into
// P = 1024 / gp contiguous ranges (gp = G rounded up to a power of two), one
// thread each; the column totals give rank_counts and rank_offsets, and the
// counts are rewritten in place as each tile's first row for each rank.
__global__ __launch_bounds__(1024) void k_ep_scan(int32_t* __restrict__ tile_counts, int n_tiles, int G,
                                                  int32_t* __restrict__ rank_counts,
                                                  int32_t* __restrict__ rank_offsets) {
  __shared__ int s_part[1024];
  __shared__ int s_off[64];
  const int tid = threadIdx.x;
  int gp = 1;
  while (gp < G) gp <<= 1;
  const int P = 1024 / gp, d = tid % gp, g = tid / gp;
  const int per = (n_tiles + P - 1) / P;
  const int lo = min(g * per, n_tiles), hi = min(lo + per, n_tiles);
  int part = 0;
  if (d < G)
    for (int b = lo; b < hi; ++b) part += tile_counts[(size_t)b * G + d];
  s_part[tid] = part;
  __syncthreads();
  if (tid < G) {
    int tot = 0;
    for (int q = 0; q < P; ++q) tot += s_part[q * gp + tid];
    s_off[tid] = tot;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int r = 0; r < G; ++r) {
      const int c = s_off[r];
      rank_counts[r] = c;
      rank_offsets[r] = run;
      s_off[r] = run;
      run += c;
    }
    rank_offsets[G] = run;
  }
  __syncthreads();
  if (d < G) {
    int base = s_off[d];
    for (int q = 0; q < g; ++q) base += s_part[q * gp + d];
    for (int b = lo; b < hi; ++b) {
      const int c = tile_counts[(size_t)b * G + d];
      tile_counts[(size_t)b * G + d] = base;
      base += c;
    }
  }
}

// Positions of a tile's rows: a token's row for rank d goes to the tile's
// first row for d plus the number of lower lanes (earlier tokens) with d.
// Rows at and beyond the rows sent (up to n_rows) are cleared by the grid.
__global__ __launch_bounds__(256) void k_ep_scatter(const int32_t* __restrict__ ids,
                                                    const float* __restrict__ gates, int T, int k, int E,
                                                    int G, const int32_t* __restrict__ tile_base, int n_tiles,
                                                    const int32_t* __restrict__ rank_offsets, int n_rows,
                                                    int32_t* __restrict__ send_token,
                                                    int32_t* __restrict__ send_ids,
                                                    float* __restrict__ send_gates,
                                                    int32_t* __restrict__ slot_send_pos) {
  __shared__ int s_rank[256][kMaxTopK];
  __shared__ int s_pos[256][kMaxTopK];
  const int S = rank_offsets[G];
  for (int p = S + blockIdx.x * 256 + threadIdx.x; p < n_rows; p += gridDim.x * 256) {
    send_token[p] = -1;
    for (int j = 0; j < k; ++j) {
      send_ids[(size_t)p * k + j] = -1;
      send_gates[(size_t)p * k + j] = 0.f;
    }
  }
  const int lane = threadIdx.x & 63;
  const int tile = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= n_tiles) return;  // whole wavefronts
  const int epr = E / G;
  const int t = tile * kEpTileTokens + lane;
  bool bad = false;  // flagged by k_ep_count
  const uint64_t m = rank_mask(ids, t, T, k, E, epr, bad);
  const uint64_t below = (1ull << lane) - 1ull;
  int n = 0;  // the token's ranks, ascending (at most min(k, G) <= kMaxTopK)
  for (int d = 0; d < G; ++d) {
    const uint64_t b = __ballot((m >> d) & 1ull);
    if ((m >> d) & 1ull) {
      s_rank[threadIdx.x][n] = d;
      s_pos[threadIdx.x][n] = tile_base[(size_t)tile * G + d] + __popcll(b & below);
      ++n;
    }
  }
  if (t >= T) return;
  for (int q = 0; q < n; ++q) {
    const int d = s_rank[threadIdx.x][q], p = s_pos[threadIdx.x][q];
    send_token[p] = t;
    for (int j = 0; j < k; ++j) {
      const int e = ids[(size_t)t * k + j];
      const bool on = e >= 0 && e < E && e / epr == d;
      send_ids[(size_t)p * k + j] = on ? e - d * epr : -1;
      send_gates[(size_t)p * k + j] = on ? gates[(size_t)t * k + j] : 0.f;
    }
  }
  for (int j = 0; j < k; ++j) {
    const int e = ids[(size_t)t * k + j];
    int p = -1;
    if (e >= 0 && e < E) {
      const int d = e / epr;
      for (int q = 0; q < n; ++q)
        if (s_rank[threadIdx.x][q] == d) p = s_pos[threadIdx.x][q];
    }
    slot_send_pos[(size_t)t * k + j] = p;
  }
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b + (((b >> 16) & 1u) + 0x7FFFu)) >> 16;
}

// One block per token (and column slice for small batches); thread i owns 4
// consecutive columns per pass.  The token's distinct returned rows are
// summed in ascending order (ascending rank), then y_shared.  KM bounds the
// rows per token (min(k, G)), so every row's loads issue before the adds.
template <bool OUT_BF16, int KM>
__global__ __launch_bounds__(256) void k_ep_combine(const float* __restrict__ partial,
                                                    const int32_t* __restrict__ slot_send_pos,
                                                    const float* __restrict__ y_shared, int H, int k,
                                                    void* __restrict__ out) {
  const int t = blockIdx.x;
  __shared__ int s_rows[KM];
  __shared__ int s_n;
  if (threadIdx.x == 0) {
    int n = 0;
    for (int j = 0; j < k; ++j) {
      const int r = slot_send_pos[(size_t)t * k + j];
      if (r < 0) continue;
      bool seen = false;
      for (int q = 0; q < n; ++q) seen |= s_rows[q] == r;
      if (seen || n >= KM) continue;
      int q = n++;
      while (q > 0 && s_rows[q - 1] > r) {
        s_rows[q] = s_rows[q - 1];
        --q;
      }
      s_rows[q] = r;
    }
    s_n = n;
  }
  __syncthreads();
  const int n = s_n;
  for (int c = (blockIdx.y * blockDim.x + threadIdx.x) * 4; c < H; c += gridDim.y * blockDim.x * 4) {
    f32x4 v[KM];
#pragma unroll
    for (int q = 0; q < KM; ++q) {
      v[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (q < n) v[q] = *reinterpret_cast<const f32x4*>(partial + (size_t)s_rows[q] * H + c);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < KM; ++q)
      if (q < n) acc += v[q];
    if (y_shared) acc += *reinterpret_cast<const f32x4*>(y_shared + (size_t)t * H + c);
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

template <int KM>
hipError_t launch_ep_combine_k(const moe_shape& s, const float* partial, const int32_t* slot_send_pos,
                               const float* y_shared, void* out, hipStream_t st) {
  const int ysplit = s.num_tokens < 512 ? std::max(1, s.hidden / 1024) : 1;
  const dim3 grid(s.num_tokens, ysplit);
  if (s.out_dtype == MOE_BF16)
    hipLaunchKernelGGL((k_ep_combine<true, KM>), grid, dim3(256), 0, st, partial, slot_send_pos, y_shared,
                       s.hidden, s.top_k, out);
  else
    hipLaunchKernelGGL((k_ep_combine<false, KM>), grid, dim3(256), 0, st, partial, slot_send_pos, y_shared,
                       s.hidden, s.top_k, out);
  return hipGetLastError();
}

}  // namespace

int ep_tiles(int num_tokens) { return (num_tokens + kEpTileTokens - 1) / kEpTileTokens; }

hipError_t launch_ep_layout(const moe_shape& s, int G, const int32_t* ids, const float* gates,
                            int32_t* rank_counts, int32_t* rank_offsets, int32_t* send_token,
                            int32_t* send_ids, float* send_gates, int32_t* slot_send_pos,
                            int32_t* tile_counts, uint32_t* flags, hipStream_t st) {
  const int T = s.num_tokens, k = s.top_k, E = s.num_experts;
  const int n_tiles = ep_tiles(T);
  const int n_rows = T * std::min(k, G);
  const int blocks = (n_tiles + 3) / 4;
  hipLaunchKernelGGL(k_ep_count, dim3(blocks), dim3(256), 0, st, ids, T, k, E, G, n_tiles, tile_counts, flags);
  hipLaunchKernelGGL(k_ep_scan, dim3(1), dim3(1024), 0, st, tile_counts, n_tiles, G, rank_counts, rank_offsets);
  hipLaunchKernelGGL(k_ep_scatter, dim3(blocks), dim3(256), 0, st, ids, gates, T, k, E, G, tile_counts, n_tiles,
                     rank_offsets, n_rows, send_token, send_ids, send_gates, slot_send_pos);
  return hipGetLastError();
}

hipError_t launch_ep_combine(const moe_shape& s, int G, const float* partial, const int32_t* slot_send_pos,
                             const float* y_shared, void* out, hipStream_t st) {
  const int km = std::min(s.top_k, G);
  if (km <= 2) return launch_ep_combine_k<2>(s, partial, slot_send_pos, y_shared, out, st);
  if (km <= 4) return launch_ep_combine_k<4>(s, partial, slot_send_pos, y_shared, out, st);
  if (km <= 8) return launch_ep_combine_k<8>(s, partial, slot_send_pos, y_shared, out, st);
  return launch_ep_combine_k<kMaxTopK>(s, partial, slot_send_pos, y_shared, out, st);
}

}  // namespace moe
