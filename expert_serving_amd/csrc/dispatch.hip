// S3-S6: dispatch indexing and the permutation gather.
//
// On one GPU the dispatch all-to-all of expert parallelism ("Expert
// Parallelism: MoE model parallel split", §3 and §12 Q2) becomes a stable
// permutation of the k_t routed copies of each token into per-expert
// contiguous row groups, sorted by destination (the "token sorting" of §7),
// with an optional per-expert capacity that drops slots beyond it in token
// order ("Expert parallelism for MoE serving", technical notes and FAQ).
//
// Determinism: counts use LDS atomics (order does not change a count); every
// position comes from scans and in-wave ranks, never from an atomic claim.
//   k_tile_hist     per tile of kDispatchTileSlots slots: expert histogram
//   k_scan_capacity column scan over tiles, capacity, offsets, drops
//   k_rank_scatter  in-tile stable rank -> row_of_slot, row_token
//   k_dispatch_single  all three in one block when the slots fit one tile
//   k_gather        x_perm[row] = x[row_token[row]]
//   k_build_sched   row tiles of the grouped GEMM from the offsets
#include <climits>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRankWaves = 4;
constexpr int kSlotsPerWave = kDispatchTileSlots / kRankWaves;
constexpr int kRankChunks = kSlotsPerWave / 64;  // 64-slot chunks per wave
static_assert(kSlotsPerWave % 64 == 0, "dispatch tile");

__global__ __launch_bounds__(256) void k_tile_hist(const int32_t* __restrict__ ids,
                                                   int total_slots, int E,
                                                   int32_t* __restrict__ tile_counts,
                                                   uint32_t* __restrict__ flags) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int bad;
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  const int s0 = blockIdx.x * kDispatchTileSlots;
  const int s1 = min(s0 + kDispatchTileSlots, total_slots);
  for (int s = s0 + threadIdx.x; s < s1; s += blockDim.x) {
    const int e = ids[s];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    else if (e != -1) bad = 1;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    tile_counts[(size_t)blockIdx.x * E + e] = cnt[e];
  if (threadIdx.x == 0 && bad) atomicOr(flags, (uint32_t)MOE_FLAG_BAD_EXPERT);
}

// One block of 1024 threads.  Turns tile_counts into per-tile bases (in place),
// writes counts, capacity-limited offsets, the drop count and the capacity.
// Each expert's column of tile counts is cut into P = 1024 / ep contiguous
// ranges (ep = E rounded up to a power of two), one thread each: a first pass
// sums the ranges, a second rewrites each range from its exclusive base.
__global__ __launch_bounds__(1024) void k_scan_capacity(int32_t* __restrict__ tile_counts,
                                                        int n_tiles, int E, float cf,
                                                        int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ num_dropped,
                                                        int32_t* __restrict__ cap_out) {
  __shared__ long long s_total[1024];
  __shared__ int s_scan[1024];
  __shared__ int s_part[1024];
  const int tid = threadIdx.x;
  int ep = 1;
  while (ep < E) ep <<= 1;
  const int P = 1024 / ep, e = tid % ep, g = tid / ep;
  const int per = (n_tiles + P - 1) / P;
  const int b_lo = min(g * per, n_tiles), b_hi = min(b_lo + per, n_tiles);
  int part = 0;
  if (e < E) {
    // eight tiles per round, so eight loads are in flight at once
    for (int b0 = b_lo; b0 < b_hi; b0 += 8) {
      int c[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = b0 + i < b_hi ? tile_counts[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) part += c[i];
    }
  }
  s_part[tid] = part;
  __syncthreads();
  if (e < E) {
    int base = 0;
    for (int q = 0; q < g; ++q) base += s_part[q * ep + e];
    for (int b0 = b_lo; b0 < b_hi; b0 += 8) {
      int c[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = b0 + i < b_hi ? tile_counts[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (b0 + i < b_hi) tile_counts[(size_t)(b0 + i) * E + e] = base;
        base += c[i];
      }
    }
  }
  // expert tid's total (tid < ep: the thread of its first range)
  int run = 0;
  if (tid < E) {
    for (int q = 0; q < P; ++q) run += s_part[q * ep + tid];
    counts[tid] = run;
  }
  s_total[tid] = tid < E ? run : 0;
  __syncthreads();
  for (int off = 512; off >= 1; off >>= 1) {
    if (tid < off) s_total[tid] += s_total[tid + off];
    __syncthreads();
  }
  const long long A = s_total[0];
  long long C = LLONG_MAX;
  if (cf > 0.0f) C = (long long)ceil((double)cf * (double)A / (double)E);
  const int kept = tid < E ? (int)(run < C ? run : C) : 0;
  // inclusive Hillis-Steele scan of kept over the block
  s_scan[tid] = kept;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = tid >= off ? s_scan[tid - off] : 0;
    __syncthreads();
    s_scan[tid] += add;
    __syncthreads();
  }
  if (tid < E) offsets[tid + 1] = s_scan[tid];
  if (tid == 0) {
    offsets[0] = 0;
    const int R = s_scan[E - 1];
    if (num_dropped) *num_dropped = (int32_t)(A - R);
    *cap_out = C > INT_MAX ? INT_MAX : (int32_t)C;
  }
}

// This wave's expert ids of tile slots [wbase, wbase + kSlotsPerWave), all
// loads issued before any is used; ids outside [0, E) become -1.
__device__ __forceinline__ void load_wave_ids(const int32_t* __restrict__ ids, int wbase,
                                              int total_slots, int E, int lane,
                                              int (&ev)[kRankChunks], bool& bad) {
#pragma unroll
  for (int i = 0; i < kRankChunks; ++i) {
    const int s = wbase + 64 * i + lane;
    ev[i] = s < total_slots ? ids[s] : -1;
  }
#pragma unroll
  for (int i = 0; i < kRankChunks; ++i) {
    if (ev[i] < -1 || ev[i] >= E) bad = true;
    if (ev[i] < 0 || ev[i] >= E) ev[i] = -1;
  }
}

// Bits that tell the ids of a chunk apart: the ids are -1 or in [0, E), so
// ceil(log2 E) bits plus one (where -1 has a 1 and every valid id a 0).
__device__ __forceinline__ int id_bits(int E) { return (E <= 1 ? 0 : 32 - __clz(E - 1)) + 1; }

// Walks the wave's slots in order, 64 at a time: a slot's rank in its expert
// is the wave's running base (wcnt_wave[e], advanced by the last lane holding
// e) plus the equal experts in earlier lanes of the chunk; ranks at or beyond
// the capacity drop the slot.  The lanes holding a lane's id are the AND, over
// the id's bits, of the ballot of lanes sharing that bit.
__device__ __forceinline__ void scatter_wave(const int (&ev)[kRankChunks], int wbase,
                                             int total_slots, int k_max, int lane, int ebits,
                                             int* __restrict__ wcnt_wave,
                                             const int* __restrict__ s_off, int cap,
                                             int32_t* __restrict__ row_of_slot,
                                             int32_t* __restrict__ row_token) {
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int i = 0; i < kRankChunks; ++i) {
    if (wbase + 64 * i >= total_slots) break;
    const int s = wbase + 64 * i + lane;
    const int e = ev[i];
    uint64_t same = ~0ull;
    for (int b = 0; b < ebits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t on = __ballot(bit);
      same &= bit ? on : ~on;
    }
    const int before = __popcll(same & below);
    const int after = __popcll(same & ~below) - 1;
    if (e >= 0) {
      const int rank = wcnt_wave[e] + before;
      const int row = rank < cap ? s_off[e] + rank : -1;
      row_of_slot[s] = row;
      if (row >= 0) row_token[row] = s / k_max;
    } else if (s < total_slots) {
      row_of_slot[s] = -1;
    }
    if (e >= 0 && after == 0) wcnt_wave[e] += before + 1;
  }
}

__global__ __launch_bounds__(256) void k_rank_scatter(const int32_t* __restrict__ ids,
                                                      int total_slots, int k_max, int E,
                                                      const int32_t* __restrict__ tile_base,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ cap_p,
                                                      int32_t* __restrict__ row_of_slot,
                                                      int32_t* __restrict__ row_token) {
  __shared__ int wcnt[kRankWaves][kMaxExperts];
  __shared__ int s_off[kMaxExperts];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tile = blockIdx.x;
  const int wbase = tile * kDispatchTileSlots + wave * kSlotsPerWave;

  int ev[kRankChunks];
  bool bad = false;  // reported by k_tile_hist
  load_wave_ids(ids, wbase, total_slots, E, lane, ev, bad);
  for (int i = threadIdx.x; i < kRankWaves * kMaxExperts; i += blockDim.x)
    (&wcnt[0][0])[i] = 0;
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_off[e] = offsets[e];
  const int cap = *cap_p;
  __syncthreads();
  // per-wave histogram of the wave's sub-tile
#pragma unroll
  for (int i = 0; i < kRankChunks; ++i)
    if (ev[i] >= 0) atomicAdd(&wcnt[wave][ev[i]], 1);
  __syncthreads();
  // running base of each wave = tile base + counts of the earlier waves
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = tile_base[(size_t)tile * E + e];
    for (int w = 0; w < kRankWaves; ++w) {
      const int c = wcnt[w][e];
      wcnt[w][e] = run;
      run += c;
    }
  }
  __syncthreads();
  scatter_wave(ev, wbase, total_slots, k_max, lane, id_bits(E), wcnt[wave], s_off, cap, row_of_slot,
               row_token);
}

// The whole of S3-S5 in one block when all slots fit one tile (decode-sized
// batches): histogram, capacity, offsets and drops, then the ranks -- the
// three launches of the tiled path in one.
__global__ __launch_bounds__(256) void k_dispatch_single(const int32_t* __restrict__ ids,
                                                         int total_slots, int k_max, int E,
                                                         float cf, int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ num_dropped,
                                                         int32_t* __restrict__ row_of_slot,
                                                         int32_t* __restrict__ row_token,
                                                         uint32_t* __restrict__ flags) {
  __shared__ int wcnt[kRankWaves][kMaxExperts];
  __shared__ int s_off[kMaxExperts];
  __shared__ int s_scan[256];
  __shared__ long long s_sum[256];
  __shared__ int s_bad;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wbase = wave * kSlotsPerWave;

  int ev[kRankChunks];
  bool bad = false;
  load_wave_ids(ids, wbase, total_slots, E, lane, ev, bad);
  for (int i = tid; i < kRankWaves * kMaxExperts; i += blockDim.x) (&wcnt[0][0])[i] = 0;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (bad) s_bad = 1;
#pragma unroll
  for (int i = 0; i < kRankChunks; ++i)
    if (ev[i] >= 0) atomicAdd(&wcnt[wave][ev[i]], 1);
  __syncthreads();
  // thread t owns experts 2t and 2t+1: counts, then wave bases (tile base 0)
  int cnt2[2] = {0, 0};
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = 2 * tid + q;
    if (e < E) {
      int run = 0;
      for (int w = 0; w < kRankWaves; ++w) {
        const int c = wcnt[w][e];
        wcnt[w][e] = run;
        run += c;
      }
      cnt2[q] = run;
      counts[e] = run;
    }
  }
  // A = total routed slots; capacity C = ceil(cf * A / E), as in k_scan_capacity
  s_sum[tid] = (long long)cnt2[0] + cnt2[1];
  __syncthreads();
  for (int off = 128; off >= 1; off >>= 1) {
    if (tid < off) s_sum[tid] += s_sum[tid + off];
    __syncthreads();
  }
  const long long A = s_sum[0];
  long long C = LLONG_MAX;
  if (cf > 0.0f) C = (long long)ceil((double)cf * (double)A / (double)E);
  const int k0 = (int)(cnt2[0] < C ? cnt2[0] : C), k1 = (int)(cnt2[1] < C ? cnt2[1] : C);
  // inclusive scan of the per-thread kept sums
  s_scan[tid] = k0 + k1;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int add = tid >= off ? s_scan[tid - off] : 0;
    __syncthreads();
    s_scan[tid] += add;
    __syncthreads();
  }
  const int excl = s_scan[tid] - k0 - k1;
  if (2 * tid < E) {
    s_off[2 * tid] = excl;
    offsets[2 * tid + 1] = excl + k0;
  }
  if (2 * tid + 1 < E) {
    s_off[2 * tid + 1] = excl + k0;
    offsets[2 * tid + 2] = excl + k0 + k1;
  }
  if (tid == 0) {
    offsets[0] = 0;
    if (num_dropped) *num_dropped = (int32_t)(A - s_scan[255]);
  }
  __syncthreads();
  if (tid == 0 && s_bad) atomicOr(flags, (uint32_t)MOE_FLAG_BAD_EXPERT);
  const int cap = C > INT_MAX ? INT_MAX : (int)C;
  scatter_wave(ev, wbase, total_slots, k_max, lane, id_bits(E), wcnt[wave], s_off, cap, row_of_slot,
               row_token);
}

// One wavefront per permuted row; 16-byte vector copies.
__global__ __launch_bounds__(256) void k_gather(const uint4* __restrict__ x,
                                                const int32_t* __restrict__ row_token,
                                                const int32_t* __restrict__ offsets, int E,
                                                int row_vecs, uint4* __restrict__ x_perm) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= offsets[E]) return;
  const uint4* src = x + (size_t)row_token[r] * row_vecs;
  uint4* dst = x_perm + (size_t)r * row_vecs;
  for (int i = lane; i < row_vecs; i += 64) dst[i] = src[i];
}

// Row tiles per expert, in expert order: experts with at least split_rows kept
// rows go to the big list in tiles of bm_big rows, the others to the small
// list in tiles of bm_small rows.
__global__ __launch_bounds__(512) void k_build_sched(const int32_t* __restrict__ offsets, int E,
                                                     int bm_big, int bm_small, int split_rows,
                                                     int tail_rows,
                                                     MTile* __restrict__ sched_big, int max_big,
                                                     MTile* __restrict__ sched_small, int max_small,
                                                     int32_t* __restrict__ count) {
  __shared__ int s_big[512], s_small[512];
  const int tid = threadIdx.x;
  // an expert with at least split_rows rows takes big tiles; smaller experts
  // take small tiles only.  A remainder of at most tail_rows rows past a big
  // expert's last full tile goes to small tiles too: a big tile would cost
  // its full height for a few rows, and a small tile streams the expert's
  // weights beside the big tiles.  (With 32-row small tiles, tails measured
  // slower on the skewed layers, whose small experts already load the memory
  // system; with 64-row tiles a tail is one stream, and those layers gain
  // 0.5-2.4%.)
  int r0 = 0, kept = 0, nb = 0, ns = 0, sbeg = 0;
  if (tid < E) {
    r0 = offsets[tid];
    kept = offsets[tid + 1] - r0;
  }
  if (tid < E) {
    if (kept >= split_rows) {
      nb = kept / bm_big;
      const int rem = kept - nb * bm_big;
      if (rem > 0 && rem <= tail_rows) {
        sbeg = nb * bm_big;
        ns = (rem + bm_small - 1) / bm_small;
      } else if (rem > 0) {
        nb += 1;
      }
    } else {
      ns = (kept + bm_small - 1) / bm_small;
    }
  }
  s_big[tid] = nb;
  s_small[tid] = ns;
  __syncthreads();
  for (int off = 1; off < 512; off <<= 1) {
    const int ab = tid >= off ? s_big[tid - off] : 0;
    const int as = tid >= off ? s_small[tid - off] : 0;
    __syncthreads();
    s_big[tid] += ab;
    s_small[tid] += as;
    __syncthreads();
  }
  for (int i = 0; i < nb; ++i) {
    const int slot = s_big[tid] - nb + i;
    if (slot < max_big) {
      MTile m;
      m.expert = tid;
      m.row0 = r0 + i * bm_big;
      m.rows = min(bm_big, kept - i * bm_big);
      m.pad = 0;
      sched_big[slot] = m;
    }
  }
  for (int i = 0; i < ns; ++i) {
    const int slot = s_small[tid] - ns + i;
    if (slot < max_small) {
      MTile m;
      m.expert = tid;
      m.row0 = r0 + sbeg + i * bm_small;
      m.rows = min(bm_small, kept - sbeg - i * bm_small);
      m.pad = 0;
      sched_small[slot] = m;
    }
  }
  if (tid == 511) {
    count[0] = min(s_big[511], max_big);
    count[1] = min(s_small[511], max_small);
  }
}

// Replica of each slot: the r-th slot of logical expert e (token-major, r =
// its row in the uncapped dispatch minus offsets[e]) takes replica r mod n_e.
__global__ __launch_bounds__(256) void k_map_replicas(const int32_t* __restrict__ ids,
                                                      int total_slots, int E,
                                                      const int32_t* __restrict__ row_of_slot,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ rep_off,
                                                      const int32_t* __restrict__ rep_exp,
                                                      int num_physical,
                                                      int32_t* __restrict__ phys,
                                                      uint32_t* __restrict__ flags) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= total_slots) return;
  const int e = ids[s];
  int p = -1;
  if (e >= 0 && e < E) {
    const int r0 = rep_off[e], n = rep_off[e + 1] - r0;
    bool bad = n <= 0;
    if (!bad) {
      const int rank = row_of_slot[s] - offsets[e];
      p = rep_exp[r0 + rank % n];
      if (p < 0 || p >= num_physical) {
        p = -1;
        bad = true;
      }
    }
    if (bad) atomicOr(flags, (uint32_t)MOE_FLAG_BAD_REPLICA);
  }
  phys[s] = p;
}

__global__ void k_clear_flags(uint32_t* flags) { *flags = 0u; }

}  // namespace

hipError_t launch_clear_flags(uint32_t* flags, hipStream_t st) {
  hipLaunchKernelGGL(k_clear_flags, dim3(1), dim3(1), 0, st, flags);
  return hipGetLastError();
}

hipError_t launch_dispatch(const moe_shape& s, const int32_t* ids, int32_t* counts,
                           int32_t* offsets, int32_t* row_of_slot, int32_t* row_token,
                           int32_t* num_dropped, int32_t* tile_counts, int n_tiles,
                           uint32_t* flags, hipStream_t st) {
  const int total = s.num_tokens * s.top_k;
  const int E = s.num_experts;
  if (n_tiles == 1) {
    hipLaunchKernelGGL(k_dispatch_single, dim3(1), dim3(256), 0, st, ids, total, s.top_k, E,
                       s.capacity_factor, counts, offsets, num_dropped, row_of_slot, row_token,
                       flags);
    return hipGetLastError();
  }
  // the capacity is kept right after the tile table
  int32_t* cap = tile_counts + (size_t)n_tiles * E;
  hipLaunchKernelGGL(k_tile_hist, dim3(n_tiles), dim3(256), 0, st, ids, total, E, tile_counts,
                     flags);
  hipLaunchKernelGGL(k_scan_capacity, dim3(1), dim3(1024), 0, st, tile_counts, n_tiles, E,
                     s.capacity_factor, counts, offsets, num_dropped, cap);
  hipLaunchKernelGGL(k_rank_scatter, dim3(n_tiles), dim3(256), 0, st, ids, total, s.top_k, E,
                     tile_counts, offsets, cap, row_of_slot, row_token);
  return hipGetLastError();
}

hipError_t launch_map_replicas(const moe_shape& s, const int32_t* ids, const int32_t* row_of_slot,
                               const int32_t* offsets, const int32_t* rep_off,
                               const int32_t* rep_exp, int num_physical, int32_t* phys,
                               uint32_t* flags, hipStream_t st) {
  const int total = s.num_tokens * s.top_k;
  hipLaunchKernelGGL(k_map_replicas, dim3((total + 255) / 256), dim3(256), 0, st, ids, total,
                     s.num_experts, row_of_slot, offsets, rep_off, rep_exp, num_physical, phys,
                     flags);
  return hipGetLastError();
}

hipError_t launch_gather(const moe_shape& s, const void* x, const int32_t* row_token,
                         const int32_t* offsets, void* x_perm, hipStream_t st) {
  const int eb = s.act_dtype == MOE_BF16 ? 2 : 4;
  const int row_vecs = s.hidden * eb / 16;
  const int max_rows = s.num_tokens * s.top_k;
  hipLaunchKernelGGL(k_gather, dim3((max_rows + 3) / 4), dim3(256), 0, st,
                     static_cast<const uint4*>(x), row_token, offsets, s.num_experts, row_vecs,
                     static_cast<uint4*>(x_perm));
  return hipGetLastError();
}

hipError_t launch_build_schedule(const int32_t* offsets, int E, const GemmPlan& plan,
                                 MTile* sched_big, int max_big, MTile* sched_small, int max_small,
                                 int32_t* count, hipStream_t st) {
  hipLaunchKernelGGL(k_build_sched, dim3(1), dim3(512), 0, st, offsets, E, plan.bm_big,
                     plan.bm_small, plan.split_rows, plan.tail_rows, sched_big, max_big, sched_small,
                     max_small, count);
  return hipGetLastError();
}

}  // namespace moe
