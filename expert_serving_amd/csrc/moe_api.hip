// Host side of the C ABI: argument validation (pure host code, before any HIP
// call), workspace planning, and the launch sequence of each entry point.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "moe_internal.h"

namespace moe {

namespace {
thread_local int32_t g_last_hip_error = 0;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int elem_bytes(int dt) { return dt == MOE_BF16 ? 2 : 4; }

moe_status hip_fail(hipError_t e) {
  g_last_hip_error = (int32_t)e;
  return MOE_ERR_HIP;
}

// Shape rules shared by every entry point.
moe_status check_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_INVALID_ARG;
  if (s->num_tokens < 0 || s->hidden <= 0 || s->intermediate <= 0) return MOE_ERR_INVALID_ARG;
  if (s->num_experts < 1) return MOE_ERR_INVALID_ARG;
  if (s->num_experts > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (s->top_k < 1 || s->top_k > s->num_experts) return MOE_ERR_INVALID_ARG;
  if (s->top_k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
  if (s->score != MOE_SCORE_SOFTMAX && s->score != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (s->renormalize != 0 && s->renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(s->routed_scale) || !std::isfinite(s->capacity_factor))
    return MOE_ERR_INVALID_ARG;
  if (s->act_dtype != MOE_F32 && s->act_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (s->out_dtype != MOE_F32 && s->out_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (s->down_dtype != 0 && s->down_dtype != s->act_dtype && s->down_dtype != MOE_F16)
    return MOE_ERR_INVALID_ARG;
  if (s->down_dtype == MOE_F16 && s->act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (s->shared_intermediate < 0) return MOE_ERR_INVALID_ARG;
  if (s->num_groups < 1) return MOE_ERR_INVALID_ARG;
  if (s->num_groups > 1) {
    if (s->num_experts % s->num_groups != 0) return MOE_ERR_INVALID_ARG;
    if (s->num_groups > 64) return MOE_ERR_UNSUPPORTED;
    if (s->topk_groups < 1 || s->topk_groups > s->num_groups) return MOE_ERR_INVALID_ARG;
    const int gs = s->num_experts / s->num_groups;
    if (s->group_topn < 0 || s->group_topn > gs) return MOE_ERR_INVALID_ARG;
    if (s->group_topn > 8) return MOE_ERR_UNSUPPORTED;
    // the kept groups must hold at least k experts
    if ((long long)s->topk_groups * gs < s->top_k) return MOE_ERR_INVALID_ARG;
  }
  const int mult = s->act_dtype == MOE_BF16 ? 64 : 4;
  if (s->hidden % mult || s->intermediate % mult || s->shared_intermediate % mult)
    return MOE_ERR_UNSUPPORTED;
  // slot and row indices are int32, and so are the GEMM's element offsets
  // inside x (gathered rows) and inside one expert's weight matrix
  if ((long long)s->num_tokens * s->top_k > (long long)INT_MAX / 2) return MOE_ERR_UNSUPPORTED;
  const long long H = s->hidden;
  if ((long long)s->num_tokens * H > (long long)INT_MAX) return MOE_ERR_UNSUPPORTED;
  if ((long long)s->intermediate * H > (long long)INT_MAX ||
      (long long)s->shared_intermediate * H > (long long)INT_MAX ||
      (long long)s->num_experts * H > (long long)INT_MAX)
    return MOE_ERR_UNSUPPORTED;
  if ((long long)s->num_tokens * s->num_experts > (long long)INT_MAX) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

#define MOE_TRY(expr)                      \
  do {                                     \
    const moe_status st_ = (expr);         \
    if (st_ != MOE_OK) return st_;         \
  } while (0)
#define MOE_HIP(expr)                      \
  do {                                     \
    const hipError_t e_ = (expr);          \
    if (e_ != hipSuccess) return hip_fail(e_); \
  } while (0)

inline moe_status need(const void* p) {
  if (!p) return MOE_ERR_INVALID_ARG;
  return aligned16(p) ? MOE_OK : MOE_ERR_INVALID_ARG;
}
// 4-byte aligned index/float arrays
inline moe_status need4(const void* p) {
  if (!p) return MOE_ERR_INVALID_ARG;
  return (reinterpret_cast<uintptr_t>(p) & 3u) ? MOE_ERR_INVALID_ARG : MOE_OK;
}
inline moe_status opt4(const void* p) { return p ? need4(p) : MOE_OK; }

// MXFP8 layers: bf16 x and router, 128-column groups along every K
moe_status check_mx_shape(const moe_shape* s) {
  MOE_TRY(check_shape(s));
  if (s->act_dtype != MOE_BF16 || s->down_dtype == MOE_F16) return MOE_ERR_UNSUPPORTED;
  if (s->hidden % 128 || s->intermediate % 128 || s->shared_intermediate % 128)
    return MOE_ERR_UNSUPPORTED;
  // the scale-word strides of the weights (E*I rows of gate/up, E*H of down;
  // E*H is bounded by check_shape) are int32 inside the kernels
  if ((long long)s->num_experts * s->intermediate > (long long)INT_MAX) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_mx_ffn(const moe_mxfp8_ffn* w) {
  if (!w) return MOE_ERR_INVALID_ARG;
  MOE_TRY(need(w->gate));
  MOE_TRY(need(w->gate_scales));
  MOE_TRY(need(w->up));
  MOE_TRY(need(w->up_scales));
  MOE_TRY(need(w->down));
  MOE_TRY(need(w->down_scales));
  return MOE_OK;
}

// Records the stage event when the caller asked for it.
inline hipError_t stage_mark(const moe_debug* d, int stage, bool start, hipStream_t st) {
  if (!d) return hipSuccess;
  void* ev = start ? d->stage_start[stage] : d->stage_stop[stage];
  return ev ? hipEventRecord(static_cast<hipEvent_t>(ev), st) : hipSuccess;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

}  // namespace

// remainder rows of a big expert that ride on one small tile
constexpr int kTailRows = 64;
// compute units of one MI355X (8 XCDs x 32)
constexpr int kComputeUnits = 256;
// K-split parts of the down projection for a batch of a token or two
constexpr int kFewKsplit = 8;
// most K-split parts of a gate/up projection (16 keeps each part >= 4 stages
// of 64 for H >= 4096)
constexpr int kGateUpKsplitMax = 16;

int router_parts(const moe_shape& s) {
  if (s.act_dtype != MOE_BF16 || router_skinny_supported(s)) return 1;
  // the MFMA router's tiles (as run_router picks them); K in 64-wide stages
  const int tiles128 = (s.num_tokens + 127) / 128 * ((s.num_experts + 127) / 128);
  const int bm = tiles128 >= 64 ? 128 : 32;
  const long long blocks = (long long)((s.num_tokens + bm - 1) / bm) * ((s.num_experts + 127) / 128);
  return (blocks < kComputeUnits && s.hidden / 64 >= 16) ? 2 : 1;
}

GemmPlan choose_gemm_plan(const moe_shape& s) {
  GemmPlan p;
  const long long slots = (long long)s.num_tokens * s.top_k;
  // rows per expert if the load were even
  const long long avg = slots / (s.num_experts > 0 ? s.num_experts : 1);
  p.bm_big = 256;
  p.bm_small = 32;
  if (s.act_dtype == MOE_F32) {
    p.bm_big = p.bm_small = 32;  // the fp32 kernel's tile height
    p.split_rows = 0;
  } else if (avg < 64) {
    p.split_rows = 0x7fffffff;   // every expert small: weight-streaming 32-row tiles
  } else {
    // both classes, in one interleaved launch for bf16 and MXFP8 layers:
    // experts with >= 128 kept rows on 256-row tiles, the rest on 64-row
    // tiles.  Even with a large average load, skew and capacity drops leave
    // many experts with a few rows (Qwen3-shaped layer: 87 of 120), and an
    // empty small class costs only a few idle blocks.
    p.split_rows = 128;
    p.bm_small = kMergedSmallRows;
    // a big expert's last rows, when few, ride on small tiles: a 256-row
    // tile costs its full height in MFMA time, while the small tiles stream
    // the expert's weights beside the big tiles of the same launch
    p.tail_rows = kTailRows;
  }
  return p;
}

namespace {

// Rows-per-tile bounds of the two schedules (worst case over any routing).
void tile_bounds(const moe_shape& s, const GemmPlan& gp, int& max_big, int& max_small) {
  const size_t E = (size_t)s.num_experts, slots = (size_t)s.num_tokens * s.top_k;
  max_big = gp.has_big() ? (int)(slots / (size_t)gp.bm_big + E + 1) : 0;
  // small tiles: every expert's rows, or, with big tiles, an expert's rows
  // below split_rows (small expert) or its tail of at most tail_rows
  const size_t bound = slots / (size_t)gp.bm_small + E + 1;
  if (!gp.has_small()) {
    max_small = 0;
  } else if (!gp.has_big()) {
    max_small = (int)bound;
  } else {
    const size_t per_expert =
        ((size_t)std::max(gp.split_rows - 1, gp.tail_rows) + gp.bm_small - 1) / gp.bm_small;
    max_small = (int)std::min(bound, per_expert * E);
  }
}

// Experts that can hold rows when there are few slots, one 32-row tile each
long long few_row_tiles(const moe_shape& s) {
  const long long slots = (long long)s.num_tokens * s.top_k;
  return std::max<long long>(std::min<long long>(slots, (long long)s.num_experts), (slots + 31) / 32);
}

// K-split parts of the layer's down projection (partial y sums, added by
// the combine; 1 = none).
int down_parts(const moe_shape& s, const GemmPlan& gp, int max_tiles_small, bool mx) {
  if (s.act_dtype != MOE_BF16) return 1;
  const long long slots = (long long)s.num_tokens * s.top_k;
  const long long H = s.hidden, I = s.intermediate;
  if (!gp.has_big() && gp.has_small()) {
    // Decode-sized layers (every expert small, few 32-row tiles) leave most
    // compute units idle in the down projection; splitting its long K (= I)
    // gives every unit weight rows to stream.
    const int bnb = (mx || I >= kDown8MinK) ? 256 : 128;  // column tile of the 32-row down kernels
    const long long blocks = (long long)max_tiles_small * ((H + bnb - 1) / bnb);
    if (blocks <= 0 || blocks >= 512) return 1;
    const long long few_blocks = std::min<long long>(max_tiles_small, few_row_tiles(s)) * ((H + bnb - 1) / bnb);
    int want;
    if (slots < s.num_experts && few_blocks > 0 && few_blocks <= kComputeUnits / 2) {
      // fewer routed slots than experts (a few tokens): up to eight parts,
      // so most compute units stream a slice of the few weight matrices;
      // the combine's extra reads are a few KB per part
      want = (int)std::min<long long>(kFewKsplit, (4LL * kComputeUnits + few_blocks - 1) / few_blocks);
    } else {
      // two parts measured best for both formats on the Mixtral-shaped
      // decode layer (four or eight: slower)
      want = (int)std::min<long long>(2, 1024 / blocks);
    }
    return std::max(1, std::min(want, (int)(I / 64) / 4));
  }
  if (gp.has_big() && gp.bm_big == 256) {
    // Few 256-row down tiles with a long K (at an even load, at most a
    // quarter of the compute units busy) leave the rest idle for the whole
    // projection.  Measured on the Mixtral-shaped layer (K = 14336): 256
    // and 512 tokens 5-10% faster per layer, both formats; at 1024 and more
    // tokens the combine's extra reads cost about what the down projection
    // gains, so no split there.
    const long long big = ((slots + 255) / 256) * ((H + 255) / 256);
    const int stages = (int)(I / 128);  // 128-element stages (MXFP8); bf16 has twice as many
    if (big > 0 && big <= kComputeUnits / 4 && stages >= 64) {
      const int want = (int)std::min<long long>(4, (4LL * kComputeUnits + big - 1) / big);
      return std::max(1, std::min(want, stages / 32));
    }
  }
  return 1;
}

// K-split parts of a gate/up projection on 32 x 256 weight-streaming tiles
// that number `blocks` (fp32 partial gate and up sums, added and passed
// through SwiGLU by a reduction kernel; 1 = none).  At most half the
// compute units busy: about one block per unit.  Measured on the
// DeepSeek-V3-shaped layer: one token 0.473 -> 0.289 ms, two 0.546 -> 0.359
// ms (the shared expert's gate/up ran 8 blocks); Mixtral-shaped single
// token unchanged (0.156 -> 0.155 ms).  `rounds`: also split when the blocks
// fill between one and two rounds of the compute units, the rounds under
// three quarters full: the split (up to 4) that fills them best
// (Mixtral-shaped layer, 3 tokens: 336 blocks, 3 parts, 0.373 -> 0.332 ms
// bf16, 0.215 -> 0.200 ms MXFP8; fuller rounds are HBM-bound already and a
// split only adds work: 4 tokens, 448 blocks in 4 parts, 2-14% slower).
int gate_up_parts(long long blocks, int stages, bool rounds) {
  if (blocks <= 0) return 1;
  if (blocks <= kComputeUnits / 2)
    return std::max(1, std::min<int>((int)std::min<long long>(kGateUpKsplitMax,
                                                              (kComputeUnits + blocks - 1) / blocks),
                                     stages / 4));
  if (!rounds || blocks > 2LL * kComputeUnits) return 1;
  auto util = [&](long long ks) {
    const long long n = blocks * ks, r = (n + kComputeUnits - 1) / kComputeUnits;
    return (double)n / (double)(r * kComputeUnits);
  };
  if (util(1) >= 0.75) return 1;
  int best = 1;
  for (int ks = 2; ks <= 4 && ks <= stages / 4; ++ks)
    if (util(ks) > util(best) + 1e-9) best = ks;
  return best;
}

}  // namespace

WsLayout plan_workspace(const moe_shape& s, bool mx) {
  WsLayout w{};
  const size_t T = (size_t)s.num_tokens, E = (size_t)s.num_experts, k = (size_t)s.top_k;
  const size_t H = (size_t)s.hidden, I = (size_t)s.intermediate, Is = (size_t)s.shared_intermediate;
  const size_t eb = mx ? 1 : (size_t)elem_bytes(s.act_dtype);  // bytes of an h element
  const size_t slots = T * k;
  const GemmPlan gp = choose_gemm_plan(s);
  w.n_dispatch_tiles = (int)((slots + kDispatchTileSlots - 1) / kDispatchTileSlots);
  tile_bounds(s, gp, w.max_tiles_big, w.max_tiles_small);
  w.ksplit = down_parts(s, gp, w.max_tiles_small, mx);
  w.ks_gu = w.ks_gus = 1;
  if (s.act_dtype == MOE_BF16) {
    const int stages = (int)(H / (mx ? 128 : 64));  // K stages (128 codes, or 64 bf16 elements)
    // routed experts of a token or a few (decode plans only)
    if (!gp.has_big() && gp.has_small())
      w.ks_gu = gate_up_parts(std::min<long long>(w.max_tiles_small, few_row_tiles(s)) *
                                  (long long)((I + 255) / 256),
                              stages, true);
    // the shared expert of a few tokens (32-row tiles below 128 tokens)
    if (Is > 0 && T < 128)
      w.ks_gus = gate_up_parts((long long)((T + 31) / 32) * (long long)((Is + 255) / 256), stages, false);
  }
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at_ = o;
    o = align_up(o + bytes, 256);
    return at_;
  };
  w.flags = take(256);
  w.logits = take(T * E * 4);
  w.logits_parts = take(router_parts(s) > 1 ? (size_t)router_parts(s) * T * E * 4 : 0);
  w.ids = take(slots * 4);
  w.gates = take(slots * 4);
  w.counts = take(E * 4);
  w.offsets = take((E + 1) * 4);
  w.tile_counts = take(((size_t)w.n_dispatch_tiles * E + 4) * 4);  // + capacity word
  w.row_of_slot = take(slots * 4);
  w.row_token = take(slots * 4);
  w.num_dropped = take(16);
  w.sched_big = take((size_t)w.max_tiles_big * sizeof(MTile));
  w.sched_small = take((size_t)w.max_tiles_small * sizeof(MTile));
  w.sched_count = take(16);
  w.h = take(slots * I * eb);
  w.y = take((size_t)w.ksplit * slots * H * 4);
  w.hs = take(T * Is * eb);
  w.ys = take(Is ? T * H * 4 : 0);
  w.gu_parts = take(std::max(w.ks_gu > 1 ? 2 * (size_t)w.ks_gu * slots * I * 4 : 0,
                             w.ks_gus > 1 ? 2 * (size_t)w.ks_gus * T * Is * 4 : 0));
  w.ep_tile_counts = take((size_t)ep_tiles((int)T) * kMaxRanks * 4);
  if (mx) {
    w.xq = take(T * H);
    w.xsc = take(T * H / 32);
    w.xscp = take(slots * H / 32);
    w.hsc = take(slots * I / 32);
    w.hssc = take(T * Is / 32);
  }
  w.total = o;
  return w;
}

// ---- shared launch sequences --------------------------------------------------
namespace {

// S1; also clears the device flag word (inside the skinny router's launch).
// With router_parts(s) = 2 the logits come as two partial sums at
// parts_buf (T*E floats apart), which the route kernel adds and stores at
// `logits`; `parts` reports which.
moe_status run_router(const moe_shape& s, const void* x, const void* w_router, const float* bias,
                      float* logits, uint32_t* flags, hipStream_t st, float* parts_buf, int& parts) {
  parts = 1;
  if (router_skinny_supported(s)) {
    MOE_HIP(launch_router_skinny(s, x, w_router, bias, logits, flags, st));
    return MOE_OK;
  }
  MOE_HIP(launch_clear_flags(flags, st));
  if (router_parts(s) > 1) {
    parts = router_parts(s);
    const int tiles128 = (s.num_tokens + 127) / 128 * ((s.num_experts + 127) / 128);
    const int bm = tiles128 >= 64 ? 128 : 32;
    MOE_HIP(launch_gemm_plain(s.act_dtype, bm, false, x, s.hidden, w_router, s.num_experts, s.hidden,
                              bias, parts_buf, s.num_experts, nullptr, nullptr, 0, s.num_tokens, st, parts,
                              (long long)s.num_tokens * s.num_experts));
    return MOE_OK;
  }
  // 128-row tiles (8-wave blocks) once there are enough of them to spread
  // over the chip; 32-row tiles for few tokens
  const int tiles128 = (s.num_tokens + 127) / 128 * ((s.num_experts + 127) / 128);
  const int bm = tiles128 >= 64 ? 128 : 32;
  MOE_HIP(launch_gemm_plain(s.act_dtype, bm, false, x, s.hidden, w_router, s.num_experts, s.hidden,
                            bias, logits, s.num_experts, nullptr, nullptr, 0, s.num_tokens, st));
  return MOE_OK;
}

// a_rows (nullable): rows of x_perm are x[a_rows[r]] (gather fused into the GEMM)
// y_half: y is fp16 (a layer call's internal rows; ksplit must be 1)
moe_status run_ffn(const moe_shape& s, const void* x_perm, const int32_t* a_rows,
                   const int32_t* offsets, const void* w_gate, const void* w_up,
                   const void* w_down, void* y, void* ws,
                   const WsLayout& L, hipStream_t st, const moe_debug* dbg = nullptr,
                   int ksplit = 1, bool y_half = false) {
  const GemmPlan gp = choose_gemm_plan(s);
  const int E = s.num_experts, H = s.hidden, I = s.intermediate;
  MTile* sb = at<MTile>(ws, L.sched_big);
  MTile* ss = at<MTile>(ws, L.sched_small);
  int32_t* cnt = at<int32_t>(ws, L.sched_count);
  uint32_t* flags = at<uint32_t>(ws, L.flags);
  MOE_HIP(launch_build_schedule(offsets, E, gp, sb, L.max_tiles_big, ss, L.max_tiles_small, cnt,
                                st));
  void* h = at<void>(ws, L.h);
  // skewed loads (both tile classes) on bf16: one interleaved launch per
  // projection, so small experts stream weights while big ones run MFMAs
  const bool merged = gp.has_big() && gp.has_small() && s.act_dtype == MOE_BF16 &&
                      gp.bm_big == 256 && gp.bm_small == kMergedSmallRows;
  MOE_HIP(stage_mark(dbg, MOE_STAGE_GATE_UP, true, st));
  if (merged) {
    MOE_HIP(launch_gemm_gateup2(x_perm, a_rows, H, w_gate, w_up, I, H, h, I, sb, cnt, L.max_tiles_big, ss,
                                cnt + 1, L.max_tiles_small, flags, st));
  } else {
    if (gp.has_big())
      MOE_HIP(launch_gemm_gateup(s.act_dtype, gp.bm_big, x_perm, a_rows, H, w_gate, w_up, I, H, h,
                                 I, sb, cnt, L.max_tiles_big, 0, flags, st));
    if (gp.has_small() && L.ks_gu > 1) {
      float* parts = at<float>(ws, L.gu_parts);
      const long long pe = (long long)s.num_tokens * s.top_k * I;
      MOE_HIP(launch_gemm_gateup_parts(x_perm, a_rows, H, w_gate, w_up, I, H, parts, ss, cnt + 1,
                                       L.max_tiles_small, 0, L.ks_gu, pe, st));
      MOE_HIP(launch_swiglu_parts(parts, L.ks_gu, pe, I, offsets + E, 0, s.num_tokens * s.top_k, h, I,
                                  flags, st));
    } else if (gp.has_small()) {
      MOE_HIP(launch_gemm_gateup(s.act_dtype, gp.bm_small, x_perm, a_rows, H, w_gate, w_up, I, H,
                                 h, I, ss, cnt + 1, L.max_tiles_small, 0, flags, st));
    }
  }
  MOE_HIP(stage_mark(dbg, MOE_STAGE_GATE_UP, false, st));
  MOE_HIP(stage_mark(dbg, MOE_STAGE_DOWN, true, st));
  const bool w16 = s.down_dtype == MOE_F16;
  if (merged) {
    MOE_HIP(launch_gemm_down2(h, I, w_down, H, I, y, H, sb, cnt, L.max_tiles_big, ss, cnt + 1,
                              L.max_tiles_small, st, ksplit, (long long)s.num_tokens * s.top_k * H, y_half,
                              flags, w16));
  } else {
    if (gp.has_big())
      MOE_HIP(launch_gemm_plain(s.act_dtype, gp.bm_big, true, h, I, w_down, H, I, nullptr, y, H, sb,
                                cnt, L.max_tiles_big, 0, st, 1, 0, y_half, flags, w16));
    if (gp.has_small())
      MOE_HIP(launch_gemm_plain(s.act_dtype, gp.bm_small, true, h, I, w_down, H, I, nullptr, y, H,
                                ss, cnt + 1, L.max_tiles_small, 0, st, gp.has_big() ? 1 : ksplit,
                                (long long)s.num_tokens * s.top_k * H, y_half, flags, w16));
  }
  MOE_HIP(stage_mark(dbg, MOE_STAGE_DOWN, false, st));
  return MOE_OK;
}

// MXFP8 S7-S8: xq rows (gathered through a_rows when given) with scales of
// stride xs_stride; h codes and scales (stride T*top_k) in the workspace.
moe_status run_ffn_mx(const moe_shape& s, const void* xq, const int32_t* a_rows,
                      const uint8_t* xsc, int xs_stride, const int32_t* offsets,
                      const moe_mxfp8_ffn& w, float* y, void* ws, const WsLayout& L,
                      hipStream_t st, const moe_debug* dbg = nullptr, int ksplit = 1,
                      bool sa_direct = false) {
  const GemmPlan gp = choose_gemm_plan(s);
  const int E = s.num_experts, H = s.hidden, I = s.intermediate;
  const int slots = s.num_tokens * s.top_k;
  MTile* sb = at<MTile>(ws, L.sched_big);
  MTile* ss = at<MTile>(ws, L.sched_small);
  int32_t* cnt = at<int32_t>(ws, L.sched_count);
  uint32_t* flags = at<uint32_t>(ws, L.flags);
  MOE_HIP(launch_build_schedule(offsets, E, gp, sb, L.max_tiles_big, ss, L.max_tiles_small, cnt,
                                st));
  void* h = at<void>(ws, L.h);
  uint8_t* hsc = at<uint8_t>(ws, L.hsc);
  const auto gsc = w.gate_scales, usc = w.up_scales, dsc = w.down_scales;
  const bool merged = gp.has_big() && gp.has_small() && gp.bm_big == 256 && gp.bm_small == kMergedSmallRows;
  MOE_HIP(stage_mark(dbg, MOE_STAGE_GATE_UP, true, st));
  if (merged) {
    MOE_HIP(launch_gemm_gateup_mx2(xq, a_rows, xsc, xs_stride, w.gate, gsc, w.up, usc, E * I, I, H, h, hsc,
                                   slots, sb, cnt, L.max_tiles_big, ss, cnt + 1, L.max_tiles_small, flags,
                                   st, sa_direct));
  } else {
    if (gp.has_big())
      MOE_HIP(launch_gemm_gateup_mx(gp.bm_big, xq, a_rows, xsc, xs_stride, w.gate, gsc, w.up, usc,
                                    E * I, I, H, h, hsc, slots, sb, cnt, L.max_tiles_big, 0, flags,
                                    st, sa_direct));
    if (gp.has_small() && L.ks_gu > 1) {
      float* parts = at<float>(ws, L.gu_parts);
      const long long pe = (long long)slots * I;
      MOE_HIP(launch_gemm_gateup_mx_parts(xq, a_rows, xsc, xs_stride, w.gate, gsc, w.up, usc, E * I, I, H,
                                          parts, ss, cnt + 1, L.max_tiles_small, 0, L.ks_gu, pe, st,
                                          sa_direct));
      MOE_HIP(launch_swiglu_parts_mx(parts, L.ks_gu, pe, I, offsets + E, 0, slots, h, hsc, slots, flags,
                                     st));
    } else if (gp.has_small()) {
      MOE_HIP(launch_gemm_gateup_mx(gp.bm_small, xq, a_rows, xsc, xs_stride, w.gate, gsc, w.up, usc,
                                    E * I, I, H, h, hsc, slots, ss, cnt + 1, L.max_tiles_small, 0,
                                    flags, st, sa_direct));
    }
  }
  MOE_HIP(stage_mark(dbg, MOE_STAGE_GATE_UP, false, st));
  MOE_HIP(stage_mark(dbg, MOE_STAGE_DOWN, true, st));
  if (merged) {
    MOE_HIP(launch_gemm_down_mx2(h, hsc, slots, w.down, dsc, E * H, H, I, y, H, sb, cnt, L.max_tiles_big, ss,
                                 cnt + 1, L.max_tiles_small, st, ksplit, (long long)slots * H));
  } else {
    if (gp.has_big())
      MOE_HIP(launch_gemm_down_mx(gp.bm_big, h, hsc, slots, w.down, dsc, E * H, H, I, y, H, sb, cnt,
                                  L.max_tiles_big, 0, st));
    if (gp.has_small())
      MOE_HIP(launch_gemm_down_mx(gp.bm_small, h, hsc, slots, w.down, dsc, E * H, H, I, y, H, ss,
                                  cnt + 1, L.max_tiles_small, 0, st, gp.has_big() ? 1 : ksplit,
                                  (long long)slots * H));
  }
  MOE_HIP(stage_mark(dbg, MOE_STAGE_DOWN, false, st));
  return MOE_OK;
}

// MXFP8 shared expert on all T quantised rows (scales of stride T)
moe_status run_shared_mx(const moe_shape& s, const void* xq, const uint8_t* xsc,
                         const moe_mxfp8_ffn& w, void* ws, const WsLayout& L, hipStream_t st) {
  const int T = s.num_tokens, H = s.hidden, Is = s.shared_intermediate;
  const int bm = T >= 2048 ? 256 : (T >= 128 ? 128 : 32);
  void* hs = at<void>(ws, L.hs);
  uint8_t* hssc = at<uint8_t>(ws, L.hssc);
  float* ys = at<float>(ws, L.ys);
  if (L.ks_gus > 1 && bm == 32) {
    float* parts = at<float>(ws, L.gu_parts);
    const long long pe = (long long)T * Is;
    MOE_HIP(launch_gemm_gateup_mx_parts(xq, nullptr, xsc, T, w.gate, w.gate_scales, w.up, w.up_scales, Is,
                                        Is, H, parts, nullptr, nullptr, 0, T, L.ks_gus, pe, st, false));
    MOE_HIP(launch_swiglu_parts_mx(parts, L.ks_gus, pe, Is, nullptr, T, T, hs, hssc, T,
                                   at<uint32_t>(ws, L.flags), st));
  } else {
    MOE_HIP(launch_gemm_gateup_mx(bm, xq, nullptr, xsc, T, w.gate, w.gate_scales, w.up, w.up_scales,
                                  Is, Is, H, hs, hssc, T, nullptr, nullptr, 0, T,
                                  at<uint32_t>(ws, L.flags), st));
  }
  MOE_HIP(launch_gemm_down_mx(bm, hs, hssc, T, w.down, w.down_scales, H, H, Is, ys, H, nullptr,
                              nullptr, 0, T, st));
  return MOE_OK;
}

moe_status run_shared(const moe_shape& s, const void* x, const void* wsg, const void* wsu,
                      const void* wsd, void* ws, const WsLayout& L, hipStream_t st, bool y_half = false) {
  const int T = s.num_tokens, H = s.hidden, Is = s.shared_intermediate;
  const int bm = s.act_dtype == MOE_F32 ? 32 : (T >= 2048 ? 256 : (T >= 128 ? 128 : 32));
  void* hs = at<void>(ws, L.hs);
  float* ys = at<float>(ws, L.ys);
  if (L.ks_gus > 1 && bm == 32) {
    float* parts = at<float>(ws, L.gu_parts);
    const long long pe = (long long)T * Is;
    MOE_HIP(launch_gemm_gateup_parts(x, nullptr, H, wsg, wsu, Is, H, parts, nullptr, nullptr, 0, T,
                                     L.ks_gus, pe, st));
    MOE_HIP(launch_swiglu_parts(parts, L.ks_gus, pe, Is, nullptr, T, T, hs, Is, at<uint32_t>(ws, L.flags),
                                st));
  } else {
    MOE_HIP(launch_gemm_gateup(s.act_dtype, bm, x, nullptr, H, wsg, wsu, Is, H, hs, Is, nullptr,
                               nullptr, 0, T, at<uint32_t>(ws, L.flags), st));
  }
  MOE_HIP(launch_gemm_plain(s.act_dtype, bm, true, hs, Is, wsd, H, Is, nullptr, ys, H, nullptr,
                            nullptr, 0, T, st, 1, 0, y_half, at<uint32_t>(ws, L.flags), s.down_dtype == MOE_F16));
  return MOE_OK;
}

// ---- the layer, shared by the workspace and the no-allocation entry points ---

// Host checks of moe_layer_forward's arguments (all but the workspace).
moe_status check_layer_args(const moe_shape* shape, const void* x, const void* w_router,
                            const float* router_bias, const int32_t* k_per_token, const void* w_gate,
                            const void* w_up, const void* w_down, const void* ws_gate,
                            const void* ws_up, const void* ws_down, const void* out,
                            const moe_debug* dbg) {
  MOE_TRY(check_shape(shape));
  const moe_shape& s = *shape;
  MOE_TRY(need(x));
  MOE_TRY(need(w_router));
  MOE_TRY(opt4(router_bias));
  MOE_TRY(opt4(k_per_token));
  MOE_TRY(need(w_gate));
  MOE_TRY(need(w_up));
  MOE_TRY(need(w_down));
  if (s.shared_intermediate > 0) {
    MOE_TRY(need(ws_gate));
    MOE_TRY(need(ws_up));
    MOE_TRY(need(ws_down));
  }
  MOE_TRY(need(out));
  if (dbg) {
    if (dbg->logits) MOE_TRY(need(dbg->logits));
    MOE_TRY(opt4(dbg->topk_ids));
    MOE_TRY(opt4(dbg->topk_gates));
    MOE_TRY(opt4(dbg->expert_counts));
    MOE_TRY(opt4(dbg->expert_offsets));
    MOE_TRY(opt4(dbg->row_of_slot));
    MOE_TRY(opt4(dbg->num_dropped));
    MOE_TRY(opt4(dbg->row_token));
  }
  return MOE_OK;
}

// S1-S10 on validated arguments, T > 0, with workspace `ws` laid out as L.
moe_status run_layer(const moe_shape& s, const void* x, const void* w_router, const float* router_bias,
                     const int32_t* k_per_token, const void* w_gate, const void* w_up,
                     const void* w_down, const void* ws_gate, const void* ws_up, const void* ws_down,
                     void* out, const moe_debug* dbg, void* ws, const WsLayout& L, hipStream_t st) {
  float* logits = (dbg && dbg->logits) ? dbg->logits : at<float>(ws, L.logits);
  int32_t* ids = (dbg && dbg->topk_ids) ? dbg->topk_ids : at<int32_t>(ws, L.ids);
  float* gates = (dbg && dbg->topk_gates) ? dbg->topk_gates : at<float>(ws, L.gates);
  int32_t* counts = (dbg && dbg->expert_counts) ? dbg->expert_counts : at<int32_t>(ws, L.counts);
  int32_t* offsets = (dbg && dbg->expert_offsets) ? dbg->expert_offsets : at<int32_t>(ws, L.offsets);
  int32_t* ros = (dbg && dbg->row_of_slot) ? dbg->row_of_slot : at<int32_t>(ws, L.row_of_slot);
  int32_t* nd = (dbg && dbg->num_dropped) ? dbg->num_dropped : at<int32_t>(ws, L.num_dropped);
  uint32_t* flags = at<uint32_t>(ws, L.flags);
  int32_t* row_token = (dbg && dbg->row_token) ? dbg->row_token : at<int32_t>(ws, L.row_token);
  void* y = at<void>(ws, L.y);
  // The expert outputs y (and the shared expert's) go to the combine as fp16
  // in bf16 layers whose down projection is not split (half the bytes of the
  // round trip through HBM); a split projection's partial sums stay fp32.
  const bool y_half = s.act_dtype == MOE_BF16 && L.ksplit == 1;

  MOE_HIP(stage_mark(dbg, MOE_STAGE_ROUTER, true, st));
  int rparts = 1;
  float* lparts = at<float>(ws, L.logits_parts);
  MOE_TRY(run_router(s, x, w_router, router_bias, logits, flags, st, lparts, rparts));
  MOE_HIP(stage_mark(dbg, MOE_STAGE_ROUTER, false, st));
  MOE_HIP(stage_mark(dbg, MOE_STAGE_ROUTE, true, st));
  MOE_HIP(launch_route_topk(s, rparts > 1 ? lparts : logits, k_per_token, ids, gates, flags, st, rparts,
                            (long long)s.num_tokens * s.num_experts, rparts > 1 ? logits : nullptr));
  MOE_HIP(stage_mark(dbg, MOE_STAGE_ROUTE, false, st));
  MOE_HIP(stage_mark(dbg, MOE_STAGE_DISPATCH, true, st));
  MOE_HIP(launch_dispatch(s, ids, counts, offsets, ros, row_token, nd,
                          at<int32_t>(ws, L.tile_counts), L.n_dispatch_tiles, flags, st));
  MOE_HIP(stage_mark(dbg, MOE_STAGE_DISPATCH, false, st));
  // S6 gather: fused into the gate/up GEMM's tile loads (rows x[row_token[r]])
  MOE_HIP(stage_mark(dbg, MOE_STAGE_GATHER, true, st));
  MOE_HIP(stage_mark(dbg, MOE_STAGE_GATHER, false, st));
  MOE_TRY(run_ffn(s, x, row_token, offsets, w_gate, w_up, w_down, y, ws, L, st, dbg, L.ksplit, y_half));
  const void* ys = nullptr;
  MOE_HIP(stage_mark(dbg, MOE_STAGE_SHARED, true, st));
  if (s.shared_intermediate > 0) {
    MOE_TRY(run_shared(s, x, ws_gate, ws_up, ws_down, ws, L, st, y_half));
    ys = at<void>(ws, L.ys);
  }
  MOE_HIP(stage_mark(dbg, MOE_STAGE_SHARED, false, st));
  MOE_HIP(stage_mark(dbg, MOE_STAGE_COMBINE, true, st));
  MOE_HIP(launch_combine(s, y, ros, gates, ys, out, st, L.ksplit,
                         (long long)s.num_tokens * s.top_k * s.hidden, y_half));
  MOE_HIP(stage_mark(dbg, MOE_STAGE_COMBINE, false, st));
  return MOE_OK;
}

// ---- workspace of the no-allocation entry point --------------------------------
// One array in the library's own device memory; every GPU the library runs on
// holds its own copy (placed when the code object is loaded on that GPU) until
// the process ends.  In host code `scratch` names a host-side stand-in, never
// the device array: host code uses only the address hipGetSymbolAddress gives
// for the current device, kept per device below.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxScratchDevices];

// Device address of the current GPU's `scratch`, looked up on the first call
// on that GPU (with it current) and kept.
moe_status static_scratch(void** ptr) {
  int dev = -1;
  MOE_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxScratchDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    MOE_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return MOE_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *ptr = g_scratch_dev[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

moe_status moe_workspace_size(const moe_shape* shape, size_t* bytes) {
  MOE_TRY(check_shape(shape));
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = plan_workspace(*shape).total;
  return MOE_OK;
}

moe_status moe_route_topk(const moe_shape* shape, const void* x, const void* w_router,
                          const float* router_bias, const float* logits_in, float* logits_out,
                          const int32_t* k_per_token, int32_t* topk_ids, float* topk_gates,
                          void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_shape(shape));
  const moe_shape& s = *shape;
  if (logits_in) {
    MOE_TRY(need4(logits_in));
  } else {
    MOE_TRY(need(x));
    MOE_TRY(need(w_router));
    MOE_TRY(opt4(router_bias));
  }
  if (logits_out) MOE_TRY(need(logits_out));
  MOE_TRY(opt4(k_per_token));
  MOE_TRY(need4(topk_ids));
  MOE_TRY(need4(topk_gates));
  MOE_TRY(need(ws));
  const WsLayout L = plan_workspace(s);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (s.num_tokens == 0) return MOE_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t* flags = at<uint32_t>(ws, L.flags);
  const float* logits = logits_in;
  int rparts = 1;
  float* sum_out = nullptr;
  if (!logits) {
    float* lo = logits_out ? logits_out : at<float>(ws, L.logits);
    float* pb = at<float>(ws, L.logits_parts);
    MOE_TRY(run_router(s, x, w_router, router_bias, lo, flags, st, pb, rparts));
    logits = rparts > 1 ? pb : lo;
    sum_out = rparts > 1 ? lo : nullptr;
  } else {
    MOE_HIP(launch_clear_flags(flags, st));
  }
  MOE_HIP(launch_route_topk(s, logits, k_per_token, topk_ids, topk_gates, flags, st, rparts,
                            (long long)s.num_tokens * s.num_experts, sum_out));
  return MOE_OK;
}

moe_status moe_dispatch(const moe_shape* shape, const void* x, const int32_t* topk_ids,
                        int32_t* expert_counts, int32_t* expert_offsets, int32_t* row_of_slot,
                        int32_t* row_token, int32_t* num_dropped, void* x_perm, void* ws,
                        size_t ws_bytes, void* stream) {
  MOE_TRY(check_shape(shape));
  const moe_shape& s = *shape;
  MOE_TRY(need4(topk_ids));
  MOE_TRY(need4(expert_counts));
  MOE_TRY(need4(expert_offsets));
  MOE_TRY(need4(row_of_slot));
  MOE_TRY(need4(row_token));
  MOE_TRY(opt4(num_dropped));
  if ((x == nullptr) != (x_perm == nullptr)) return MOE_ERR_INVALID_ARG;
  if (x) {
    MOE_TRY(need(x));
    MOE_TRY(need(x_perm));
  }
  MOE_TRY(need(ws));
  const WsLayout L = plan_workspace(s);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (s.num_tokens == 0) return MOE_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  MOE_HIP(launch_clear_flags(at<uint32_t>(ws, L.flags), st));
  MOE_HIP(launch_dispatch(s, topk_ids, expert_counts, expert_offsets, row_of_slot, row_token,
                          num_dropped, at<int32_t>(ws, L.tile_counts), L.n_dispatch_tiles,
                          at<uint32_t>(ws, L.flags), st));
  if (x) MOE_HIP(launch_gather(s, x, row_token, expert_offsets, x_perm, st));
  return MOE_OK;
}

moe_status moe_map_replicas(const moe_shape* shape, const int32_t* topk_ids,
                            const int32_t* replica_offsets, const int32_t* replica_experts,
                            int32_t num_physical, int32_t* phys_ids, void* ws, size_t ws_bytes,
                            void* stream) {
  MOE_TRY(check_shape(shape));
  MOE_TRY(need4(topk_ids));
  MOE_TRY(need4(replica_offsets));
  MOE_TRY(need4(replica_experts));
  MOE_TRY(need4(phys_ids));
  MOE_TRY(need(ws));
  if (num_physical < 1) return MOE_ERR_INVALID_ARG;
  // the token-major rank of every slot comes from an uncapped dispatch of the
  // logical ids into the workspace
  moe_shape s = *shape;
  s.capacity_factor = 0.0f;
  const WsLayout L = plan_workspace(s);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (s.num_tokens == 0) return MOE_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t* flags = at<uint32_t>(ws, L.flags);
  int32_t* counts = at<int32_t>(ws, L.counts);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* ros = at<int32_t>(ws, L.row_of_slot);
  MOE_HIP(launch_clear_flags(flags, st));
  MOE_HIP(launch_dispatch(s, topk_ids, counts, offsets, ros, at<int32_t>(ws, L.row_token),
                          at<int32_t>(ws, L.num_dropped), at<int32_t>(ws, L.tile_counts),
                          L.n_dispatch_tiles, flags, st));
  MOE_HIP(launch_map_replicas(s, topk_ids, ros, offsets, replica_offsets, replica_experts,
                              num_physical, phys_ids, flags, st));
  return MOE_OK;
}

moe_status moe_grouped_ffn(const moe_shape* shape, const void* x_perm,
                           const int32_t* expert_offsets, const void* w_gate, const void* w_up,
                           const void* w_down, float* y_perm, void* ws, size_t ws_bytes,
                           void* stream) {
  MOE_TRY(check_shape(shape));
  const moe_shape& s = *shape;
  MOE_TRY(need(x_perm));
  MOE_TRY(need4(expert_offsets));
  MOE_TRY(need(w_gate));
  MOE_TRY(need(w_up));
  MOE_TRY(need(w_down));
  MOE_TRY(need(y_perm));
  MOE_TRY(need(ws));
  const WsLayout L = plan_workspace(s);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (s.num_tokens == 0) return MOE_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  MOE_HIP(launch_clear_flags(at<uint32_t>(ws, L.flags), st));
  return run_ffn(s, x_perm, nullptr, expert_offsets, w_gate, w_up, w_down, y_perm, ws, L, st);
}

moe_status moe_combine(const moe_shape* shape, const float* y_perm, const int32_t* row_of_slot,
                       const float* topk_gates, const float* y_shared, void* out, void* stream) {
  MOE_TRY(check_shape(shape));
  const moe_shape& s = *shape;
  MOE_TRY(need(y_perm));
  MOE_TRY(need4(row_of_slot));
  MOE_TRY(need4(topk_gates));
  if (y_shared) MOE_TRY(need(y_shared));
  MOE_TRY(need(out));
  if (s.num_tokens == 0) return MOE_OK;
  MOE_HIP(launch_combine(s, y_perm, row_of_slot, topk_gates, y_shared, out,
                         static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_layer_forward(const moe_shape* shape, const void* x, const void* w_router,
                             const float* router_bias, const int32_t* k_per_token,
                             const void* w_gate, const void* w_up, const void* w_down,
                             const void* ws_gate, const void* ws_up, const void* ws_down,
                             void* out, const moe_debug* dbg, void* ws, size_t ws_bytes,
                             void* stream) {
  MOE_TRY(check_layer_args(shape, x, w_router, router_bias, k_per_token, w_gate, w_up, w_down, ws_gate,
                           ws_up, ws_down, out, dbg));
  MOE_TRY(need(ws));
  const WsLayout L = plan_workspace(*shape);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (shape->num_tokens == 0) return MOE_OK;
  return run_layer(*shape, x, w_router, router_bias, k_per_token, w_gate, w_up, w_down, ws_gate, ws_up,
                   ws_down, out, dbg, ws, L, static_cast<hipStream_t>(stream));
}

moe_status moe_layer_forward_noalloc(const moe_shape* shape, const void* x, const void* w_router,
                                     const float* router_bias, const int32_t* k_per_token,
                                     const void* w_gate, const void* w_up, const void* w_down,
                                     const void* ws_gate, const void* ws_up, const void* ws_down,
                                     void* out, const moe_debug* dbg, void* stream) {
  MOE_TRY(check_layer_args(shape, x, w_router, router_bias, k_per_token, w_gate, w_up, w_down, ws_gate,
                           ws_up, ws_down, out, dbg));
  const WsLayout L = plan_workspace(*shape);
  if (L.total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  if (shape->num_tokens == 0) return MOE_OK;
  void* ws = nullptr;
  MOE_TRY(static_scratch(&ws));
  return run_layer(*shape, x, w_router, router_bias, k_per_token, w_gate, w_up, w_down, ws_gate, ws_up,
                   ws_down, out, dbg, ws, L, static_cast<hipStream_t>(stream));
}

moe_status moe_ep_dispatch_layout(const moe_shape* shape, int32_t num_ranks, const int32_t* topk_ids,
                                  const float* topk_gates, const void* x, int32_t* rank_counts,
                                  int32_t* rank_offsets, int32_t* send_token, int32_t* send_ids,
                                  float* send_gates, int32_t* slot_send_pos, void* send_x, void* ws,
                                  size_t ws_bytes, void* stream) {
  MOE_TRY(check_shape(shape));
  const moe_shape& s = *shape;
  if (num_ranks < 1) return MOE_ERR_INVALID_ARG;
  if (num_ranks > kMaxRanks) return MOE_ERR_UNSUPPORTED;
  if (s.num_experts % num_ranks != 0) return MOE_ERR_INVALID_ARG;
  MOE_TRY(need4(topk_ids));
  MOE_TRY(need4(topk_gates));
  MOE_TRY(need4(rank_counts));
  MOE_TRY(need4(rank_offsets));
  MOE_TRY(need4(send_token));
  MOE_TRY(need4(send_ids));
  MOE_TRY(need4(send_gates));
  MOE_TRY(need4(slot_send_pos));
  if ((x == nullptr) != (send_x == nullptr)) return MOE_ERR_INVALID_ARG;
  if (x) {
    MOE_TRY(need(x));
    MOE_TRY(need(send_x));
  }
  MOE_TRY(need(ws));
  const WsLayout L = plan_workspace(s);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (s.num_tokens == 0) return MOE_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t* flags = at<uint32_t>(ws, L.flags);
  MOE_HIP(launch_clear_flags(flags, st));
  MOE_HIP(launch_ep_layout(s, num_ranks, topk_ids, topk_gates, rank_counts, rank_offsets, send_token, send_ids,
                           send_gates, slot_send_pos, at<int32_t>(ws, L.ep_tile_counts), flags, st));
  if (x) {
    // the payload: row p of the send buffer is x[send_token[p]] for p below
    // rank_offsets[G] (the gather of the dispatch, over G groups of rows)
    moe_shape g = s;
    g.num_experts = num_ranks;
    g.top_k = std::min(s.top_k, (int32_t)num_ranks);
    MOE_HIP(launch_gather(g, x, send_token, rank_offsets, send_x, st));
  }
  return MOE_OK;
}

moe_status moe_ep_combine(const moe_shape* shape, int32_t num_ranks, const float* partial,
                          const int32_t* slot_send_pos, const float* y_shared, void* out, void* stream) {
  MOE_TRY(check_shape(shape));
  const moe_shape& s = *shape;
  if (num_ranks < 1) return MOE_ERR_INVALID_ARG;
  if (num_ranks > kMaxRanks) return MOE_ERR_UNSUPPORTED;
  if (s.num_experts % num_ranks != 0) return MOE_ERR_INVALID_ARG;
  MOE_TRY(need(partial));
  MOE_TRY(need4(slot_send_pos));
  if (y_shared) MOE_TRY(need(y_shared));
  MOE_TRY(need(out));
  if (s.num_tokens == 0) return MOE_OK;
  MOE_HIP(launch_ep_combine(s, num_ranks, partial, slot_send_pos, y_shared, out, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_quantize_mxfp8(int32_t rows, int32_t cols, int32_t src_dtype, const void* src,
                              int32_t scale_stride, void* codes, uint8_t* scales, void* stream) {
  if (rows < 0 || cols <= 0 || scale_stride < rows) return MOE_ERR_INVALID_ARG;
  if (src_dtype != MOE_BF16 && src_dtype != MOE_F32) return MOE_ERR_INVALID_ARG;
  if (cols % 128) return MOE_ERR_UNSUPPORTED;
  MOE_TRY(need(src));
  MOE_TRY(need(codes));
  MOE_TRY(need(scales));
  if (rows == 0) return MOE_OK;
  MOE_HIP(launch_quant_mxfp8(src_dtype, src, rows, cols, scale_stride, static_cast<uint8_t*>(codes),
                             scales, nullptr, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_convert_bf16_to_f16(int64_t n, const void* src, void* dst, void* stream) {
  if (n < 0) return MOE_ERR_INVALID_ARG;
  if (n == 0) return MOE_OK;
  MOE_TRY(need(src));
  MOE_TRY(need(dst));
  MOE_HIP(launch_bf16_to_f16(src, dst, (long long)n, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_workspace_size_mxfp8(const moe_shape* shape, size_t* bytes) {
  MOE_TRY(check_mx_shape(shape));
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = plan_workspace(*shape, true).total;
  return MOE_OK;
}

moe_status moe_grouped_ffn_mxfp8(const moe_shape* shape, const void* x_codes,
                                 const uint8_t* x_scales, int32_t x_scale_stride,
                                 const int32_t* expert_offsets, const moe_mxfp8_ffn* experts,
                                 float* y_perm, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_mx_shape(shape));
  const moe_shape& s = *shape;
  MOE_TRY(need(x_codes));
  MOE_TRY(need(x_scales));
  MOE_TRY(need4(expert_offsets));
  MOE_TRY(check_mx_ffn(experts));
  MOE_TRY(need(y_perm));
  MOE_TRY(need(ws));
  if ((long long)x_scale_stride < (long long)s.num_tokens * s.top_k) return MOE_ERR_INVALID_ARG;
  const WsLayout L = plan_workspace(s, true);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (s.num_tokens == 0) return MOE_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  MOE_HIP(launch_clear_flags(at<uint32_t>(ws, L.flags), st));
  return run_ffn_mx(s, x_codes, nullptr, x_scales, x_scale_stride, expert_offsets, *experts,
                    y_perm, ws, L, st);
}

moe_status moe_layer_forward_mxfp8(const moe_shape* shape, const void* x, const void* w_router,
                                   const float* router_bias, const int32_t* k_per_token,
                                   const moe_mxfp8_ffn* experts, const moe_mxfp8_ffn* shared,
                                   void* out, const moe_debug* dbg, void* ws, size_t ws_bytes,
                                   void* stream) {
  MOE_TRY(check_mx_shape(shape));
  const moe_shape& s = *shape;
  MOE_TRY(need(x));
  MOE_TRY(need(w_router));
  MOE_TRY(opt4(router_bias));
  MOE_TRY(opt4(k_per_token));
  MOE_TRY(check_mx_ffn(experts));
  if (s.shared_intermediate > 0) MOE_TRY(check_mx_ffn(shared));
  MOE_TRY(need(out));
  MOE_TRY(need(ws));
  if (dbg) {
    if (dbg->logits) MOE_TRY(need(dbg->logits));
    MOE_TRY(opt4(dbg->topk_ids));
    MOE_TRY(opt4(dbg->topk_gates));
    MOE_TRY(opt4(dbg->expert_counts));
    MOE_TRY(opt4(dbg->expert_offsets));
    MOE_TRY(opt4(dbg->row_of_slot));
    MOE_TRY(opt4(dbg->num_dropped));
    MOE_TRY(opt4(dbg->row_token));
  }
  const WsLayout L = plan_workspace(s, true);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (s.num_tokens == 0) return MOE_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int T = s.num_tokens;

  float* logits = (dbg && dbg->logits) ? dbg->logits : at<float>(ws, L.logits);
  int32_t* ids = (dbg && dbg->topk_ids) ? dbg->topk_ids : at<int32_t>(ws, L.ids);
  float* gates = (dbg && dbg->topk_gates) ? dbg->topk_gates : at<float>(ws, L.gates);
  int32_t* counts = (dbg && dbg->expert_counts) ? dbg->expert_counts : at<int32_t>(ws, L.counts);
  int32_t* offsets = (dbg && dbg->expert_offsets) ? dbg->expert_offsets : at<int32_t>(ws, L.offsets);
  int32_t* ros = (dbg && dbg->row_of_slot) ? dbg->row_of_slot : at<int32_t>(ws, L.row_of_slot);
  int32_t* nd = (dbg && dbg->num_dropped) ? dbg->num_dropped : at<int32_t>(ws, L.num_dropped);
  uint32_t* flags = at<uint32_t>(ws, L.flags);
  int32_t* row_token = (dbg && dbg->row_token) ? dbg->row_token : at<int32_t>(ws, L.row_token);
  float* y = at<float>(ws, L.y);
  uint8_t* xq = at<uint8_t>(ws, L.xq);
  uint8_t* xsc = at<uint8_t>(ws, L.xsc);

  MOE_HIP(stage_mark(dbg, MOE_STAGE_ROUTER, true, st));
  int rparts = 1;
  float* lparts = at<float>(ws, L.logits_parts);
  MOE_TRY(run_router(s, x, w_router, router_bias, logits, flags, st, lparts, rparts));
  MOE_HIP(stage_mark(dbg, MOE_STAGE_ROUTER, false, st));
  MOE_HIP(stage_mark(dbg, MOE_STAGE_ROUTE, true, st));
  MOE_HIP(launch_route_topk(s, rparts > 1 ? lparts : logits, k_per_token, ids, gates, flags, st, rparts,
                            (long long)s.num_tokens * s.num_experts, rparts > 1 ? logits : nullptr));
  MOE_HIP(stage_mark(dbg, MOE_STAGE_ROUTE, false, st));
  MOE_HIP(stage_mark(dbg, MOE_STAGE_DISPATCH, true, st));
  MOE_HIP(launch_dispatch(s, ids, counts, offsets, ros, row_token, nd,
                          at<int32_t>(ws, L.tile_counts), L.n_dispatch_tiles, flags, st));
  MOE_HIP(stage_mark(dbg, MOE_STAGE_DISPATCH, false, st));
  // S6: the dispatch payload is x quantised once per token; the row gather
  // itself is fused into the gate/up GEMM's tile loads, and the scale words
  // are also written in dispatch-row order for it
  MOE_HIP(stage_mark(dbg, MOE_STAGE_GATHER, true, st));
  uint8_t* xscp = at<uint8_t>(ws, L.xscp);
  MOE_HIP(launch_quant_mxfp8(MOE_BF16, x, T, s.hidden, T, xq, xsc, flags, st, ros, s.top_k, xscp,
                             T * s.top_k));
  MOE_HIP(stage_mark(dbg, MOE_STAGE_GATHER, false, st));
  MOE_TRY(run_ffn_mx(s, xq, row_token, xscp, T * s.top_k, offsets, *experts, y, ws, L, st, dbg, L.ksplit,
                     true));
  const float* ys = nullptr;
  MOE_HIP(stage_mark(dbg, MOE_STAGE_SHARED, true, st));
  if (s.shared_intermediate > 0) {
    MOE_TRY(run_shared_mx(s, xq, xsc, *shared, ws, L, st));
    ys = at<float>(ws, L.ys);
  }
  MOE_HIP(stage_mark(dbg, MOE_STAGE_SHARED, false, st));
  MOE_HIP(stage_mark(dbg, MOE_STAGE_COMBINE, true, st));
  MOE_HIP(launch_combine(s, y, ros, gates, ys, out, st, L.ksplit,
                         (long long)s.num_tokens * s.top_k * s.hidden));
  MOE_HIP(stage_mark(dbg, MOE_STAGE_COMBINE, false, st));
  return MOE_OK;
}

moe_status moe_group_score_sigmoid(const float* x, float* y, int64_t n, void* stream) {
  if (n < 0) return MOE_ERR_INVALID_ARG;
  if (n == 0) return MOE_OK;
  MOE_TRY(need4(x));
  MOE_TRY(need4(y));
  MOE_HIP(launch_logistic(x, y, (long long)n, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

const char* moe_status_string(moe_status status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or option";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

int32_t moe_last_hip_error(void) { return g_last_hip_error; }

moe_status moe_read_device_flags(const void* ws, void* stream, uint32_t* flags) {
  if (!ws || !flags) return MOE_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the flag word sits at offset 0 of every workspace layout
  MOE_HIP(hipMemcpyAsync(flags, ws, sizeof(uint32_t), hipMemcpyDeviceToHost, st));
  MOE_HIP(hipStreamSynchronize(st));
  return MOE_OK;
}

}  // extern "C"
