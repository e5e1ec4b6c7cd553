// Internal declarations of the gfx950 MoE-layer library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_mi355x.h"

namespace moe {

constexpr int kMaxExperts = 512;
constexpr int kMaxTopK = 16;
constexpr int kDispatchTileSlots = 1024;  // slots per dispatch tile (one block)

// One row-tile of the grouped GEMM: `rows` (1..BM) consecutive permuted rows
// starting at row0, all belonging to `expert`.
struct MTile {
  int expert;
  int row0;
  int rows;
  int pad;
};

// Byte offsets of every region inside the caller's workspace.
// MXFP8 layers add the quantised x (xq, scales xsc with stride T, and the
// same scales in dispatch-row order, xscp with stride T*top_k) and the scales
// of h (hsc, stride T*top_k) and of the shared expert's h (hssc, stride T);
// h and hs then hold one-byte codes.
struct WsLayout {
  size_t flags, logits, logits_parts, ids, gates, counts, offsets, tile_counts, row_of_slot, row_token,
      num_dropped, sched_big, sched_small, sched_count, h, y, hs, ys, xq, xsc, xscp, hsc, hssc, gu_parts,
      ep_tile_counts, total;
  int n_dispatch_tiles;
  // K-split of the layer's down projection (decode-sized layers, and layers
  // with few 256-row tiles): y holds ksplit partial sums,
  // part p at y + p * slots * H floats (1: no split)
  int ksplit;
  // K-split of the gate/up projection for a token or two (routed experts,
  // ks_gu) and of the shared expert's for a few tokens (ks_gus): fp32
  // partial gate and up sums in gu_parts, reduced by launch_swiglu_parts
  int ks_gu, ks_gus;
  int max_tiles_big, max_tiles_small;
};

// K from which the 32-row bf16 down tiles are 8-wave 32 x 256 blocks (else
// 4-wave 32 x 128)
constexpr int kDown8MinK = 2048;

// Row-tile height of the weight-streaming class in the interleaved
// (big + small) launches: an expert of up to 64 rows (or a big expert's tail
// of up to 64 rows) streams each weight tile once, where 32-row tiles would
// stream it once per 32 rows; the extra MFMA work stays hidden behind the
// weight stream.
constexpr int kMergedSmallRows = 64;

// K-split parts of the MFMA router (E > 32 and more tokens than the sliced
// vector router takes): 2 when its tiles keep fewer blocks than compute
// units busy, else 1
int router_parts(const moe_shape& s);

// GEMM tile configuration chosen by the host for a shape.
// Row tiling of the grouped GEMMs.  Experts with at least split_rows kept rows
// are cut into tiles of bm_big rows, the others into tiles of bm_small rows;
// each class gets its own tile list and launch (split_rows = 0: all big,
// INT_MAX: all small).
struct GemmPlan {
  int bm_big, bm_small, split_rows;
  int tail_rows = 0;  // remainder rows of a big expert placed on small tiles (0: none)
  bool has_big() const { return split_rows != 0x7fffffff; }
  bool has_small() const { return split_rows != 0; }
};

GemmPlan choose_gemm_plan(const moe_shape& s);
WsLayout plan_workspace(const moe_shape& s, bool mx = false);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---- launchers (each returns the launch status) ----------------------------
hipError_t launch_clear_flags(uint32_t* flags, hipStream_t st);

// logits may come in `parts` partial sums part_stride floats apart (a
// K-split router); their sums are then also written to sum_out (nullable)
hipError_t launch_route_topk(const moe_shape& s, const float* logits, const int32_t* k_per_token,
                             int32_t* ids, float* gates, uint32_t* flags, hipStream_t st, int parts = 1,
                             long long part_stride = 0, float* sum_out = nullptr);

hipError_t launch_logistic(const float* x, float* y, long long n, hipStream_t st);

// S1 without MFMA for bf16 layers with at most kRouterSkinnyMaxExperts experts
constexpr int kRouterSkinnyMaxExperts = 32;
// ... and for more experts up to this many tokens (slices of 8 experts; the
// 128-row MFMA router keeps only a few compute units busy below it)
constexpr int kRouterSlicedMaxTokens = 1024;
bool router_skinny_supported(const moe_shape& s);
// (flags, nullable: cleared to 0 by the launch)
hipError_t launch_router_skinny(const moe_shape& s, const void* x, const void* w_router,
                                const float* bias, float* logits, uint32_t* flags, hipStream_t st);

hipError_t launch_dispatch(const moe_shape& s, const int32_t* ids, int32_t* counts,
                           int32_t* offsets, int32_t* row_of_slot, int32_t* row_token,
                           int32_t* num_dropped, int32_t* tile_counts, int n_tiles,
                           uint32_t* flags, hipStream_t st);

// phys[s] = replica of slot s's expert (rank in the uncapped dispatch mod n_e)
hipError_t launch_map_replicas(const moe_shape& s, const int32_t* ids, const int32_t* row_of_slot,
                               const int32_t* offsets, const int32_t* rep_off,
                               const int32_t* rep_exp, int num_physical, int32_t* phys,
                               uint32_t* flags, hipStream_t st);

hipError_t launch_gather(const moe_shape& s, const void* x, const int32_t* row_token,
                         const int32_t* offsets, void* x_perm, hipStream_t st);

// Both tile lists (see GemmPlan); count[0] = big tiles, count[1] = small tiles.
hipError_t launch_build_schedule(const int32_t* offsets, int E, const GemmPlan& plan,
                                 MTile* sched_big, int max_big, MTile* sched_small, int max_small,
                                 int32_t* count, hipStream_t st);

// Grouped GEMMs.  `sched`/`count` give the row tiles; when sched == nullptr
// the rows [0, static_rows) form one group (expert 0) tiled statically.
// gate/up + SwiGLU: h[r][n] = silu(A[r].Bg[e][n]) * (A[r].Bu[e][n]); for bf16
// layers h is fp16 and values outside fp16's range set MOE_FLAG_H_RANGE
// a_rows (nullable): A row r is A[a_rows[r]] (the dispatch gather fused into
// the tile loads); else A is contiguous.
hipError_t launch_gemm_gateup(int dtype, int bm, const void* A, const int32_t* a_rows, int lda,
                              const void* Bg, const void* Bu, int N, int K, void* h, int ldh,
                              const MTile* sched, const int32_t* count, int max_tiles,
                              int static_rows, uint32_t* flags, hipStream_t st);
// gate/up on 32-row tiles with K split into ksplit ranges, no SwiGLU: range
// p's fp32 sums A.Bg^T at parts + p * part_elems and A.Bu^T at parts +
// (ksplit + p) * part_elems (rows of N floats); bf16 layers.
hipError_t launch_gemm_gateup_parts(const void* A, const int32_t* a_rows, int lda, const void* Bg,
                                    const void* Bu, int N, int K, float* parts, const MTile* sched,
                                    const int32_t* count, int max_tiles, int static_rows, int ksplit,
                                    long long part_elems, hipStream_t st);
// h[r] = fp16(silu(sum of gate parts) * sum of up parts) for r below *rows_dev
// (or static_rows when rows_dev is null); max_rows bounds the grid.
hipError_t launch_swiglu_parts(const float* parts, int nparts, long long part_elems, int N,
                               const int32_t* rows_dev, int static_rows, int max_rows, void* h, int ldh,
                               uint32_t* flags, hipStream_t st);
// The same two steps on MXFP8 operands; the reduction re-quantises h (codes
// [rows][N], scales as the MXFP8 gate/up epilogue writes them).
hipError_t launch_gemm_gateup_mx_parts(const void* A, const int32_t* a_rows, const uint8_t* sa,
                                       int sa_stride, const void* Bg, const uint8_t* sbg, const void* Bu,
                                       const uint8_t* sbu, int sb_stride, int N, int K, float* parts,
                                       const MTile* sched, const int32_t* count, int max_tiles,
                                       int static_rows, int ksplit, long long part_elems, hipStream_t st,
                                       bool sa_direct);
hipError_t launch_swiglu_parts_mx(const float* parts, int nparts, long long part_elems, int N,
                                  const int32_t* rows_dev, int static_rows, int max_rows, void* h,
                                  uint8_t* hsc, int hs_stride, uint32_t* flags, hipStream_t st);
// plain: Y[r][n] = A[r].B[e][n] (+ bias[n]), fp32 out.  a_is_h: A is the
// fp16 h of a bf16 layer (down projection), B is converted to fp16 on load.
// ksplit > 1 (32-row down tiles): K in ksplit ranges of whole 64-element
// stages, range p's partial sums at Y + p * part_elems.
// y_half (down projections of a bf16 layer, ksplit 1): Y is fp16 instead of
// fp32; values outside fp16's range set MOE_FLAG_Y_RANGE in flags.
hipError_t launch_gemm_plain(int dtype, int bm, bool a_is_h, const void* A, int lda,
                             const void* B, int N, int K, const float* bias, void* Y, int ldy,
                             const MTile* sched, const int32_t* count, int max_tiles,
                             int static_rows, hipStream_t st,
                             int ksplit = 1, long long part_elems = 0, bool y_half = false,
                             uint32_t* flags = nullptr, bool w16 = false);
// w16 (down projections, a_is_h): B holds fp16 weights (moe_convert_bf16_to_f16)
hipError_t launch_bf16_to_f16(const void* src, void* dst, long long n, hipStream_t st);

// MXFP8 path (codes + E8M0 scales; scale words group-major, see mxfp8.hip).
// Quantises rows x cols (cols a multiple of 128) of bf16 / fp32 src; inf/NaN
// inputs set MOE_FLAG_H_RANGE when flags is given.
// row_of_slot (nullable, [rows][k]): also write each scale byte at the
// dispatch rows of the row's kept slots in perm_scales (stride perm_stride).
hipError_t launch_quant_mxfp8(int src_dtype, const void* src, int rows, int cols, int stride,
                              uint8_t* codes, uint8_t* scales, uint32_t* flags, hipStream_t st,
                              const int32_t* row_of_slot = nullptr, int k = 0,
                              uint8_t* perm_scales = nullptr, int perm_stride = 0);
// gate/up + SwiGLU with h re-quantised to MXFP8; bm 256 / 128 / 32
hipError_t launch_gemm_gateup_mx(int bm, const void* A, const int32_t* a_rows, const uint8_t* sa,
                                 int sa_stride, const void* Bg, const uint8_t* sbg, const void* Bu,
                                 const uint8_t* sbu, int sb_stride, int N, int K, void* h,
                                 uint8_t* hsc, int hs_stride, const MTile* sched,
                                 const int32_t* count, int max_tiles, int static_rows,
                                 uint32_t* flags, hipStream_t st, bool sa_direct = false);
hipError_t launch_gemm_down_mx(int bm, const void* A, const uint8_t* hsc, int hs_stride,
                               const void* B, const uint8_t* sb, int sb_stride, int N, int K,
                               void* Y, int ldy, const MTile* sched, const int32_t* count,
                               int max_tiles, int static_rows, hipStream_t st,
                               int ksplit = 1, long long part_elems = 0, bool y_half = false,
                               uint32_t* flags = nullptr);

// Both row-tile classes (256-row and 32-row tiles of the big and small
// schedules) in one interleaved launch.
hipError_t launch_gemm_gateup2(const void* A, const int32_t* a_rows, int lda, const void* Bg,
                               const void* Bu, int N, int K, void* h, int ldh, const MTile* sb,
                               const int32_t* cb, int mb, const MTile* ss, const int32_t* cs, int ms,
                               uint32_t* flags, hipStream_t st);
hipError_t launch_gemm_down2(const void* A, int lda, const void* B, int N, int K, void* Y, int ldy,
                             const MTile* sb, const int32_t* cb, int mb, const MTile* ss,
                             const int32_t* cs, int ms, hipStream_t st, int ksplit = 1,
                             long long part_elems = 0, bool y_half = false, uint32_t* flags = nullptr,
                             bool w16 = false);
hipError_t launch_gemm_gateup_mx2(const void* A, const int32_t* a_rows, const uint8_t* sa, int sa_stride,
                                  const void* Bg, const uint8_t* sbg, const void* Bu, const uint8_t* sbu,
                                  int sb_stride, int N, int K, void* h, uint8_t* hsc, int hs_stride,
                                  const MTile* sb, const int32_t* cb, int mb, const MTile* ss,
                                  const int32_t* cs, int ms, uint32_t* flags, hipStream_t st,
                                  bool sa_direct = false);
hipError_t launch_gemm_down_mx2(const void* A, const uint8_t* hsc, int hs_stride, const void* B,
                                const uint8_t* sb_w, int sb_stride, int N, int K, void* Y, int ldy,
                                const MTile* sb, const int32_t* cb, int mb, const MTile* ss,
                                const int32_t* cs, int ms, hipStream_t st, int ksplit = 1,
                                long long part_elems = 0, bool y_half = false, uint32_t* flags = nullptr);

// Row-tile height the GEMM launchers use for a dtype and a requested height.
int gemm_tile_rows(int dtype, int bm_hint);

// ---- expert-parallel exchange over G virtual ranks (ep.hip) -----------------
constexpr int kMaxRanks = 64;
// 64-token tiles of the send-layout kernels (tile_counts: tiles x G ints)
int ep_tiles(int num_tokens);
hipError_t launch_ep_layout(const moe_shape& s, int G, const int32_t* ids, const float* gates,
                            int32_t* rank_counts, int32_t* rank_offsets, int32_t* send_token,
                            int32_t* send_ids, float* send_gates, int32_t* slot_send_pos,
                            int32_t* tile_counts, uint32_t* flags, hipStream_t st);
hipError_t launch_ep_combine(const moe_shape& s, int G, const float* partial, const int32_t* slot_send_pos,
                             const float* y_shared, void* out, hipStream_t st);

// y_half: y_perm and y_shared hold fp16 values (then parts must be 1)
hipError_t launch_combine(const moe_shape& s, const void* y_perm, const int32_t* row_of_slot,
                          const float* gates, const void* y_shared, void* out, hipStream_t st,
                          int parts = 1, long long part_stride = 0, bool y_half = false);

}  // namespace moe
