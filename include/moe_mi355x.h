/*
 * moe_mi355x.h -- C ABI of the MI355X (gfx950) MoE-layer forward library.
 *
 * One GPU's share of an expert-parallel Mixture-of-Experts layer forward:
 * router scoring and top-k selection, dispatch of token rows into per-expert
 * contiguous groups, the per-expert SwiGLU FFN as a grouped GEMM, and the
 * gate-weighted combine back to token order.  On one GPU the dispatch and
 * combine all-to-alls of expert parallelism become an on-device permutation
 * and its inverse.
 *
 * Problem statement the arguments follow:
 *   - tokens x hidden in, a router choosing the top-k of E experts per token
 *     ("Expert parallelism for MoE serving", overview and deep dive;
 *     "Expert Parallelism: MoE model parallel split", §1);
 *   - router weights weight the sum of the k expert outputs (same page, §1 and
 *     §12 Q2);
 *   - a per-expert capacity with tokens beyond it dropped ("Expert parallelism
 *     for MoE serving", technical notes and FAQ);
 *   - k as a per-request runtime control (MoE-Prism summary, §1 and §5);
 *   - a shared expert ("LLM MoE Expert Parallel production practice", launch
 *     checklist; "Expert Parallelism: MoE model parallel split", §4);
 *   - node-limited (group-limited) routing ("Expert parallelism for MoE
 *     serving", deployment examples).
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers, row-major, owned by the caller and
 *     aligned to 16 bytes.  The library allocates no memory and keeps no state
 *     between calls; scratch space is the caller's workspace `ws` of at least
 *     moe_workspace_size() bytes.  Calls on different streams need distinct
 *     workspaces.  (The one exception, moe_layer_forward_noalloc, takes its
 *     workspace from an array in the library's own device memory.)
 *   - Weights are output-major with K contiguous: router [E][H]; gate and up
 *     [E][I][H]; down [E][H][I]; shared gate/up [Is][H], shared down [H][Is].
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues work; none synchronises with the host (except
 *     moe_read_device_flags), so calls can be captured in a graph.
 *   - Host-checkable errors return before anything is enqueued.
 *   - Every call that takes a workspace clears its flag word at the start;
 *     the word reports that call only.  A failed
 *     launch returns MOE_ERR_HIP (the HIP error code is kept per thread, see
 *     moe_last_hip_error).  Errors found in data on the device (a k_t outside
 *     [1, k_max], an expert id outside [-1, E)) mark the affected slot unused
 *     and set bits in a flag word at the head of the workspace.
 *   - Routing, counts, offsets and the permutation are bitwise deterministic;
 *     all other outputs are run-to-run deterministic (no atomics in sums).
 *   - num_tokens == 0 is valid and enqueues nothing.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, inconsistent shape       */
  MOE_ERR_UNSUPPORTED = -2,  /* valid but outside what the kernels handle         */
  MOE_ERR_WORKSPACE = -3,    /* ws smaller than moe_workspace_size()              */
  MOE_ERR_HIP = -4           /* a HIP call or kernel launch failed                */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_F16 = 2 } moe_dtype;
typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score;

/* device flag bits (moe_read_device_flags) */
#define MOE_FLAG_BAD_K 1u       /* some k_per_token[t] outside [1, top_k]: token routed nowhere */
#define MOE_FLAG_BAD_EXPERT 2u  /* some topk_ids entry outside [-1, E): slot treated as unused  */
#define MOE_FLAG_H_RANGE 4u     /* some SwiGLU activation h exceeded fp16 range (bf16 layers)
                                   or was not finite (MXFP8 layers)                           */
#define MOE_FLAG_BAD_REPLICA 8u /* a routed expert without a replica, or a replica id out of range */
#define MOE_FLAG_Y_RANGE 16u    /* some expert output exceeded fp16 range inside a layer call
                                   (moe_layer_forward, moe_layer_forward_mxfp8)                */

typedef struct {
  int32_t num_tokens;          /* T >= 0                                                  */
  int32_t hidden;              /* H; bf16: multiple of 64; fp32: multiple of 4            */
  int32_t num_experts;         /* E in [1, 512]                                            */
  int32_t intermediate;        /* I; same rule as H                                        */
  int32_t top_k;               /* k, or k_max when k_per_token is given; 1..min(E, 16)    */
  int32_t score;               /* moe_score                                                */
  int32_t renormalize;         /* 1: gates divided by their sum over the token's slots     */
  float routed_scale;          /* multiplies routed gates after renormalising (usually 1) */
  int32_t num_groups;          /* G >= 1 consecutive expert groups; 1 = no group limit     */
  int32_t topk_groups;         /* groups kept per token, 1..G (ignored when G == 1)        */
  int32_t group_topn;          /* group score = sum of the group's n best sigmoid scores;
                                  0 means 1; at most E/G                                   */
  float capacity_factor;       /* C = ceil(cf * A / E), A = routed slots; <= 0: no limit   */
  int32_t shared_intermediate; /* Is; 0 = no shared expert; same rule as H                 */
  int32_t act_dtype;           /* moe_dtype of x and of every weight (MOE_F32 or MOE_BF16)  */
  int32_t out_dtype;           /* moe_dtype of the layer output (MOE_F32 or MOE_BF16)       */
  int32_t down_dtype;          /* 0 or act_dtype: the down weights (routed and shared) have
                                  act_dtype; MOE_F16 (bf16 layers only): they were converted
                                  once by moe_convert_bf16_to_f16 -- the same products, without
                                  the conversion inside every call                           */
} moe_shape;
/* Element offsets are int32 inside the kernels: T*top_k <= 2^30 and each of
 * T*H, E*H, I*H and Is*H <= 2^31-1, else MOE_ERR_UNSUPPORTED. */

/* Stages of moe_layer_forward, for the timing events of moe_debug. */
typedef enum {
  MOE_STAGE_ROUTER = 0,   /* S1 router logits                         */
  MOE_STAGE_ROUTE = 1,    /* S2 scoring, top-k, gates                 */
  MOE_STAGE_DISPATCH = 2, /* S3-S5 histogram, capacity, permutation   */
  MOE_STAGE_GATHER = 3,   /* S6 x_perm gather (fused into S7: empty)  */
  MOE_STAGE_GATE_UP = 4,  /* S7 grouped gate/up GEMM + SwiGLU         */
  MOE_STAGE_DOWN = 5,     /* S8 grouped down GEMM                     */
  MOE_STAGE_SHARED = 6,   /* S9 shared expert (both GEMMs)            */
  MOE_STAGE_COMBINE = 7,  /* S10 combine                              */
  MOE_NUM_STAGES = 8
} moe_stage;

/* Optional outputs of moe_layer_forward for inspection and timing.  Each
 * member may be NULL.  Device buffer sizes: logits T*E, topk_ids/topk_gates/
 * row_of_slot/row_token T*top_k, expert_counts E, expert_offsets E+1,
 * num_dropped 1 (row_token as moe_dispatch writes it: entries at and beyond
 * expert_offsets[E] are left untouched).
 * stage_start[i]/stage_stop[i] are hipEvent_t handles recorded on the call's
 * stream immediately before the first and after the last launch of stage i
 * (a stage that does not run records both at the same point). */
typedef struct {
  float* logits;
  int32_t* topk_ids;
  float* topk_gates;
  int32_t* expert_counts;
  int32_t* expert_offsets;
  int32_t* row_of_slot;
  int32_t* num_dropped;
  void* stage_start[MOE_NUM_STAGES];
  void* stage_stop[MOE_NUM_STAGES];
  int32_t* row_token;
} moe_debug;

/* Bytes of workspace every call below needs for this shape (host only, no HIP
 * call).  The same workspace serves all calls. */
moe_status moe_workspace_size(const moe_shape* shape, size_t* bytes);

/* S1 + S2: router logits and top-k selection.  A router picks the top-k
 * experts of each token ("Expert parallelism for MoE serving", deep dive;
 * "Expert Parallelism: MoE model parallel split", §1: router -> top-k experts
 * -> weighted sum), optionally limited to a few groups of experts (node-
 * limited routing, "Expert parallelism for MoE serving", deployment
 * examples), with k chosen per request (MoE-Prism summary, §1 and §5).
 * logits[t][e] = sum_h x[t][h] * w_router[e][h] + router_bias[e], fp32 accumulate.
 * If logits_in is non-NULL it is used instead and x/w_router/router_bias are
 * ignored (may be NULL).  logits_out (nullable) receives the computed logits.
 * Per token t with k_t = k_per_token ? k_per_token[t] : top_k:
 *   eligible experts: all, or with num_groups > 1 those in the topk_groups
 *   groups of E/G consecutive experts with the largest group score;
 *   selection: the k_t eligible experts with the largest logits, equal logits
 *   going to the lower expert index, written to slots 0..k_t-1 in that order;
 *   gates: softmax over all E logits (or sigmoid of the logit), divided by
 *   their sum over the k_t slots when renormalize, times routed_scale.
 * Outputs topk_ids [T][top_k] int32 (-1 in unused slots) and topk_gates
 * [T][top_k] fp32 (0 in unused slots).  Clears the workspace flag word. */
moe_status moe_route_topk(const moe_shape* shape, const void* x, const void* w_router,
                          const float* router_bias, const float* logits_in, float* logits_out,
                          const int32_t* k_per_token, int32_t* topk_ids, float* topk_gates,
                          void* ws, size_t ws_bytes, void* stream);

/* S3-S6: dispatch ("Expert Parallelism: MoE model parallel split" §3 and §12
 * Q2; token sorting §7; capacity from "Expert parallelism for MoE serving").
 * Slots s = t*top_k + j are visited in token-major order.
 *   expert_counts[e]  = routed slots with id e                         [E]
 *   C                 = ceil(capacity_factor * A / E) in fp64 (A = sum of counts),
 *                       unlimited when capacity_factor <= 0
 *   expert_offsets    = exclusive prefix sum of min(count, C)          [E+1]
 *   row_of_slot[s]    = expert_offsets[e] + (rank of s among slots of e), or -1
 *                       when the slot is unused or its rank >= C       [T][top_k]
 *   row_token[row]    = t for every kept row (rows >= R left untouched) [T*top_k]
 *   num_dropped       = A - R, R = expert_offsets[E]                   [1]
 *   x_perm[row]       = x[row_token[row]] (skipped when x or x_perm is NULL)
 * Clears the workspace flag word, then sets MOE_FLAG_BAD_EXPERT in it for ids
 * outside [-1, E).  expert_offsets[E] <= T*top_k always holds on return. */
moe_status moe_dispatch(const moe_shape* shape, const void* x, const int32_t* topk_ids,
                        int32_t* expert_counts, int32_t* expert_offsets, int32_t* row_of_slot,
                        int32_t* row_token, int32_t* num_dropped, void* x_perm, void* ws,
                        size_t ws_bytes, void* stream);

/* S7-S8: grouped SwiGLU FFN over permuted rows ("LLM MoE Expert Parallel
 * production practice", four-step layer: local expert compute).
 * For every expert e and row r in [expert_offsets[e], expert_offsets[e+1]):
 *   h = silu(x_perm[r] . w_gate[e]^T) * (x_perm[r] . w_up[e]^T),
 *       silu(z) = z / (1 + exp(-z)); fp32 accumulation; h is kept in fp32
 *       for fp32 layers and rounded to fp16 (11-bit significand) for bf16
 *       layers, whose down projection then runs on fp16 inputs (w_down
 *       converted from bf16, exact for |w| >= 2^-14, or already fp16 when
 *       shape->down_dtype is MOE_F16); |h| > 65504 sets MOE_FLAG_H_RANGE
 *   y_perm[r] = h . w_down[e]^T                                    (fp32)
 * Rows at or beyond expert_offsets[E] are not written.  x_perm [T*top_k][H],
 * y_perm [T*top_k][H] fp32.  expert_offsets must be non-decreasing with
 * expert_offsets[0] = 0 and expert_offsets[E] <= T*top_k (as moe_dispatch
 * writes them); the kernels trust them. */
moe_status moe_grouped_ffn(const moe_shape* shape, const void* x_perm,
                           const int32_t* expert_offsets, const void* w_gate, const void* w_up,
                           const void* w_down, float* y_perm, void* ws, size_t ws_bytes,
                           void* stream);

/* Redundant experts: the replica each routed slot goes to.  A hot expert may
 * have identical copies ("LLM MoE Expert Parallel production practice", step
 * 3: selective replicas, the router picks the copy with the lower load;
 * "Expert Parallelism: MoE model parallel split" §6.2: static replicas, the
 * router splits by load).  Logical expert e (of shape->num_experts) has the
 * replicas replica_experts[replica_offsets[e] .. replica_offsets[e+1]),
 * physical expert ids in [0, num_physical).  Slots are visited in token-major
 * order; each goes to the replica of its expert with the fewest slots of this
 * batch assigned so far, ties to the lower replica index -- so the r-th slot
 * of e (token-major) takes replica r mod n_e.
 *   phys_ids[s] = physical expert of slot s, -1 when topk_ids[s] is unused,
 *                 outside [0, E), or e has no valid replica       [T][top_k]
 * topk_ids as moe_route_topk writes them; replica_offsets [E+1] and
 * replica_experts are device arrays (contents checked on the device: an
 * empty replica list or an id outside [0, num_physical) sets
 * MOE_FLAG_BAD_REPLICA and leaves the slot at -1).  The physical ids then go
 * through moe_dispatch / moe_grouped_ffn / moe_combine with num_experts =
 * num_physical and weights [num_physical][..] in which every replica holds its
 * expert's weights; no capacity applies here.  Uses the workspace of
 * `shape`; clears its flag word. */
moe_status moe_map_replicas(const moe_shape* shape, const int32_t* topk_ids,
                            const int32_t* replica_offsets, const int32_t* replica_experts,
                            int32_t num_physical, int32_t* phys_ids, void* ws, size_t ws_bytes,
                            void* stream);

/* S10: combine ("Expert Parallelism: MoE model parallel split" §1 weighted
 * sum, §12 Q2 combine).  out[t] = sum over j ascending with
 * row_of_slot[t][j] >= 0 of topk_gates[t][j] * y_perm[row_of_slot[t][j]],
 * plus y_shared[t] when y_shared is non-NULL; fp32 arithmetic, out in
 * out_dtype. */
moe_status moe_combine(const moe_shape* shape, const float* y_perm, const int32_t* row_of_slot,
                       const float* topk_gates, const float* y_shared, void* out, void* stream);

/* The whole layer: S1-S10 in one call (may fuse steps internally).  The four
 * steps of an MoE layer of "LLM MoE Expert Parallel production practice"
 * (route each token to its top-K experts, send its activations to them, run
 * the expert FFNs, send the outputs back and merge them), with the sends of
 * expert parallelism replaced by an on-device permutation and its inverse
 * ("Expert Parallelism: MoE model parallel split", §1 weighted sum, §3 the
 * dispatch and combine exchanges, §12 Q2 k target positions per token;
 * "Expert parallelism for MoE serving", deep dive and technical notes).
 * out[t] = sum over kept slots of gate * FFN_e(x[t]) + FFN_shared(x[t]):
 * the routing, dispatch, FFN and combine of moe_route_topk, moe_dispatch,
 * moe_grouped_ffn and moe_combine, with the same argument rules.
 * The shared expert runs when shape->shared_intermediate > 0 (then ws_gate,
 * ws_up and ws_down are required; "LLM MoE Expert Parallel production
 * practice", launch checklist; "Expert Parallelism…" §4).  dbg (nullable)
 * receives intermediates.  Clears the workspace flag word. */
moe_status moe_layer_forward(const moe_shape* shape, const void* x, const void* w_router,
                             const float* router_bias, const int32_t* k_per_token,
                             const void* w_gate, const void* w_up, const void* w_down,
                             const void* ws_gate, const void* ws_up, const void* ws_down,
                             void* out, const moe_debug* dbg, void* ws, size_t ws_bytes,
                             void* stream);

/* ---- the expert-parallel exchange over G ranks, on one GPU -------------
 * With expert parallelism over G GPUs ("Expert Parallelism: MoE model
 * parallel split", §8: each GPU holds one contiguous block of E/G experts)
 * every MoE layer exchanges twice (§3, §12 Q2): dispatch sends each token's
 * hidden state to the ranks holding its experts, combine returns their
 * outputs to the token's own rank.  Rows bound for one rank are grouped into
 * one send (§7 and §12, token sorting), and a token travels once to each
 * rank holding any of its experts -- with node-limited routing ("Expert
 * parallelism for MoE serving", deployment examples; group-limited routing
 * with num_groups = G here) at most topk_groups ranks rather than k copies.
 * The two calls below are the source side of both exchanges, run with G
 * virtual ranks on one GPU: the send layout, and the sum of the rows the
 * ranks return.  A rank's own work on the rows it receives is the step
 * chain moe_dispatch / moe_grouped_ffn / moe_combine with its local expert
 * ids, its E/G experts' weights and the received gates (num_tokens = its
 * row count): one pre-reduced row per received row.  Capacity, if any, is
 * the receiving rank's: the layout sends every routed slot. */

/* Send layout of the dispatch exchange.  Rank d holds experts d*E/G ..
 * (d+1)*E/G - 1 (1 <= G <= 64, E % G == 0).  Rows are destination-major,
 * tokens ascending within a rank, no padding:
 *   rank_counts[d]      rows for rank d                                  [G]
 *   rank_offsets        exclusive prefix sum of rank_counts              [G+1]
 *   send_token[p]       token of row p                                   [n_rows]
 *   send_ids[p][j]      topk_ids[t][j] - d*E/G for the slots j of token t
 *                       on rank d, -1 for its other slots                [n_rows][k]
 *   send_gates[p][j]    topk_gates[t][j] where send_ids[p][j] >= 0, else 0
 *   slot_send_pos[t][j] row p of token t's row for the rank of slot j,
 *                       -1 for an unused slot                            [T][k]
 *   send_x[p]           x[send_token[p]] for p < rank_offsets[G]  [n_rows][H]
 *                       (skipped when x and send_x are NULL)
 * n_rows = T * min(top_k, G).  Rows from rank_offsets[G] to n_rows - 1 get
 * send_token -1, send_ids -1 and send_gates 0 (send_x is not written there).
 * topk_ids / topk_gates as moe_route_topk writes them; ids outside [-1, E)
 * count as unused and set MOE_FLAG_BAD_EXPERT.  Uses the workspace of
 * `shape`; clears its flag word.  Positions are bitwise deterministic. */
moe_status moe_ep_dispatch_layout(const moe_shape* shape, int32_t num_ranks, const int32_t* topk_ids,
                                  const float* topk_gates, const void* x, int32_t* rank_counts,
                                  int32_t* rank_offsets, int32_t* send_token, int32_t* send_ids,
                                  float* send_gates, int32_t* slot_send_pos, void* send_x, void* ws,
                                  size_t ws_bytes, void* stream);

/* The combine exchange's last step at the source: partial [n_rows][H] fp32
 * holds, at each row p of the send layout, the gate-weighted sum of the
 * outputs of the experts of rank d for token send_token[p] (what rank d
 * returns).  out[t] = sum of the token's distinct rows (the non-negative
 * slot_send_pos[t][*]) in ascending order -- ascending rank -- plus
 * y_shared[t] when non-NULL; fp32 arithmetic; out in out_dtype.  A token
 * with no routed slot gets y_shared[t] or 0.  No workspace. */
moe_status moe_ep_combine(const moe_shape* shape, int32_t num_ranks, const float* partial,
                          const int32_t* slot_send_pos, const float* y_shared, void* out, void* stream);

/* ---- the layer without a caller workspace ------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Computes
 * exactly what moe_layer_forward computes (same kernels, bit-identical
 * results) with its workspace taken from an array the library keeps in its
 * own device memory: MOE_NOALLOC_SCRATCH_BYTES per GPU, placed when the
 * library's code is loaded on that GPU and held until the process ends.  The
 * call allocates nothing (no hipMalloc, hipFree or allocating library call);
 * its first call on a GPU looks up that GPU's array (the current device's;
 * `stream` must belong to it).  Shapes whose moe_workspace_size() exceeds
 * MOE_NOALLOC_SCRATCH_BYTES return MOE_ERR_WORKSPACE before anything is
 * enqueued (e.g. decode-sized layers fit: 64 tokens of a Mixtral-8x7B-shaped
 * layer need 7.5 MiB, of a DeepSeek-V3-shaped layer 34 MiB).  Every call on a
 * GPU shares that GPU's array and leaves its contents behind; each call
 * clears what it needs cleared (the flag word) itself.  Calls that overlap in
 * time on one GPU (different streams or threads, or a graph replay beside an
 * eager call) race on the array: serialise them.  The flag word of the array
 * is not readable through moe_read_device_flags. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_layer_forward_noalloc(const moe_shape* shape, const void* x, const void* w_router,
                                     const float* router_bias, const int32_t* k_per_token,
                                     const void* w_gate, const void* w_up, const void* w_down,
                                     const void* ws_gate, const void* ws_up, const void* ws_down,
                                     void* out, const moe_debug* dbg, void* stream);

/* ---- 8-bit experts (MXFP8) ---------------------------------------------
 * The pages serve the experts with FP8 quantisation and keep the router in
 * higher precision ("LLM MoE Expert Parallel production practice", deployment
 * examples; "Expert parallelism for MoE serving", FAQ on router precision);
 * they fix no scaling granularity.  The format is MXFP8 of the OCP
 * Microscaling Formats specification v1.0, whose 32-element block scales
 * CDNA4's scaled MFMA applies in hardware:
 *   - each run of 32 consecutive elements of a row (the reduction axis of the
 *     GEMM that reads it) shares one E8M0 scale byte, value 2^(byte - 127);
 *   - each element is an E4M3 byte (OCP FP8: exponent bias 7, largest finite
 *     448, no infinities, 0x7F / 0xFF NaN);
 *   - quantisation: s = floor(log2 amax) - 8, at least -127 (byte 0 for an
 *     all-zero block); element = v / 2^s rounded to the nearest E4M3 value,
 *     ties to even, saturated to +-448, sign kept (a negative value that
 *     rounds to zero is 0x80).
 * Codes are [rows][cols] bytes.  Scales "with stride S" (S >= rows): the
 * four scales of columns [128 g, 128 g + 128) of row r form 32-bit word
 * g * S + r, the block of columns [128 g + 32 i, +32) in byte i.  cols must
 * be a multiple of 128.  The MXFP8 layer keeps x and the router in bf16 for
 * routing, quantises x per token, and re-quantises h per token along I
 * inside the gate/up GEMM.  H, I and Is must be multiples of 128, act_dtype
 * MOE_BF16. */
typedef struct {
  const void* gate;            /* [E][I][H] codes                      */
  const uint8_t* gate_scales;  /* MX scales, stride E*I                */
  const void* up;              /* [E][I][H] codes                      */
  const uint8_t* up_scales;    /* stride E*I                           */
  const void* down;            /* [E][H][I] codes                      */
  const uint8_t* down_scales;  /* stride E*H                           */
} moe_mxfp8_ffn;
/* The shared expert uses the same struct with E = 1: gate/up [Is][H] (scale
 * stride Is), down [H][Is] (scale stride H). */

/* Quantises src [rows][cols] (src_dtype MOE_BF16 or MOE_F32) to MXFP8 codes
 * [rows][cols] and scales with stride scale_stride >= rows.  Inputs are
 * assumed finite (inf / NaN give unspecified codes).  Expert weights are
 * quantised once with this call (rows = E*I or E*H). */
moe_status moe_quantize_mxfp8(int32_t rows, int32_t cols, int32_t src_dtype, const void* src,
                              int32_t scale_stride, void* codes, uint8_t* scales, void* stream);

/* Weight preparation for bf16 layers: dst[i] = src[i] (bf16) as fp16, for
 * i < n (device arrays, 16-byte aligned), with the conversion the down
 * projection applies to bf16 weights inside every layer call (fp16 is the
 * down projection's operand type; exact for |w| in [2^-14, 65504]); layer
 * calls whose shape has down_dtype = MOE_F16 take the converted down weights
 * and skip that conversion, with identical results.  Down weights are
 * converted once with this call (n = E*H*I, and H*Is for the shared expert). */
moe_status moe_convert_bf16_to_f16(int64_t n, const void* src, void* dst, void* stream);

/* Workspace of the two MXFP8 calls below (host only). */
moe_status moe_workspace_size_mxfp8(const moe_shape* shape, size_t* bytes);

/* S7-S8 with MXFP8 operands: as moe_grouped_ffn, with x_perm given as MXFP8
 * codes [T*top_k][H] and scales with stride x_scale_stride >= T*top_k; the
 * dot products accumulate the decoded products in fp32; h = silu(a) * u is
 * rounded from fp32 to MXFP8 along I (blocks of 32 per row) before the down
 * projection; y_perm fp32.  A non-finite h sets
 * MOE_FLAG_H_RANGE.  Clears the workspace flag word. */
moe_status moe_grouped_ffn_mxfp8(const moe_shape* shape, const void* x_codes,
                                 const uint8_t* x_scales, int32_t x_scale_stride,
                                 const int32_t* expert_offsets, const moe_mxfp8_ffn* experts,
                                 float* y_perm, void* ws, size_t ws_bytes, void* stream);

/* The whole layer with MXFP8 experts: S1-S5 as moe_layer_forward on the bf16
 * x and router; x quantised to MXFP8 per token (timed as the gather stage:
 * it is the dispatch payload); S7-S8 as moe_grouped_ffn_mxfp8 on the
 * gathered rows; the shared expert (shape->shared_intermediate > 0, `shared`
 * then required) on the quantised x; S10 as moe_combine. */
moe_status moe_layer_forward_mxfp8(const moe_shape* shape, const void* x, const void* w_router,
                                   const float* router_bias, const int32_t* k_per_token,
                                   const moe_mxfp8_ffn* experts, const moe_mxfp8_ffn* shared,
                                   void* out, const moe_debug* dbg, void* ws, size_t ws_bytes,
                                   void* stream);

/* The fp32 logistic function that group-limited routing sums into group
 * scores, evaluated elementwise: y[i] = sigma(x[i]) for i < n (device
 * arrays).  Node-limited routing ("Expert parallelism for MoE serving",
 * deployment examples) ranks groups by these sums, so the selected groups
 * depend on every bit of them; this entry point lets a checker compare those
 * bits with an independent implementation of the same operation sequence:
 * clamp to [-30, 30]; n = rint(-x * fp32(log2 e)); r = fma(-n, ln2_hi, -x),
 * r = fma(-n, ln2_lo, r) with ln2_hi = ln 2 to 17 significant bits and
 * ln2_lo = fp32(ln 2 - ln2_hi); p = degree-7 Taylor polynomial of e^r with
 * coefficients fp32(1/i!) in Horner form with fma; e = ldexp(p, n);
 * sigma = 1 / (1 + e); IEEE fp32 operations rounded to nearest even. */
moe_status moe_group_score_sigmoid(const float* x, float* y, int64_t n, void* stream);

/* Static text for a status code. */
const char* moe_status_string(moe_status status);

/* hipError_t of the last failed HIP call on this thread (0 if none). */
int32_t moe_last_hip_error(void);

/* Copies the workspace flag word to *flags and waits for it (synchronises the
 * stream).  For tests and diagnostics. */
moe_status moe_read_device_flags(const void* ws, void* stream, uint32_t* flags);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
