/*
 * moe_oracle.c -- plain CPU oracle for one GPU's share of an expert-parallel
 * Mixture-of-Experts layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the GPU library and must never serve as a
 * fallback for it.
 *
 * What it computes (plain definitions, slow on purpose):
 *   "Expert Parallelism: MoE model parallel split" (jwzheng96 sglang-learning),
 *   §1: an MoE layer is Router -> choose top-k experts -> weighted sum; §12 Q2:
 *   dispatch gives every token k target positions (the hidden state copied k
 *   times) and combine merges the k outputs back into the token's position,
 *   weighted by the router weights.
 *   "Expert parallelism for MoE serving" (aiunderstanding.org), deep dive and
 *   FAQ: a router picks the top-k experts per token; a per-expert capacity
 *   (a maximum token count) drops tokens beyond it.
 *   "LLM MoE Expert Parallel production practice" (oh-bug.com), the four
 *   steps of an MoE layer: route top-K, send activations to the expert,
 *   run the local expert, send outputs back and merge.
 *
 * Precision: every dot product and every gate is accumulated in fp64 in plain
 * ascending order, then rounded once to fp32.  Decisions that floating point
 * turns into integers (which experts a token picks, which groups survive) are
 * taken on fp32 values, the precision the GPU takes them in: selection
 * compares fp32 logits; group scores are fp32 sums of the sigmoid defined by
 * sigmoid_spec below.
 */
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_F32 0
#define OR_BF16 1
#define OR_SOFTMAX 0
#define OR_SIGMOID 1

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* element i of an fp32 or raw-bf16 array, widened exactly */
static double elem(const void* base, int dtype, size_t i) {
  if (dtype == OR_BF16) {
    uint32_t bits = ((uint32_t)((const uint16_t*)base)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
  }
  return (double)((const float*)base)[i];
}

/* ---- router logits: logits[t][e] = sum_h x[t][h] * Wr[e][h] + b[e] --------- */
void oracle_router_logits(int T, int H, int E, int dtype, const void* x, const void* w_router,
                          const float* bias, float* logits) {
#pragma omp parallel for schedule(dynamic, 4)
  for (int t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) {
      double s = 0.0;
      for (int h = 0; h < H; ++h)
        s += elem(x, dtype, (size_t)t * H + h) * elem(w_router, dtype, (size_t)e * H + h);
      if (bias) s += (double)bias[e];
      logits[(size_t)t * E + e] = (float)s;
    }
  }
}

/* ---- sigmoid_spec: the fp32 logistic function both sides compute bit-for-bit.
 * Definition (written out as IEEE single-precision operations, each rounded to
 * nearest even, no contraction):
 *   x <- min(max(x, -30), 30); z = -x
 *   n = rint(z * log2e)                       (Cody & Waite argument reduction)
 *   r = fma(-n, ln2_hi, z); r = fma(-n, ln2_lo, r)
 *   p = sum_{i=0..7} r^i / i!  in Horner form with fma (Taylor series of e^r)
 *   e = ldexp(p, n);  sigma = 1 / (1 + e)
 * log2e = fp32(1/ln 2); ln2_hi = ln 2 truncated to 17 significant bits (so
 * n*ln2_hi is exact for |n| < 128); ln2_lo = fp32(ln 2 - ln2_hi); the Taylor
 * coefficients are fp32(1/i!). */
float oracle_sigmoid_spec(float x) {
  const float log2e = 0x1.715476p+0f;
  const float ln2_hi = 0x1.62e400p-1f;
  const float ln2_lo = 0x1.7f7d1cp-20f;
  const float c7 = 0x1.a01a02p-13f, c6 = 0x1.6c16c2p-10f, c5 = 0x1.111112p-7f;
  const float c4 = 0x1.555556p-5f, c3 = 0x1.555556p-3f, c2 = 0x1.0p-1f, c1 = 1.0f, c0 = 1.0f;
  if (x < -30.0f) x = -30.0f;
  if (x > 30.0f) x = 30.0f;
  float z = -x;
  float zl = z * log2e;
  float n = rintf(zl);
  float r = fmaf(-n, ln2_hi, z);
  r = fmaf(-n, ln2_lo, r);
  float p = c7;
  p = fmaf(p, r, c6);
  p = fmaf(p, r, c5);
  p = fmaf(p, r, c4);
  p = fmaf(p, r, c3);
  p = fmaf(p, r, c2);
  p = fmaf(p, r, c1);
  p = fmaf(p, r, c0);
  float e = ldexpf(p, (int)n);
  float den = 1.0f + e;
  return 1.0f / den;
}

void oracle_sigmoid_spec_array(int64_t n, const float* x, float* y) {
  for (int64_t i = 0; i < n; ++i) y[i] = oracle_sigmoid_spec(x[i]);
}

/* (value a, index ia) ranks before (value b, index ib): larger value first,
 * equal values by the lower index. */
static int ranks_before(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

/* ---- routing: scoring, optional group limit, top-k_t, gates ---------------
 * Selection key is the fp32 logit (after bias); the scoring function is monotone
 * so it picks the same set, and ranking logits avoids the ties fp32 sigmoid
 * saturation would create.  Group-limited routing ("node-limited routing",
 * deployment list of "Expert parallelism for MoE serving"): experts form G
 * consecutive groups of E/G; a group's score is the fp32 sum of its `topn`
 * largest sigmoid_spec scores added largest first (topn <= 0 means 1); the
 * topk_groups best groups (score desc, index asc) stay eligible.
 * Gates: softmax over all E (or sigmoid) in fp64; renormalised over the k_t
 * selected when asked; multiplied by routed_scale.  Unused slots: id -1,
 * gate 0.  A k_t outside [1, k_max] leaves the token with no slots.  */
void oracle_route(int T, int E, const float* logits, int k_max, const int32_t* k_per_token,
                  int score, int renorm, float routed_scale, int G, int topk_groups, int topn,
                  int32_t* ids, float* gates) {
  if (topn <= 0) topn = 1;
#pragma omp parallel
  {
    unsigned char* eligible = (unsigned char*)malloc((size_t)E);
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
    float* gscore = (float*)malloc(sizeof(float) * (size_t)(G > 0 ? G : 1));
    unsigned char* gkeep = (unsigned char*)malloc((size_t)(G > 0 ? G : 1));
    float* vals = (float*)malloc(sizeof(float) * (size_t)E);
#pragma omp for schedule(static)
    for (int t = 0; t < T; ++t) {
      const float* l = logits + (size_t)t * E;
      int32_t* id = ids + (size_t)t * k_max;
      float* gt = gates + (size_t)t * k_max;
      for (int j = 0; j < k_max; ++j) { id[j] = -1; gt[j] = 0.0f; }
      int kt = k_per_token ? k_per_token[t] : k_max;
      if (kt < 1 || kt > k_max) continue;

      for (int e = 0; e < E; ++e) { eligible[e] = 1; taken[e] = 0; }
      if (G > 1) {
        int gs = E / G;
        for (int g = 0; g < G; ++g) {
          int n = 0;
          for (int e = g * gs; e < (g + 1) * gs; ++e) vals[n++] = oracle_sigmoid_spec(l[e]);
          /* partial selection sort: the topn largest, in descending order */
          int m = topn < n ? topn : n;
          for (int a = 0; a < m; ++a) {
            int best = a;
            for (int b = a + 1; b < n; ++b) if (vals[b] > vals[best]) best = b;
            float tmp = vals[a]; vals[a] = vals[best]; vals[best] = tmp;
          }
          float s = vals[0];
          for (int a = 1; a < m; ++a) s = s + vals[a];
          gscore[g] = s;
          gkeep[g] = 0;
        }
        int keep = topk_groups < G ? topk_groups : G;
        for (int q = 0; q < keep; ++q) {
          int best = -1;
          for (int g = 0; g < G; ++g) {
            if (gkeep[g]) continue;
            if (best < 0 || ranks_before(gscore[g], g, gscore[best], best)) best = g;
          }
          gkeep[best] = 1;
        }
        for (int e = 0; e < E; ++e) eligible[e] = gkeep[e / gs];
      }

      int nsel = 0;
      for (int j = 0; j < kt; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
          if (!eligible[e] || taken[e]) continue;
          if (best < 0 || ranks_before(l[e], e, l[best], best)) best = e;
        }
        if (best < 0) break;          /* fewer eligible experts than k_t */
        taken[best] = 1;
        id[j] = best;
        nsel++;
      }

      double p[64];
      double* pp = nsel <= 64 ? p : (double*)malloc(sizeof(double) * (size_t)nsel);
      if (score == OR_SOFTMAX) {
        double mx = -INFINITY;
        for (int e = 0; e < E; ++e) if ((double)l[e] > mx) mx = (double)l[e];
        double den = 0.0;
        for (int e = 0; e < E; ++e) den += exp((double)l[e] - mx);
        for (int j = 0; j < nsel; ++j) pp[j] = exp((double)l[id[j]] - mx) / den;
      } else {
        for (int j = 0; j < nsel; ++j) pp[j] = 1.0 / (1.0 + exp(-(double)l[id[j]]));
      }
      if (renorm) {
        double s = 0.0;
        for (int j = 0; j < nsel; ++j) s += pp[j];
        for (int j = 0; j < nsel; ++j) pp[j] /= s;
      }
      for (int j = 0; j < nsel; ++j) gt[j] = (float)(pp[j] * (double)routed_scale);
      if (pp != p) free(pp);
    }
    free(eligible); free(taken); free(gscore); free(gkeep); free(vals);
  }
}

/* ---- capacity ---------------------------------------------------------------
 * C = ceil(cf * A / E) in fp64, A = number of routed slots; cf <= 0: no limit. */
int64_t oracle_capacity(float cf, int64_t A, int E) {
  if (!(cf > 0.0f)) return INT64_MAX;
  return (int64_t)ceil((double)cf * (double)A / (double)E);
}

/* ---- dispatch: histogram, capacity, offsets, stable permutation ------------
 * Slots are visited token-major (t ascending, then slot j).  Each expert keeps
 * its first C slots in that order ("per-expert capacity ... drop tokens beyond
 * it", FAQ of "Expert parallelism for MoE serving"); the kept rows of an expert
 * are contiguous and in token order ("token sorting" of §7, "Expert
 * Parallelism: MoE model parallel split").
 * row_of_slot[s] = offsets[e] + rank, or -1 when unused or dropped;
 * row_token[row] = t.  Returns the number of kept rows R. */
int32_t oracle_dispatch(int T, int E, int k_max, const int32_t* ids, float cf, int32_t* counts,
                        int32_t* offsets, int32_t* row_of_slot, int32_t* row_token,
                        int32_t* num_dropped) {
  int64_t A = 0;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t s = 0; s < (int64_t)T * k_max; ++s) {
    int e = ids[s];
    if (e >= 0 && e < E) { counts[e]++; A++; }
  }
  int64_t C = oracle_capacity(cf, A, E);
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) {
    int64_t kept = counts[e] < C ? counts[e] : C;
    offsets[e + 1] = offsets[e] + (int32_t)kept;
  }
  int32_t* seen = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  for (int t = 0; t < T; ++t) {
    for (int j = 0; j < k_max; ++j) {
      int64_t s = (int64_t)t * k_max + j;
      int e = ids[s];
      if (e < 0 || e >= E) { row_of_slot[s] = -1; continue; }
      int32_t r = seen[e]++;
      if (r < C) {
        int32_t row = offsets[e] + r;
        row_of_slot[s] = row;
        row_token[row] = t;
      } else {
        row_of_slot[s] = -1;
      }
    }
  }
  free(seen);
  if (num_dropped) *num_dropped = (int32_t)(A - offsets[E]);
  return offsets[E];
}

/* ---- redundant experts: replica choice per slot ----------------------------
 * A hot expert may have several identical copies ("replicas"); the router
 * sends each of its tokens to the copy with the lower load ("LLM MoE Expert
 * Parallel production practice", step 3: selective replicas of hot experts;
 * "Expert Parallelism: MoE model parallel split" §6.2: static replicas, the
 * router splits by load).  Plain definition on one batch: slots are visited
 * token-major; a slot of logical expert e goes to the replica of e with the
 * fewest slots assigned so far in this batch, ties to the lower replica
 * index; that replica's count then grows by one.
 * replica_offsets [E+1], replica_experts [replica_offsets[E]]: the physical
 * experts (in [0, num_physical)) holding copies of e.  phys_ids[s] = -1 when
 * the slot is unused, its expert is outside [0, E), e has no replica, or the
 * chosen physical id is outside [0, num_physical).  Returns the number of
 * slots with an invalid replica table entry. */
int32_t oracle_map_replicas(int T, int E, int k_max, const int32_t* ids,
                            const int32_t* replica_offsets, const int32_t* replica_experts,
                            int num_physical, int32_t* phys_ids) {
  int32_t n_total = replica_offsets[E];
  int64_t* load = (int64_t*)calloc((size_t)(n_total > 0 ? n_total : 1), sizeof(int64_t));
  int32_t bad = 0;
  for (int t = 0; t < T; ++t) {
    for (int j = 0; j < k_max; ++j) {
      int64_t s = (int64_t)t * k_max + j;
      int e = ids[s];
      phys_ids[s] = -1;
      if (e < 0 || e >= E) continue;
      int32_t r0 = replica_offsets[e], r1 = replica_offsets[e + 1];
      if (r1 <= r0) { bad++; continue; }
      int32_t best = r0;
      for (int32_t r = r0 + 1; r < r1; ++r)
        if (load[r] < load[best]) best = r;
      load[best]++;
      int32_t p = replica_experts[best];
      if (p < 0 || p >= num_physical) { bad++; continue; }
      phys_ids[s] = p;
    }
  }
  free(load);
  return bad;
}

/* ---- one expert's SwiGLU FFN on one activation row -----------------------
 * y = Wd . (silu(Wg . x) * (Wu . x)), silu(z) = z / (1 + e^-z); fp64 sums.
 * wg, wu: [I][H] rows for this expert; wd: [H][I]. */
static void ffn_row(int H, int I, int dtype, const void* x, size_t xo, const void* wg,
                    const void* wu, size_t wo_gu, const void* wd, size_t wo_d, double* hbuf,
                    double* y) {
  for (int i = 0; i < I; ++i) {
    double a = 0.0, u = 0.0;
    for (int h = 0; h < H; ++h) {
      double xv = elem(x, dtype, xo + h);
      a += elem(wg, dtype, wo_gu + (size_t)i * H + h) * xv;
      u += elem(wu, dtype, wo_gu + (size_t)i * H + h) * xv;
    }
    hbuf[i] = a / (1.0 + exp(-a)) * u;
  }
  for (int c = 0; c < H; ++c) {
    double s = 0.0;
    for (int i = 0; i < I; ++i) s += elem(wd, dtype, wo_d + (size_t)c * I + i) * hbuf[i];
    y[c] = s;
  }
}

/* ---- grouped FFN on permuted rows ----------------------------------------
 * y_perm[r] = FFN_{e(r)}(x_perm[r]) where e(r) is the expert whose range
 * [offsets[e], offsets[e+1]) holds r.  rows: optional subset (n_rows entries);
 * NULL computes rows 0..offsets[E]-1 and n_rows is ignored.  y is [n][H] fp32
 * in the order of `rows`. */
void oracle_grouped_ffn(int E, int H, int I, int dtype, const void* x_perm,
                        const int32_t* offsets, const void* w_gate, const void* w_up,
                        const void* w_down, const int32_t* rows, int n_rows, float* y) {
  int n = rows ? n_rows : offsets[E];
#pragma omp parallel
  {
    double* hb = (double*)malloc(sizeof(double) * (size_t)I);
    double* yb = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
    for (int q = 0; q < n; ++q) {
      int r = rows ? rows[q] : q;
      int e = 0;
      while (e < E && !(r >= offsets[e] && r < offsets[e + 1])) ++e;
      if (e == E) {
        for (int c = 0; c < H; ++c) y[(size_t)q * H + c] = 0.0f;
        continue;
      }
      ffn_row(H, I, dtype, x_perm, (size_t)r * H, w_gate, w_up, (size_t)e * I * H, w_down,
              (size_t)e * H * I, hb, yb);
      for (int c = 0; c < H; ++c) y[(size_t)q * H + c] = (float)yb[c];
    }
    free(hb);
    free(yb);
  }
}

/* ---- combine: out[t] = sum_j g[t][j] * y[row_of_slot[t][j]] (+ y_shared[t]) -
 * j ascending; unused or dropped slots (row -1) contribute nothing; the shared
 * expert's output is added last with weight 1. */
void oracle_combine(int T, int H, int k_max, const float* y_perm, const int32_t* row_of_slot,
                    const float* gates, const float* y_shared, float* out) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    for (int c = 0; c < H; ++c) {
      double acc = 0.0;
      for (int j = 0; j < k_max; ++j) {
        int32_t r = row_of_slot[(size_t)t * k_max + j];
        if (r < 0) continue;
        acc += (double)gates[(size_t)t * k_max + j] * (double)y_perm[(size_t)r * H + c];
      }
      if (y_shared) acc += (double)y_shared[(size_t)t * H + c];
      out[(size_t)t * H + c] = (float)acc;
    }
  }
}

/* ---- whole layer, per token over its chosen experts -----------------------
 * out_t = sum over kept slots j (ascending) of g_{t,j} * FFN_{e_{t,j}}(x_t)
 *         + FFN_shared(x_t)   (when a shared expert is given; weight 1).
 * Routing and dispatch run over all T tokens (capacity depends on all of
 * them); the FFN part runs for the tokens in `tokens` (n_tok entries, or all T
 * when tokens is NULL).  out is [n][H] in the order of `tokens`.
 * logits/ids/gates/counts/offsets/row_of_slot/row_token are caller buffers
 * (sizes T*E, T*k_max, T*k_max, E, E+1, T*k_max, T*k_max).
 * logits_in (nullable): router logits [T][E] to route on instead of computing
 * them -- routing is then a function of these fp32 values alone, which is how
 * another implementation's routing is compared with this one bit for bit. */
void oracle_layer_forward(int T, int H, int E, int I, int k_max, int dtype, const void* x,
                          const void* w_router, const float* bias, const int32_t* k_per_token,
                          int score, int renorm, float routed_scale, int G, int topk_groups,
                          int topn, float cf, const void* w_gate, const void* w_up,
                          const void* w_down, int Is, const void* ws_gate, const void* ws_up,
                          const void* ws_down, const int32_t* tokens, int n_tok, float* out,
                          float* logits, int32_t* ids, float* gates, int32_t* counts,
                          int32_t* offsets, int32_t* row_of_slot, int32_t* row_token,
                          int32_t* num_dropped, const float* logits_in) {
  if (logits_in)
    memcpy(logits, logits_in, sizeof(float) * (size_t)T * (size_t)E);
  else
    oracle_router_logits(T, H, E, dtype, x, w_router, bias, logits);
  oracle_route(T, E, logits, k_max, k_per_token, score, renorm, routed_scale, G, topk_groups,
               topn, ids, gates);
  oracle_dispatch(T, E, k_max, ids, cf, counts, offsets, row_of_slot, row_token, num_dropped);
  int n = tokens ? n_tok : T;
  int Imax = I > Is ? I : Is;
#pragma omp parallel
  {
    double* hb = (double*)malloc(sizeof(double) * (size_t)Imax);
    double* yb = (double*)malloc(sizeof(double) * (size_t)H);
    double* acc = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
    for (int q = 0; q < n; ++q) {
      int t = tokens ? tokens[q] : q;
      for (int c = 0; c < H; ++c) acc[c] = 0.0;
      for (int j = 0; j < k_max; ++j) {
        size_t s = (size_t)t * k_max + j;
        if (row_of_slot[s] < 0) continue;
        int e = ids[s];
        ffn_row(H, I, dtype, x, (size_t)t * H, w_gate, w_up, (size_t)e * I * H, w_down,
                (size_t)e * H * I, hb, yb);
        double g = (double)gates[s];
        for (int c = 0; c < H; ++c) acc[c] += g * yb[c];
      }
      if (Is > 0 && ws_gate) {
        ffn_row(H, Is, dtype, x, (size_t)t * H, ws_gate, ws_up, 0, ws_down, 0, hb, yb);
        for (int c = 0; c < H; ++c) acc[c] += yb[c];
      }
      for (int c = 0; c < H; ++c) out[(size_t)q * H + c] = (float)acc[c];
    }
    free(hb);
    free(yb);
    free(acc);
  }
}

/* ---- MXFP8: 8-bit expert weights and activations ------------------------
 * "LLM MoE Expert Parallel production practice" (oh-bug.com), the
 * deployment examples, serve the experts with FP8 quantisation and keep the
 * router in higher precision ("Expert parallelism for MoE serving", FAQ on
 * router precision).  The pages give no scaling granularity; the format here
 * is MXFP8 from the OCP Microscaling Formats specification v1.0: blocks of 32
 * consecutive elements along the reduction axis share one E8M0 scale
 * X = 2^s, and each element is an E4M3 code (1 sign, 4 exponent bits with
 * bias 7, 3 mantissa bits; no infinities; 0x7F and 0xFF are NaN; largest
 * finite value 448; subnormals m * 2^-9).
 *
 * Value of an E4M3 code, from the bit fields. */
double oracle_e4m3_value(int code) {
  const int sign = (code >> 7) & 1, ex = (code >> 3) & 15, man = code & 7;
  if (ex == 15 && man == 7) return NAN;
  double mag = ex == 0 ? ldexp((double)man, -9) : ldexp(1.0 + man / 8.0, ex - 7);
  return sign ? -mag : mag;
}

/* Nearest E4M3 value to q (|q| < 512 here), ties to the even code; values at
 * or beyond 448 in magnitude saturate to 448.  The sign is kept, so a
 * negative value that rounds to zero gives 0x80.  The code of the rounded
 * value r is read off its binary form, inverting oracle_e4m3_value: r =
 * (1 + m/8) * 2^E with E >= -6 is code ((E + 7) << 3) | m; below 2^-6, r =
 * m * 2^-9 is code m. */
static uint8_t e4m3_encode(double q) {
  const int neg = signbit(q) != 0;
  double a = fabs(q);
  uint8_t mag;
  if (a >= 448.0) {
    mag = 0x7E;
  } else {
    /* the spacing of E4M3 values around a: 2^(e-3) for a in [2^e, 2^(e+1)),
     * e >= -6; subnormals share the spacing 2^-9 of the first binade */
    int e2;
    (void)frexp(a, &e2); /* a = f * 2^e2, f in [0.5, 1) */
    int e = a > 0.0 ? e2 - 1 : -6;
    if (e < -6) e = -6;
    const double ulp = ldexp(1.0, e - 3);
    const double r = rint(a / ulp) * ulp; /* default rounding: to nearest, ties to even */
    if (r < 0x1p-6) {
      mag = (uint8_t)(r * 512.0);          /* subnormal (or zero): m * 2^-9 */
    } else {
      int er;
      (void)frexp(r, &er);                 /* r in [2^(er-1), 2^er) */
      const int E = er - 1;
      const int m = (int)((ldexp(r, -E) - 1.0) * 8.0);
      mag = (uint8_t)(((E + 7) << 3) | m);
    }
  }
  return (uint8_t)(mag | (neg ? 0x80 : 0));
}

/* Quantise a [rows][cols] fp32 / bf16 matrix to MXFP8 along its rows:
 * codes [rows][cols] (one byte each) and scales [rows][cols/32] (E8M0 bytes,
 * value 2^(byte-127)).  Per block of 32: amax = max |v|; the shared exponent
 * is floor(log2 amax) - 8 (8 = exponent of E4M3's largest binade), clamped to
 * [-127, 127], and -127 for an all-zero block; each element is v / 2^s
 * rounded to E4M3 as above.  cols must be a multiple of 32. */
void oracle_mxfp8_quantize(int rows, int cols, int dtype, const void* src, uint8_t* codes,
                           uint8_t* scales) {
  const int nb = cols / 32;
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r) {
    for (int b = 0; b < nb; ++b) {
      const size_t o = (size_t)r * cols + (size_t)b * 32;
      double amax = 0.0;
      for (int i = 0; i < 32; ++i) {
        const double v = fabs(elem(src, dtype, o + i));
        if (v > amax) amax = v;
      }
      int s = -127;
      if (amax > 0.0) {
        int e2;
        (void)frexp(amax, &e2);
        s = (e2 - 1) - 8;
        if (s < -127) s = -127;
        if (s > 127) s = 127;
      }
      scales[(size_t)r * nb + b] = (uint8_t)(s + 127);
      const double inv = ldexp(1.0, -s); /* 2^-s: the division by the scale is exact */
      for (int i = 0; i < 32; ++i) codes[o + i] = e4m3_encode(elem(src, dtype, o + i) * inv);
    }
  }
}

/* Decodes row `row` of an MXFP8 matrix with `cols` columns into out[cols]:
 * element = value(code) * 2^(scale - 127), exact in fp64 (tbl[c] is the
 * value of code c). */
static void mx_decode_row(const double* tbl, const uint8_t* codes, const uint8_t* scales, int cols,
                          size_t row, double* out) {
  const uint8_t* c = codes + row * (size_t)cols;
  const uint8_t* s = scales + row * (size_t)(cols / 32);
  for (int b = 0; b < cols / 32; ++b) {
    const double p = ldexp(1.0, (int)s[b] - 127);
    for (int i = 0; i < 32; ++i) out[b * 32 + i] = tbl[c[b * 32 + i]] * p;
  }
}

/* One expert's SwiGLU FFN on one MXFP8 activation row, with MXFP8 weights:
 * a = Wg . x and u = Wu . x over the decoded values (fp64 sums in ascending
 * k); h = silu(a)*u is rounded to fp32 and re-quantised to MXFP8 along I (the
 * input of the down projection is 8-bit as well); y = Wd . h over the decoded
 * h (fp64, ascending i).  dg, du: the expert's decoded gate and up weights
 * [I][H]; dd: its decoded down weights [H][I] (mx_decode_row of every weight
 * row, done once per expert by the caller).  Scratch: xd [H], hd [I]. */
static void ffn_row_mxfp8(const double* tbl, int H, int I, const uint8_t* xq, const uint8_t* xs,
                          size_t xrow, const double* dg, const double* du, const double* dd,
                          float* h32, uint8_t* hq, uint8_t* hs, double* xd, double* hd, double* y) {
  mx_decode_row(tbl, xq, xs, H, xrow, xd);
  for (int i = 0; i < I; ++i) {
    const double* wg = dg + (size_t)i * H;
    const double* wu = du + (size_t)i * H;
    double a = 0.0, u = 0.0;
    for (int k = 0; k < H; ++k) {
      a += wg[k] * xd[k];
      u += wu[k] * xd[k];
    }
    h32[i] = (float)(a / (1.0 + exp(-a)) * u);
  }
  oracle_mxfp8_quantize(1, I, OR_F32, h32, hq, hs);
  mx_decode_row(tbl, hq, hs, I, 0, hd);
  for (int c = 0; c < H; ++c) {
    const double* wd = dd + (size_t)c * I;
    double s = 0.0;
    for (int i = 0; i < I; ++i) s += wd[i] * hd[i];
    y[c] = s;
  }
}

/* Grouped FFN on permuted MXFP8 rows: y_perm[r] = FFN_{e(r)}(x_perm[r]) with
 * e(r) the expert whose range [offsets[e], offsets[e+1]) holds r.  xq/xs are
 * the quantised permuted rows ([R][H] codes, [R][H/32] scales); rows/n_rows
 * select a subset as in oracle_grouped_ffn.  h_out (nullable) receives each
 * computed row's fp32 h before its MXFP8 rounding, [n][I]. */
void oracle_grouped_ffn_mxfp8(int E, int H, int I, const uint8_t* xq, const uint8_t* xs,
                              const int32_t* offsets, const uint8_t* wgq, const uint8_t* wgs,
                              const uint8_t* wuq, const uint8_t* wus, const uint8_t* wdq,
                              const uint8_t* wds, const int32_t* rows, int n_rows, float* y,
                              float* h_out) {
  int n = rows ? n_rows : offsets[E];
  double tbl[256];
  for (int c = 0; c < 256; ++c) tbl[c] = oracle_e4m3_value(c);
  /* the expert of every requested row (E: none) */
  int* eq = (int*)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
  for (int q = 0; q < n; ++q) {
    int r = rows ? rows[q] : q;
    int e = 0;
    while (e < E && !(r >= offsets[e] && r < offsets[e + 1])) ++e;
    eq[q] = e;
    if (e == E) {
      for (int c = 0; c < H; ++c) y[(size_t)q * H + c] = 0.0f;
      if (h_out) memset(h_out + (size_t)q * I, 0, sizeof(float) * (size_t)I);
    }
  }
  /* expert by expert: its weights decoded once, then its rows */
  double* dg = (double*)malloc(sizeof(double) * (size_t)I * H);
  double* du = (double*)malloc(sizeof(double) * (size_t)I * H);
  double* dd = (double*)malloc(sizeof(double) * (size_t)H * I);
  for (int e = 0; e < E; ++e) {
    int any = 0;
    for (int q = 0; q < n && !any; ++q) any = eq[q] == e;
    if (!any) continue;
#pragma omp parallel for schedule(static)
    for (int i = 0; i < I; ++i) {
      mx_decode_row(tbl, wgq, wgs, H, (size_t)e * I + i, dg + (size_t)i * H);
      mx_decode_row(tbl, wuq, wus, H, (size_t)e * I + i, du + (size_t)i * H);
    }
#pragma omp parallel for schedule(static)
    for (int c = 0; c < H; ++c) mx_decode_row(tbl, wdq, wds, I, (size_t)e * H + c, dd + (size_t)c * I);
#pragma omp parallel
    {
      float* h32 = (float*)malloc(sizeof(float) * (size_t)I);
      uint8_t* hq = (uint8_t*)malloc((size_t)I);
      uint8_t* hs = (uint8_t*)malloc((size_t)I / 32 + 1);
      double* yb = (double*)malloc(sizeof(double) * (size_t)H);
      double* xd = (double*)malloc(sizeof(double) * (size_t)H);
      double* hd = (double*)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(dynamic, 1)
      for (int q = 0; q < n; ++q) {
        if (eq[q] != e) continue;
        int r = rows ? rows[q] : q;
        ffn_row_mxfp8(tbl, H, I, xq, xs, (size_t)r, dg, du, dd, h32, hq, hs, xd, hd, yb);
        for (int c = 0; c < H; ++c) y[(size_t)q * H + c] = (float)yb[c];
        if (h_out) memcpy(h_out + (size_t)q * I, h32, sizeof(float) * (size_t)I);
      }
      free(h32);
      free(hq);
      free(hs);
      free(yb);
      free(xd);
      free(hd);
    }
  }
  free(dg);
  free(du);
  free(dd);
  free(eq);
}

/* ---- expert-parallel exchange over G ranks ---------------------------------
 * "Expert Parallelism: MoE model parallel split" (jwzheng96 sglang-learning):
 * §8, with expert parallelism over G GPUs the experts form G contiguous blocks
 * of E/G (rank d holds experts d*E/G .. (d+1)*E/G - 1); §3 and §12 Q2, each
 * MoE layer exchanges twice: dispatch sends a token's hidden state to the
 * ranks of its chosen experts, combine sends the expert outputs back to the
 * token's own rank, where they are summed with the router weights; §7 and
 * §12, token sorting: the rows bound for one rank are grouped so they travel
 * in one send.  "Expert parallelism for MoE serving", deployment examples:
 * node-limited routing bounds the number of nodes a token's experts span,
 * which lowers traffic only if a token travels once to each rank that holds
 * any of its experts (not once per expert) -- the reading taken here; the
 * receiving rank then applies the token's several experts to that one row
 * and returns their gate-weighted sum as one row.
 *
 * Layout of the send buffer (destination-major, ragged, no padding rows):
 * for d = 0 .. G-1, for t ascending, one row for each token with at least one
 * routed slot (expert id in [0, E)) on rank d.
 *   rank_counts[d]     rows for rank d                               [G]
 *   rank_offsets       exclusive prefix sum of rank_counts           [G+1]
 *   send_token[p]      the token of row p                            [n_rows]
 *   send_ids[p][j]     id[t][j] - d*E/G for each slot j of t on rank d,
 *                      -1 for its other slots                        [n_rows][k]
 *   send_gates[p][j]   gates[t][j] where send_ids[p][j] >= 0, else 0 [n_rows][k]
 *   slot_send_pos[t][j] the row p of token t's row for the rank of slot
 *                      j, -1 for an unused slot                      [T][k]
 * n_rows = T * min(k, G) rows are provided; rows from rank_offsets[G] on hold
 * send_token -1, send_ids -1 and send_gates 0.  Ids outside [-1, E) count as
 * unused.  Returns the number of rows sent, rank_offsets[G]. */
int32_t oracle_ep_layout(int T, int E, int k, int G, const int32_t* ids, const float* gates,
                         int32_t* rank_counts, int32_t* rank_offsets, int32_t* send_token,
                         int32_t* send_ids, float* send_gates, int32_t* slot_send_pos) {
  const int epr = E / G;
  const int n_rows = T * (k < G ? k : G);
  for (int64_t s = 0; s < (int64_t)T * k; ++s) slot_send_pos[s] = -1;
  for (int p = 0; p < n_rows; ++p) {
    send_token[p] = -1;
    for (int j = 0; j < k; ++j) {
      send_ids[(size_t)p * k + j] = -1;
      send_gates[(size_t)p * k + j] = 0.0f;
    }
  }
  int32_t p = 0;
  rank_offsets[0] = 0;
  for (int d = 0; d < G; ++d) {
    for (int t = 0; t < T; ++t) {
      int on_rank = 0;
      for (int j = 0; j < k; ++j) {
        const int e = ids[(size_t)t * k + j];
        if (e >= 0 && e < E && e / epr == d) on_rank = 1;
      }
      if (!on_rank) continue;
      send_token[p] = t;
      for (int j = 0; j < k; ++j) {
        const int e = ids[(size_t)t * k + j];
        if (e >= 0 && e < E && e / epr == d) {
          send_ids[(size_t)p * k + j] = e - d * epr;
          send_gates[(size_t)p * k + j] = gates[(size_t)t * k + j];
          slot_send_pos[(size_t)t * k + j] = p;
        }
      }
      ++p;
    }
    rank_counts[d] = p - rank_offsets[d];
    rank_offsets[d + 1] = p;
  }
  return p;
}

/* The combine exchange's last step, at the token's own rank: every rank that
 * received token t returned one row, the gate-weighted sum of its experts'
 * outputs for t (partial[p], p = the token's row in the send layout);
 * out[t] = the sum of those rows, ascending p (ascending rank), plus
 * y_shared[t] when given (the shared expert, weight 1, added last); fp64
 * sums rounded once.  A token with no routed slot gets y_shared[t] or 0. */
void oracle_ep_combine(int T, int H, int k, const float* partial, const int32_t* slot_send_pos,
                       const float* y_shared, float* out) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    /* the token's distinct rows, ascending */
    int32_t rows[64];
    int n = 0;
    for (int j = 0; j < k; ++j) {
      const int32_t r = slot_send_pos[(size_t)t * k + j];
      if (r < 0) continue;
      int seen = 0;
      for (int q = 0; q < n; ++q) seen |= rows[q] == r;
      if (!seen) rows[n++] = r;
    }
    for (int a = 1; a < n; ++a)
      for (int b = a; b > 0 && rows[b - 1] > rows[b]; --b) {
        const int32_t tmp = rows[b];
        rows[b] = rows[b - 1];
        rows[b - 1] = tmp;
      }
    for (int c = 0; c < H; ++c) {
      double acc = 0.0;
      for (int q = 0; q < n; ++q) acc += (double)partial[(size_t)rows[q] * H + c];
      if (y_shared) acc += (double)y_shared[(size_t)t * H + c];
      out[(size_t)t * H + c] = (float)acc;
    }
  }
}
