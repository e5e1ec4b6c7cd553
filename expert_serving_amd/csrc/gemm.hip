// S7-S9 (and the router projection S1): grouped GEMMs over ragged expert row
// groups with device-side row tiles.
//
// Each expert's FFN runs on the rows dispatched to it ("LLM MoE Expert
// Parallel production practice", four-step layer; "Expert parallelism for MoE
// serving", deep dive).  The groups are ragged: no padding rows exist in
// memory ("Expert Parallelism: MoE model parallel split", §12 Q4 avoids
// padding); rows past a group's end inside a tile are clamped on load and
// masked on store.
//
// bf16 kernels (gfx950):
//   * v_mfma_f32_32x32x16_bf16 (f16 for the down projection), fp32
//     accumulation; the weight tile is the MFMA A operand and the token tile
//     the B operand, so a lane's accumulators are runs of consecutive output
//     columns of one token row;
//   * 8-wave blocks (256-, 128-, 64- and 32-row tiles): two waves per SIMD
//     in a ping-pong over register-staged loads and two LDS stages of K = 64
//     (128-byte rows, 16-byte chunks XOR-swizzled by row); 4-wave blocks (the
//     32-row tiles of some small-expert launches): direct-to-LDS loads into a
//     ring of K = 32 stages;
//   * gate/up variant: one block computes the same column range of X.Wg^T
//     and X.Wu^T and applies SwiGLU in the epilogue (h never exists unfused);
//   * skewed loads: the big experts' tiles and the small experts' tiles run
//     interleaved in one launch; tiles of at most four token rows there take
//     a vector-ALU path that streams the weights straight into registers;
//   * block -> tile map: blocks are dealt round-robin to the 8 XCDs, so block
//     b is remapped to give each XCD a contiguous range of logical tiles, and
//     logical tiles sweep groups of kGroupM row tiles across all column tiles
//     so the XCD's L2 serves both the token rows and the weight rows.
// The MXFP8 modes run the same 8-wave schedule on E4M3 codes with the scaled
// fp8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4).
#include <atomic>

#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Row tiles per group of the tile order (groups sweep all column tiles; the
// blocks an XCD runs together then cover about 8 row tiles x 4 column
// tiles).  Measured on one box against 16, 4, 2 and 1: Mixtral-shaped layer
// 1.9% and Qwen3-shaped 1.6% faster than 16, DeepSeek-V3-shaped within 0.1%.
constexpr int kGroupM = 8;

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b + (((b >> 16) & 1u) + 0x7FFFu)) >> 16;
}

// silu(g) * u with silu(g) = g / (1 + e^-g).  The reciprocal is the
// hardware's v_rcp_f32 (about 1 ulp) rather than an IEEE division: the
// correctly rounded divide expands to a dozen instructions per element and
// cost a tenth of the gate/up kernel's time in its epilogue, while h is
// rounded to fp16 or E4M3 right after.  For e^-g = inf (g < -88) the
// reciprocal is 0 and the result a signed zero, as with the division.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Row tile m and column tile n of logical tile L of a class with mtiles x
// ntiles tiles: groups of group_m row tiles sweep all column tiles.
__device__ __forceinline__ void tile_of(int L, int mtiles, int ntiles, int& m, int& n, int group_m) {
  const int groups_full = mtiles / group_m;
  const int per_group = group_m * ntiles;
  const int g = L / per_group;
  const int gm = g < groups_full ? group_m : mtiles - groups_full * group_m;  // last group may be short
  const int r = L - g * per_group;
  n = r / gm;
  m = g * group_m + (r - n * gm);
}

// Logical index of this block among `real` tiles, XCD by XCD: block b runs on
// XCD b % 8 and takes (b % 8) * ceil(real / 8) + b / 8, so every XCD gets a
// contiguous range; false for the padding blocks of a worst-case grid.
__device__ __forceinline__ bool xcd_index(int real, int& L) {
  const int b = blockIdx.x;
  const int per_xcd = (real + 7) >> 3;
  const int slot = b >> 3;
  if (slot >= per_xcd) return false;
  L = (b & 7) * per_xcd + slot;
  return L < real;
}

// Logical tile of this block.  Blocks are dealt round-robin to the 8 XCDs
// (block b runs on XCD b % 8), so block b takes logical tile
// (b % 8) * per_xcd + b / 8: each XCD gets a contiguous range of the `real`
// tiles that exist (row tiles known on the device x column tiles), and the
// padding blocks of the launch (grid sized for the worst case) exit.  Logical
// tiles sweep groups of group_m row tiles across all column tiles, so the
// blocks an XCD runs together share both token rows and weight rows in L2.
__device__ __forceinline__ bool block_tile(int mtiles, int ntiles, int& m, int& n, int group_m) {
  int L;
  if (!xcd_index(mtiles * ntiles, L)) return false;
  tile_of(L, mtiles, ntiles, m, n, group_m);
  return true;
}

// Two classes of real0 and real1 tiles (class 0 the long MFMA-bound tiles,
// class 1 the short weight-streaming ones) over logical indices L (XCD by XCD
// as above).  Each XCD's range takes its even share of both classes (the
// count of class-1 tiles before L is floor(L * real1 / total) at the range
// ends) and orders them in time: the last r of its s class-1 tiles go at the
// end of the range, the rest are spread evenly (Bresenham) over the front.
// Blocks reach an XCD's compute units in range order, so short tiles at the
// end fill the units while the last long tiles finish:
//   - many short tiles (real1 > real0 / 4, skewed layers): r = s / 4; more
//     would end the launch on a phase of weight streams alone;
//   - few short tiles and at most about two and a half rounds of long tiles
//     on the 256 compute units: r = s, longest first;
//   - few short tiles over many rounds: r = 0, their weight streams spread
//     between the MFMA-bound tiles.
// idx is the tile's index within its class (cls 0 or 1), in increasing order
// along L, so each XCD's tiles of a class are contiguous.
__device__ __forceinline__ bool block_tile2(int real0, int real1, int& cls, int& idx) {
  const int total = real0 + real1;
  int L;
  if (!xcd_index(total, L)) return false;
  const int per_xcd = (total + 7) >> 3;
  const int a = (L / per_xcd) * per_xcd;  // the XCD's range [a, a + n)
  const int n = min(per_xcd, total - a);
  const int sa = (int)((long long)a * real1 / total);
  const int s = (int)((long long)(a + n) * real1 / total) - sa;  // its class-1 tiles
  const int r = 4LL * real1 > real0 ? s / 4 : (2LL * real0 <= 5 * 256 ? s : 0);
  const int p = L - a;
  // class-1 tiles among positions [0, q) of the range
  auto before = [&](int q) {
    return q >= n - r ? (s - r) + (q - (n - r)) : (int)((long long)q * (s - r) / (n - r));
  };
  const int c0 = before(p), c1 = before(p + 1);
  if (c1 > c0) {
    cls = 1;
    idx = sa + c0;
  } else {
    cls = 0;
    idx = a - sa + p - c0;
  }
  return true;
}

// Kernel modes.
//   kGateUp: A = bf16 token rows, B0/B1 = bf16 gate/up weights;
//            out h (fp16) = silu(A.B0^T) * (A.B1^T)
//   kDown:   A = fp16 h rows, B0 = bf16 down weights converted to fp16 while
//            staged into LDS (exact for |w| in fp16's normal range);
//            out y (fp32) = A.B0^T
//   kPlain:  A = bf16 rows, B0 = bf16 weights; out fp32 = A.B0^T + bias
//   kGateUpMX: A = MXFP8 token rows, B0/B1 = MXFP8 gate/up weights; out h =
//            silu(A.B0^T) * (A.B1^T) re-quantised to MXFP8 (codes + scales)
//   kDownMX: A = MXFP8 h rows, B0 = MXFP8 down weights; out y (fp32)
// The MX modes take every row length, K and lda in 16-bit units (two E4M3
// codes), so the byte layout of their tiles is that of the bf16 modes.
//   kGateUpPart: as kGateUp on one K range of a split K, without SwiGLU: the
//            fp32 partial sums A.B0^T at Out and A.B1^T at Out + up_off
//   kGateUpMXPart: the same on MXFP8 operands
//   kDownW16: kDown with the down weights already fp16 (converted once, ahead
//            of the layer calls, by the same conversion kDown applies)
enum GemmMode {
  kGateUp = 0, kDown = 1, kPlain = 2, kGateUpMX = 3, kDownMX = 4, kGateUpPart = 5, kGateUpMXPart = 6,
  kDownW16 = 7
};

// modes that multiply by both the gate and the up weights
constexpr bool gemm_dual(int MODE) {
  return MODE == kGateUp || MODE == kGateUpMX || MODE == kGateUpPart || MODE == kGateUpMXPart;
}
// modes on MXFP8 operands
constexpr bool gemm_mx(int MODE) { return MODE == kGateUpMX || MODE == kDownMX || MODE == kGateUpMXPart; }
// split-K gate/up modes (fp32 partial gate and up sums out)
constexpr bool gemm_part(int MODE) { return MODE == kGateUpPart || MODE == kGateUpMXPart; }

// Scales of the MXFP8 operands (E8M0 bytes, four blocks of a 128-column group
// per 32-bit word, words group-major: the word of group g of row r is
// g * stride + r): token rows (sa), weight rows (sb0 / sb1; expert e's rows
// start at e * N), and the scales of the h output (sout).
struct MxArgs {
  const uint8_t* sa;
  const uint8_t* sb0;
  const uint8_t* sb1;
  uint8_t* sout;
  int sa_stride, sb_stride, sout_stride;
  // 1: the token scales are already in tile-row order (word row0 + r) even
  // when the codes are gathered through a_rows, so a wavefront's scale words
  // are contiguous instead of one cache line per lane
  int sa_direct;
};

// E8M0 byte of a block with maximum magnitude amax (finite, >= 0):
// floor(log2 amax) - 8 + 127, at least 0 (also the byte of an all-zero block)
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
  const int e = (int)(__float_as_uint(amax) >> 23);
  return e > 8 ? (uint32_t)(e - 8) : 0u;
}

// four values already divided by their block scale -> four E4M3 bytes
// (element 0 lowest), nearest-even, saturated to +-448
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  c = fminf(fmaxf(c, -448.f), 448.f);
  d = fminf(fmaxf(d, -448.f), 448.f);
  int p = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  p = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, p, true);
  return (uint32_t)p;
}

// the 32 E4M3 codes of one lane for v_mfma_scale_f32_32x32x64_f8f6f4: bytes
// 0-15 belong to the slice's first 32-element block, bytes 16-31 to its
// second (lanes 32-63 hold the upper 16 of each block)
__device__ __forceinline__ i32x8 cat8(u32x4 lo, u32x4 hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  const float lo = __uint_as_float(w << 16);
  const float hi = __uint_as_float(w & 0xFFFF0000u);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v) {
  return u32x4{bf16x2_to_f16x2(v[0]), bf16x2_to_f16x2(v[1]), bf16x2_to_f16x2(v[2]),
               bf16x2_to_f16x2(v[3])};
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

template <int MODE>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (MODE == kDown || MODE == kDownW16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

constexpr int kSK = 32;            // K elements per step (and per LDS row of 4-wave blocks)
constexpr int kPingRowElems = 64;  // K elements per LDS row of 8-wave blocks (128 bytes)

// Rows of one stage, padded to whole wavefront loads per wave: 16 rows per
// load for 4-wave blocks, 8 rows per load for 8-wave blocks.
constexpr int gemm_stage_rows(int BM, int BNB, int MODE, int NW) {
  return (BM + BNB * (gemm_dual(MODE) ? 2 : 1) + (NW == 8 ? 8 : 16) * NW - 1) /
         ((NW == 8 ? 8 : 16) * NW) * ((NW == 8 ? 8 : 16) * NW);
}
// Bytes of LDS one block of k_gemm_mfma<BM, BNB, MODE, NS, NW> uses: NS
// stages of tiles, and for the MXFP8 modes one 32-bit scale word per tile row
// and stage.
constexpr int gemm_lds_bytes(int BM, int BNB, int MODE, int NS, int NW) {
  return NS * gemm_stage_rows(BM, BNB, MODE, NW) *
         ((NW == 8 ? kPingRowElems : kSK) * 2 + (gemm_mx(MODE) ? 4 : 0));
}

// Word 3 of a raw buffer resource on gfx9-family GPUs (32-bit data format).
constexpr int kBufferRsrcWord3 = 0x00020000;

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef const __attribute__((address_space(1))) void* gbl_ptr_t;

// s_waitcnt that waits for vmcnt <= n and lgkmcnt/expcnt not at all (gfx9 encoding).
#define MOE_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

// s_waitcnt that waits for lgkmcnt == 0 (LDS reads landed) and nothing else.
#define MOE_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4))

// Workgroup barrier without a memory fence: the pipeline's own s_waitcnt
// orders the LDS traffic; the empty asm keeps the compiler from moving memory
// operations across it.
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// BM token rows x BNB weight rows (per weight matrix) per block, NW waves
// (2 x NW/2, or 1 x NW when BM = 32), v_mfma_f32_32x32x16 (bf16, or f16 for
// the down projection).  8-wave blocks (two waves per SIMD) run a ping-pong
// schedule over register-staged loads; 4-wave blocks (the 32-row tiles of
// small experts) stream tiles straight into LDS.  Both schedules are
// described where they are implemented, in the main loop below.
//
// The weight tile is the MFMA A operand and the token tile the B operand, so
// a lane's 16 accumulators are 4 runs of 4 consecutive output columns of one
// token row.
template <int BM, int BNB, int MODE, int NS, int NW>
__device__ __forceinline__ void gemm_tile(
    uint16_t* __restrict__ smem, const uint16_t* __restrict__ A, const int32_t* __restrict__ a_rows,
    int lda, const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1, long long strideB,
    int N, int K, void* __restrict__ Out, int ldo, const float* __restrict__ bias,
    const MTile* __restrict__ sched, int static_rows, uint32_t* __restrict__ flags, const MxArgs mx,
    int mi, int ni, int kst0, int kstn, long long up_off = 0, bool out_half = false) {
  constexpr bool DUAL = gemm_dual(MODE);
  constexpr bool MX = gemm_mx(MODE);
  constexpr int WAVES_M = BM >= 64 ? 2 : 1, WAVES_N = NW / WAVES_M;
  constexpr int WM = BM / WAVES_M, WN = BNB / WAVES_N;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int NB = DUAL ? 2 : 1;
  constexpr int ROWS = gemm_stage_rows(BM, BNB, MODE, NW);  // rows of one stage (padded)
  // 8-wave blocks: register-staged ping-pong over two LDS stages; 4-wave
  // blocks: direct-to-LDS loads over an NS-stage ring
  constexpr bool PING = NW == 8;
  // bf16 down weights are converted to fp16 once when staged through
  // registers (8-wave blocks), else on every fragment read; kDownW16 weights
  // arrive as fp16
  constexpr bool CVT_ON_READ = MODE == kDown && !PING;
  static_assert(BM % 32 == 0 && BNB % 32 == 0 && FM >= 1 && FN >= 1, "tile shape");
  static_assert(!PING || NS == 2, "ping-pong uses two LDS stages");
  static_assert(!MX || PING, "MXFP8 modes run the 8-wave schedule");

  int expert = 0, row0, rows;
  if (sched) {
    const MTile t = sched[mi];
    expert = t.expert;
    row0 = t.row0;
    rows = t.rows;
  } else {
    row0 = mi * BM;
    rows = min(BM, static_rows - row0);
  }
  const int n0 = ni * BNB;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: lets chunk offsets live in SGPRs
  __builtin_assume(wave >= 0 && wave < NW);
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;

  // A rows are contiguous from row0, or gathered: tile row r is row a_rows[row0 + r]
  // K range of this block: 64-element stages kst0 .. kst0 + kstn (all of K
  // unless the launch splits K into partial sums)
  const uint16_t* Ab = (a_rows ? A : A + (size_t)row0 * lda) + kst0 * kPingRowElems;
  const uint16_t* B0b = B0 + (size_t)expert * strideB + kst0 * kPingRowElems;
  const uint16_t* B1b = DUAL ? B1 + (size_t)expert * strideB + kst0 * kPingRowElems : B0b;

  f32x16 acc0[FN][FM];
  f32x16 acc1[DUAL ? FN : 1][DUAL ? FM : 1];
#pragma unroll
  for (int a = 0; a < FN; ++a)
#pragma unroll
    for (int b = 0; b < FM; ++b) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        acc0[a][b][q] = 0.f;
        if constexpr (DUAL) acc1[a][b][q] = 0.f;
      }
    }

  const int fr = lane & 31;   // row of a 32-row fragment this lane feeds
  const int fk = lane >> 5;   // which 8-element K chunk (of 2) of a slice this lane feeds

  u32x4 xa[MX ? 1 : 2][FM], wb0[MX ? 1 : 2][FN], wb1[MX ? 1 : 2][DUAL ? FN : 1];
  // MXFP8 fragments: both 16-byte halves of a step in one 8-register operand
  i32x8 xa8[MX ? FM : 1], wg8[MX ? FN : 1], wu8[MX && DUAL ? FN : 1];
#define MOE_MFMAS(set_)                                                                 \
  do {                                                                                  \
    _Pragma("unroll") for (int a = 0; a < FN; ++a) {                                    \
      const u32x4 w0_ = CVT_ON_READ ? bf16x8_to_f16x8(wb0[set_][a]) : wb0[set_][a];      \
      _Pragma("unroll") for (int b = 0; b < FM; ++b) {                                  \
        acc0[a][b] = mfma32<MODE>(w0_, xa[set_][b], acc0[a][b]);                        \
        if constexpr (DUAL) acc1[a][b] = mfma32<MODE>(wb1[set_][a], xa[set_][b], acc1[a][b]); \
      }                                                                                 \
    }                                                                                   \
  } while (0)
  // MXFP8: one v_mfma_scale_f32_32x32x64_f8f6f4 per fragment pair and step
  // (K = 64 codes, two 32-element blocks: a lane's bytes 0-15 are its 16 codes
  // of the first block, bytes 16-31 of the second); the scale words are
  // pre-shifted so that byte 2h selects this lane's block of slice h.
#define MOE_MFMAS_MX(h_)                                                                \
  do {                                                                                  \
    _Pragma("unroll") for (int a = 0; a < FN; ++a) {                                    \
      _Pragma("unroll") for (int b = 0; b < FM; ++b) {                                  \
        acc0[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                   \
            wg8[a], xa8[b], acc0[a][b], 0, 0, 2 * (h_), scc[FM + a], 2 * (h_), scc[b]); \
        if constexpr (DUAL)                                                             \
          acc1[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                 \
              wu8[a], xa8[b], acc1[a][b], 0, 0, 2 * (h_), scc[FM + FN + a], 2 * (h_),   \
              scc[b]);                                                                  \
      }                                                                                 \
    }                                                                                   \
  } while (0)
  // global element offset of tile row rho, 16-byte chunk ch (K offset added per load)
  auto row_goff = [&](int rho, int ch) -> int {
    if (rho < BM) {
      const int r = min(rho, rows - 1);
      return (a_rows ? a_rows[row0 + r] : r) * lda + ch * 8;
    }
    if (rho < BM + NB * BNB) return min(n0 + (rho - BM) % BNB, N - 1) * K + ch * 8;
    return ch * 8;  // pad rows: any valid address (row 0 of the A tile)
  };

  constexpr int NRD = FM + NB * FN;   // fragment reads per slice
  constexpr int NMF = NB * FN * FM;   // MFMAs per slice
  if constexpr (PING) {
    // Two groups of four waves, one wave of each per SIMD, offset by half a
    // step: while one group runs its MFMAs the other reads its fragments from
    // LDS and writes the next stage into LDS; then they swap at a barrier.
    // Every wave runs the same loop -- a memory phase M(t), a barrier, a
    // compute phase C(t), a barrier -- and the second group starts one
    // barrier late, so its M(t) runs beside the first group's C(t).
    //
    // A step t covers K = 32 (two MFMA slices); an LDS stage holds K = 64
    // (128-byte rows, so every global load fetches whole 128-byte lines: 8
    // rows of 8 lanes per wavefront load, which the vector-memory path moves
    // at nearly twice the rate of 16 rows of 64 bytes).  Chunk c of row r
    // sits at c ^ ((r >> 1) & 7), so the 16 lanes an LDS cycle serves (16
    // consecutive rows of one chunk, or 2 rows of 8 chunks) hit distinct
    // banks.  Two LDS buffers, stage s in buffer s % 2.
    //
    // Tiles go global -> registers -> LDS.  M(t), t = 2s + h: read the
    // fragments of step t (half h of stage s) and write half h of stage s+1
    // (loaded two steps earlier into register set h).  C(t): the global
    // loads of half h of stage s+2 (into set h, just written out), then the
    // MFMAs of step t, so the vector-memory unit works through one group's
    // loads while the LDS serves the other group.  Stage
    // s+1's buffer last held stage s-1, read by both groups before the
    // barrier that precedes the first write; all four writes of stage s+1
    // land before the leading group's first read of it, two phases later.
    //
    // MXFP8 modes: the same schedule on E4M3 codes (a 128-byte LDS row holds
    // 128 codes, a step K = 64 codes, one scaled MFMA per fragment pair).
    // The E8M0 scale words (four blocks of a row per 128-code stage) travel
    // with the tiles: each wave loads the words of the 8-row chunks it
    // stages (lane L: chunk L/8, row L%8) with its first half stage, writes
    // them into the stage's scale area of LDS (one word per tile row) with
    // that half's rows, and reads the words of its fragment rows with the
    // fragments of the stage's first step.  Weight chunks never straddle the
    // end of the weight matrix (N is a multiple of 128), so their rows are
    // clamped per chunk and their offsets differ from one chunk to the next
    // only by a uniform term.
    constexpr int RW = kPingRowElems;
    // 32- and 64-row tiles (small experts): each weight row is read by one or
    // two row tiles only, so its loads are non-temporal and do not displace
    // the L2 lines that the big tiles of an interleaved launch reuse
    constexpr bool STREAM_W = BM <= 64;
    constexpr int PSTAGE = ROWS * RW;   // elements of one stage
    constexpr int NI = ROWS / (8 * NW); // 8-row loads per wave per stage
    constexpr int NH0 = (NI + 1) / 2;   // ... in the first half stage
    constexpr int NH1 = NI / 2;         // ... in the second
    constexpr int NA = MX ? (BM + 8 * NW - 1) / (8 * NW) : NI;  // chunks that may hold token rows
      static_assert(!MX || NI <= 16, "scale words: at most two per lane and stage");
    uint32_t* const sc_lds = reinterpret_cast<uint32_t*>(smem + 2 * PSTAGE);  // [2][ROWS] (MX)
    // scale word of tile row r sits at r ^ (((r >> 6) & 7) << 3): the eight
    // 8-row chunks a wavefront stores (rows 64 apart) then fall in distinct
    // banks, and 32 consecutive fragment rows stay in distinct banks
    auto sc_idx = [](int r) { return r ^ (((r >> 6) & 7) << 3); };
#define MOE_READ_FRAGS_P(set_, step_, ks_)                                              \
  do {                                                                                  \
    const uint16_t* sA_ = smem + (((step_) >> 1) & 1) * PSTAGE;                         \
    const uint16_t* sB0_ = sA_ + BM * RW;                                               \
    const uint16_t* sB1_ = sB0_ + BNB * RW;                                             \
    const int c_ = ((step_) & 1) * 4 + (ks_) * 2 + fk;                                  \
    _Pragma("unroll") for (int b = 0; b < FM; ++b) {                                    \
      const int r = wm * WM + b * 32 + fr;                                              \
      xa[set_][b] = *reinterpret_cast<const u32x4*>(sA_ + r * RW + ((c_ ^ ((r >> 1) & 7)) << 3)); \
    }                                                                                   \
    _Pragma("unroll") for (int a = 0; a < FN; ++a) {                                    \
      const int r = wn * WN + a * 32 + fr;                                              \
      wb0[set_][a] = *reinterpret_cast<const u32x4*>(sB0_ + r * RW + ((c_ ^ ((r >> 1) & 7)) << 3)); \
      if constexpr (DUAL)                                                               \
        wb1[set_][a] = *reinterpret_cast<const u32x4*>(sB1_ + r * RW + ((c_ ^ ((r >> 1) & 7)) << 3)); \
    }                                                                                   \
  } while (0)
    // MXFP8: chunks c and c + 2 of a step form one 32-byte operand; on the
    // first step of a stage also the scale words of the fragment rows
#define MOE_READ_FRAGS_MX(step_)                                                        \
  do {                                                                                  \
    const uint16_t* sA_ = smem + (((step_) >> 1) & 1) * PSTAGE;                         \
    const uint16_t* sB0_ = sA_ + BM * RW;                                               \
    const uint16_t* sB1_ = sB0_ + BNB * RW;                                             \
    const int c_ = ((step_) & 1) * 4 + fk;                                              \
    _Pragma("unroll") for (int b = 0; b < FM; ++b) {                                    \
      const int r = wm * WM + b * 32 + fr;                                              \
      const uint16_t* row_ = sA_ + r * RW;                                              \
      xa8[b] = cat8(*reinterpret_cast<const u32x4*>(row_ + ((c_ ^ ((r >> 1) & 7)) << 3)), \
                    *reinterpret_cast<const u32x4*>(row_ + (((c_ + 2) ^ ((r >> 1) & 7)) << 3))); \
    }                                                                                   \
    _Pragma("unroll") for (int a = 0; a < FN; ++a) {                                    \
      const int r = wn * WN + a * 32 + fr;                                              \
      const uint16_t* row0_ = sB0_ + r * RW;                                            \
      wg8[a] = cat8(*reinterpret_cast<const u32x4*>(row0_ + ((c_ ^ ((r >> 1) & 7)) << 3)), \
                    *reinterpret_cast<const u32x4*>(row0_ + (((c_ + 2) ^ ((r >> 1) & 7)) << 3))); \
      if constexpr (DUAL) {                                                             \
        const uint16_t* row1_ = sB1_ + r * RW;                                          \
        wu8[a] = cat8(*reinterpret_cast<const u32x4*>(row1_ + ((c_ ^ ((r >> 1) & 7)) << 3)), \
                      *reinterpret_cast<const u32x4*>(row1_ + (((c_ + 2) ^ ((r >> 1) & 7)) << 3))); \
      }                                                                                 \
    }                                                                                   \
    if (((step_) & 1) == 0) {                                                           \
      const uint32_t* sc_ = sc_lds + (((step_) >> 1) & 1) * ROWS;                       \
      _Pragma("unroll") for (int b = 0; b < FM; ++b) scc[b] = sc_[sc_idx(wm * WM + b * 32 + fr)]; \
      _Pragma("unroll") for (int a = 0; a < FN; ++a) {                                  \
        scc[FM + a] = sc_[sc_idx(BM + wn * WN + a * 32 + fr)];                          \
        if constexpr (DUAL) scc[FM + FN + a] = sc_[sc_idx(BM + BNB + wn * WN + a * 32 + fr)]; \
      }                                                                                 \
    }                                                                                   \
  } while (0)
    const bool lag = wave >= NW / 2;
    const int stages = kstn;
    // per-lane global offsets: every chunk (bf16 modes) or the chunks that may
    // hold token rows (MX); MX weight chunks share one lane offset
    int goff[NA];
#pragma unroll
    for (int j = 0; j < NA; ++j) goff[j] = row_goff(8 * (wave + NW * j) + (lane >> 3), lane & 7);
    const int lw = (lane >> 3) * K + (lane & 7) * 8;
    u32x4 ldr[2][NH0];
    // MX scale words: the current stage's words of this lane's fragments
    // (token fragments, then gate / down weight fragments, then up weight
    // fragments), shifted so that byte 2h selects the lane's block of step h
    constexpr int NSC = MX ? FM + NB * FN : 1;
    constexpr int NSL = MX ? (NI > 8 ? 2 : 1) : 1;  // scale-word loads per lane and stage
    uint32_t scc[NSC];
    uint32_t scl[NSL];           // staged words (loaded with half 0, written with half 0)
    const uint32_t* scp[NSL];    // this lane's scale rows (group 0) ...
    int scs[NSL];                // ... and their group stride
    if constexpr (MX) {
#pragma unroll
      for (int q = 0; q < NSL; ++q) {
        const int rho = 8 * (wave + NW * (8 * q + (lane >> 3))) + (lane & 7);
        const uint32_t* base;
        int row, strd;
        if (rho < BM) {
          const int r = min(rho, rows - 1);
          base = reinterpret_cast<const uint32_t*>(mx.sa);
          row = (a_rows && !mx.sa_direct) ? a_rows[row0 + r] : row0 + r;
          strd = mx.sa_stride;
        } else if (rho < BM + NB * BNB) {
          base = reinterpret_cast<const uint32_t*>(rho < BM + BNB ? mx.sb0 : mx.sb1);
          row = expert * N + min(n0 + (rho - BM) % BNB, N - 1);
          strd = mx.sb_stride;
        } else {  // pad rows: any valid word (never read back)
          base = reinterpret_cast<const uint32_t*>(mx.sb0);
          row = expert * N;
          strd = mx.sb_stride;
        }
        scp[q] = base + row + (size_t)kst0 * strd;
        scs[q] = strd;
      }
    }
#define MOE_ISSUE_SC(stage_)                                                            \
  do {                                                                                  \
    if constexpr (MX) {                                                                 \
      const int st_ = (stage_) < stages ? (stage_) : stages - 1;                        \
      _Pragma("unroll") for (int q = 0; q < NSL; ++q) {                                 \
        if (8 * q + (lane >> 3) < NI) scl[q] = scp[q][(size_t)st_ * scs[q]];            \
      }                                                                                 \
    }                                                                                   \
  } while (0)
#define MOE_STORE_SC(stage_)                                                            \
  do {                                                                                  \
    if constexpr (MX) {                                                                 \
      _Pragma("unroll") for (int q = 0; q < NSL; ++q) {                                 \
        if (8 * q + (lane >> 3) < NI)                                                   \
          sc_lds[((stage_) & 1) * ROWS + sc_idx(8 * (wave + NW * (8 * q + (lane >> 3))) + (lane & 7))] = scl[q]; \
      }                                                                                 \
    }                                                                                   \
  } while (0)
#define MOE_ISSUE(set_, stage_, half_)                                                  \
  do {                                                                                  \
    const int st_ = (stage_) < stages ? (stage_) : stages - 1;                          \
    _Pragma("unroll") for (int jj = 0; jj < ((half_) ? NH1 : NH0); ++jj) {              \
      const int j_ = (half_) * NH0 + jj;                                                \
      const int r0_ = 8 * (wave + NW * j_);                                             \
      const uint16_t* src_;                                                             \
      if constexpr (MX) {                                                               \
        if (j_ < NA && r0_ < BM) {                                                      \
          src_ = Ab + goff[j_ < NA ? j_ : 0];                                           \
        } else if (r0_ < BM + NB * BNB) {                                               \
          const int rb_ = min(n0 + (r0_ - BM) % BNB, N - 8);                            \
          src_ = (r0_ < BM + BNB ? B0b : B1b) + (size_t)rb_ * K + lw;                   \
        } else {                                                                        \
          src_ = Ab + (lane & 7) * 8;                                                   \
        }                                                                               \
      } else {                                                                          \
        src_ = (r0_ < BM ? Ab : (r0_ < BM + BNB ? B0b : (r0_ < BM + NB * BNB ? B1b : Ab))) + goff[j_]; \
      }                                                                                 \
      if (STREAM_W && r0_ >= BM)                                                        \
        ldr[set_][jj] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src_ + st_ * RW)); \
      else                                                                              \
        ldr[set_][jj] = *reinterpret_cast<const u32x4*>(src_ + st_ * RW);               \
    }                                                                                   \
  } while (0)
#define MOE_STORE(set_, stage_, half_)                                                  \
  do {                                                                                  \
    uint16_t* base_ = smem + ((stage_) & 1) * PSTAGE;                                   \
    _Pragma("unroll") for (int jj = 0; jj < ((half_) ? NH1 : NH0); ++jj) {              \
      const int j_ = (half_) * NH0 + jj;                                                \
      const int r0_ = 8 * (wave + NW * j_);                                             \
      const int row_ = r0_ + (lane >> 3);                                               \
      u32x4 v_ = ldr[set_][jj];                                                         \
      if (MODE == kDown && r0_ >= BM && r0_ < BM + BNB) v_ = bf16x8_to_f16x8(v_);       \
      *reinterpret_cast<u32x4*>(base_ + row_ * RW + (((lane & 7) ^ ((row_ >> 1) & 7)) << 3)) = v_; \
    }                                                                                   \
    if ((half_) == 0) MOE_STORE_SC(stage_);                                             \
  } while (0)
#define MOE_PP_STEP(tt_, h_)                                                            \
  do {                                                                                  \
    if constexpr (MX) {                                                                 \
      MOE_READ_FRAGS_MX(tt_);                                                           \
    } else {                                                                            \
      MOE_READ_FRAGS_P(0, (tt_), 0);                                                    \
      MOE_READ_FRAGS_P(1, (tt_), 1);                                                    \
    }                                                                                   \
    MOE_STORE(h_, ((tt_) >> 1) + 1, h_);                                                \
    __builtin_amdgcn_sched_barrier(0);                                                  \
    MOE_WAIT_LGKM0();                                                                   \
    raw_barrier();                                                                      \
    __builtin_amdgcn_sched_barrier(0);                                                  \
    __builtin_amdgcn_s_setprio(1);                                                      \
    if constexpr (MX) {                                                                 \
      if ((h_) == 0) {                                                                  \
        _Pragma("unroll") for (int f = 0; f < NSC; ++f) scc[f] >>= 8 * fk;              \
        MOE_ISSUE_SC(((tt_) >> 1) + 2);                                                 \
      }                                                                                 \
    }                                                                                   \
    MOE_ISSUE(h_, ((tt_) >> 1) + 2, h_);                                                \
    if constexpr (MX) {                                                                 \
      MOE_MFMAS_MX(h_);                                                                 \
    } else {                                                                            \
      MOE_MFMAS(0);                                                                     \
      MOE_MFMAS(1);                                                                     \
    }                                                                                   \
    __builtin_amdgcn_sched_group_barrier(0x020, ((h_) ? NH1 : NH0) + (MX && (h_) == 0 ? NSL : 0), 3); \
    __builtin_amdgcn_sched_group_barrier(0x008, MX ? NMF : 2 * NMF, 3);                 \
    __builtin_amdgcn_s_setprio(0);                                                      \
    __builtin_amdgcn_sched_barrier(0);                                                  \
    raw_barrier();                                                                      \
    __builtin_amdgcn_sched_barrier(0);                                                  \
  } while (0)
    MOE_ISSUE_SC(0);
    MOE_ISSUE(0, 0, 0);
    MOE_ISSUE(1, 0, 1);
    MOE_STORE(0, 0, 0);
    MOE_STORE(1, 0, 1);
    MOE_ISSUE_SC(1);
    MOE_ISSUE(0, 1, 0);
    MOE_ISSUE(1, 1, 1);
    MOE_WAIT_LGKM0();
    raw_barrier();
    if (lag) raw_barrier();
    // two steps per stage (K is a multiple of 64), so register sets alternate statically
    for (int t = 0; t < 2 * stages; t += 2) {
      MOE_PP_STEP(t, 0);
      MOE_PP_STEP(t + 1, 1);
    }
    if (!lag) raw_barrier();
#undef MOE_PP_STEP
#undef MOE_READ_FRAGS_MX
#undef MOE_ISSUE_SC
#undef MOE_STORE_SC
#undef MOE_STORE
#undef MOE_ISSUE
#undef MOE_READ_FRAGS_P
  } else {
    // 4-wave blocks.  Tiles move from global memory straight into LDS with
    // global_load_lds_dwordx4 (lane L of a wavefront writes 16 bytes at LDS
    // base + 16 L), so no registers stage them.  A stage covers 32 K
    // elements: rows [A tile | B0 tile | B1 tile | pad], each 64 bytes = four
    // 16-byte chunks, chunk c of row r stored at c ^ ((r >> 2) & 3) so the 16
    // rows one 16-lane phase of a fragment read touches fall in distinct
    // banks; the swizzle is applied on the global side by choosing the chunk
    // each lane fetches.  NS stages form a ring: NS - 2 stages stay in flight
    // ahead of the one being multiplied.
    //
    // Per step (one stage, two K=16 MFMA slices): the second slice's
    // fragments are read, the first slice's MFMAs run, the wave waits for
    // its loads of the next stage and meets the others at a barrier, the
    // loads NS-1 stages ahead are issued into the stage freed one step ago,
    // the next step's first-slice fragments are read, and the second slice's
    // MFMAs run -- so fragment reads and loads always overlap queued MFMAs.
    constexpr int STAGE = ROWS * kSK;      // elements of one stage
    constexpr int NL = ROWS / (16 * NW);   // 16-row loads per wave per stage
    static_assert(NS >= 3 && NL * (NS - 2) <= 63, "pipeline depth");
    // load i of this wave fills stage rows 16*(wave + NW i) .. +16; lane -> (row, chunk)
    int goff[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int rho = 16 * (wave + NW * i) + (lane >> 2);
      goff[i] = row_goff(rho, (lane & 3) ^ ((rho >> 2) & 3));
    }
    const int steps = kstn * (kPingRowElems / kSK);
#define MOE_LOAD_STAGE(step_)                                                           \
  do {                                                                                  \
    const int st_ = (step_) < steps ? (step_) : steps - 1;                              \
    uint16_t* base_ = smem + ((step_) % NS) * STAGE;                                    \
    _Pragma("unroll") for (int i = 0; i < NL; ++i) {                                    \
      const int r0_ = 16 * (wave + NW * i);                                             \
      const uint16_t* src_ = r0_ < BM ? Ab : (r0_ < BM + BNB ? B0b : (r0_ < BM + NB * BNB ? B1b : Ab)); \
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(src_ + goff[i] + st_ * kSK),         \
                                       (lds_ptr_t)(base_ + r0_ * kSK), 16, 0, 0);       \
    }                                                                                   \
  } while (0)
    // fragments of slice ks (0/1) of the stage holding `step_` into set `set_`
#define MOE_READ_FRAGS(set_, step_, ks_)                                                \
  do {                                                                                  \
    const uint16_t* sA_ = smem + ((step_) % NS) * STAGE;                                \
    const uint16_t* sB0_ = sA_ + BM * kSK;                                              \
    const uint16_t* sB1_ = sB0_ + BNB * kSK;                                            \
    const int c_ = (ks_) * 2 + fk;                                                      \
    _Pragma("unroll") for (int b = 0; b < FM; ++b) {                                    \
      const int r = wm * WM + b * 32 + fr;                                              \
      xa[set_][b] = *reinterpret_cast<const u32x4*>(sA_ + r * kSK + ((c_ ^ ((r >> 2) & 3)) << 3)); \
    }                                                                                   \
    _Pragma("unroll") for (int a = 0; a < FN; ++a) {                                    \
      const int r = wn * WN + a * 32 + fr;                                              \
      wb0[set_][a] = *reinterpret_cast<const u32x4*>(sB0_ + r * kSK + ((c_ ^ ((r >> 2) & 3)) << 3)); \
      if constexpr (DUAL)                                                               \
        wb1[set_][a] = *reinterpret_cast<const u32x4*>(sB1_ + r * kSK + ((c_ ^ ((r >> 2) & 3)) << 3)); \
    }                                                                                   \
  } while (0)
    // prologue: stages 0 .. NS-2 in flight; wait for stage 0; first slice of step 0
#pragma unroll
    for (int s0 = 0; s0 < NS - 1; ++s0) MOE_LOAD_STAGE(s0);
    MOE_WAIT_VMCNT(NL * (NS - 2));
    raw_barrier();
    MOE_READ_FRAGS(0, 0, 0);
    for (int t = 0; t < steps; ++t) {
      // region 1: slice-0 MFMAs with the slice-1 fragment reads between them
      MOE_READ_FRAGS(1, t, 1);
      MOE_MFMAS(0);
#pragma unroll
      for (int q = 0; q < NMF; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);            // MFMA
        if (q < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);  // DS read
      }
      __builtin_amdgcn_sched_barrier(0);
      MOE_WAIT_VMCNT(NL * (NS - 3));  // this wave's loads of step t+1 have landed
      raw_barrier();                  // ... and every wave's; step t-1's stage is free
      __builtin_amdgcn_sched_barrier(0);
      // region 2: slice-1 MFMAs with the loads NS-1 steps ahead and the next
      // step's slice-0 fragment reads between them (on the last step that read
      // is of a stale stage and unused)
      MOE_LOAD_STAGE(t + NS - 1);
      MOE_READ_FRAGS(0, t + 1, 0);
      MOE_MFMAS(1);
#pragma unroll
      for (int q = 0; q < NMF; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);             // MFMA
        if (q < NL) __builtin_amdgcn_sched_group_barrier(0x020, 1, 2);   // VMEM load
        if (q < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 2);  // DS read
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#undef MOE_READ_FRAGS
#undef MOE_LOAD_STAGE
  }
#undef MOE_MFMAS
#undef MOE_MFMAS_MX
  __builtin_amdgcn_s_waitcnt(0);  // drain the clamped tail loads before the block ends

  // epilogue: accumulator q of fragment (a, b) is output column
  // n = a*32 + 8*(q/4) + 4*(lane/32) + q%4 of token row m = b*32 + lane%32
  bool overflow = false;
  // Gate/up outputs: the 32 columns of fragment (a, b) in token row m sit in
  // lanes l (columns 8q + 0..3) and l ^ 32 (8q + 4..7), q = 0..3.  One
  // v_permlane32_swap per pair of words gives lane l the columns 0..15 and
  // lane l ^ 32 the columns 16..31 of the row, each stored as whole 16-byte
  // chunks (one per lane for E4M3 codes, two for fp16) instead of four
  // scattered 4- or 8-byte stores.  Cross-lane steps run on every lane; the
  // row and column bounds only gate the stores.
  if constexpr (MODE == kGateUpMX) {
    // the block's maximum magnitude (both lane halves) sets its E8M0 scale;
    // lane l < 32 also writes the scale byte
#pragma unroll
    for (int b = 0; b < FM; ++b) {
      const int m = wm * WM + b * 32 + fr;
#pragma unroll
      for (int a = 0; a < FN; ++a) {
        const int nb = n0 + wn * WN + a * 32;
        float hv[16];
        float amax = 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          hv[q] = silu_mul(acc0[a][b][q], acc1[a][b][q]);
          amax = fmaxf(amax, fabsf(hv[q]));
        }
        const auto am = __builtin_amdgcn_permlane32_swap(__float_as_uint(amax), __float_as_uint(amax),
                                                         false, false);
        amax = fmaxf(amax, __uint_as_float(fk ? am[0] : am[1]));
        const uint32_t sb = mx_scale_byte(amax);
        const int sh = 127 - (int)sb;
        uint32_t w[4];
#pragma unroll
        for (int qi = 0; qi < 4; ++qi)
          w[qi] = e4m3x4(ldexpf(hv[4 * qi], sh), ldexpf(hv[4 * qi + 1], sh), ldexpf(hv[4 * qi + 2], sh),
                         ldexpf(hv[4 * qi + 3], sh));
        const auto s02 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
        const auto s13 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
        if (m >= rows || nb >= N) continue;
        overflow |= !(amax <= 3.402823466e38f);
        *reinterpret_cast<u32x4*>(static_cast<uint8_t*>(Out) + (size_t)(row0 + m) * ldo + nb + 16 * fk) =
            u32x4{s02[0], s02[1], s13[0], s13[1]};
        if (fk == 0)
          mx.sout[((size_t)(nb >> 7) * mx.sout_stride + row0 + m) * 4 + ((nb >> 5) & 3)] =
              (uint8_t)sb;
      }
    }
  } else if constexpr (MODE == kGateUp) {
    // fp16 h (N is a multiple of 64, so a 32-column block is all in or out)
#pragma unroll
    for (int b = 0; b < FM; ++b) {
      const int m = wm * WM + b * 32 + fr;
#pragma unroll
      for (int a = 0; a < FN; ++a) {
        const int nb = n0 + wn * WN + a * 32;
        const f32x16 g = acc0[a][b], u = acc1[a][b];
        uint32_t px[4], py[4];
        bool ovf = false;
#pragma unroll
        for (int qi = 0; qi < 4; ++qi) {
          const float h0 = silu_mul(g[4 * qi], u[4 * qi]);
          const float h1 = silu_mul(g[4 * qi + 1], u[4 * qi + 1]);
          const float h2 = silu_mul(g[4 * qi + 2], u[4 * qi + 2]);
          const float h3 = silu_mul(g[4 * qi + 3], u[4 * qi + 3]);
          ovf |= !(fabsf(h0) <= 65504.f && fabsf(h1) <= 65504.f && fabsf(h2) <= 65504.f &&
                   fabsf(h3) <= 65504.f);
          px[qi] = f32_to_f16_bits(h0) | (f32_to_f16_bits(h1) << 16);
          py[qi] = f32_to_f16_bits(h2) | (f32_to_f16_bits(h3) << 16);
        }
        const auto x02 = __builtin_amdgcn_permlane32_swap(px[0], px[2], false, false);
        const auto y02 = __builtin_amdgcn_permlane32_swap(py[0], py[2], false, false);
        const auto x13 = __builtin_amdgcn_permlane32_swap(px[1], px[3], false, false);
        const auto y13 = __builtin_amdgcn_permlane32_swap(py[1], py[3], false, false);
        if (m >= rows || nb >= N) continue;
        overflow |= ovf;
        uint16_t* dst = static_cast<uint16_t*>(Out) + (size_t)(row0 + m) * ldo + nb + 16 * fk;
        *reinterpret_cast<u32x4*>(dst) = u32x4{x02[0], y02[0], x02[1], y02[1]};
        *reinterpret_cast<u32x4*>(dst + 8) = u32x4{x13[0], y13[0], x13[1], y13[1]};
      }
    }
  } else if (!gemm_part(MODE) && out_half) {
    // fp16 outputs (a layer's down projection), stored as the gate/up
    // epilogue stores h: after the lane-half exchanges lane l holds columns
    // 0..15 and lane l ^ 32 columns 16..31 of its row, two 16-byte stores
    // each instead of four 8-byte ones (the stores had been the largest part
    // of a short-K tile's epilogue)
#pragma unroll
    for (int b = 0; b < FM; ++b) {
      const int m = wm * WM + b * 32 + fr;
#pragma unroll
      for (int a = 0; a < FN; ++a) {
        const int nb = n0 + wn * WN + a * 32;
        const f32x16 v = acc0[a][b];
        uint32_t px[4], py[4];
        bool ovf = false;
#pragma unroll
        for (int qi = 0; qi < 4; ++qi) {
          ovf |= !(fabsf(v[4 * qi]) <= 65504.f && fabsf(v[4 * qi + 1]) <= 65504.f &&
                   fabsf(v[4 * qi + 2]) <= 65504.f && fabsf(v[4 * qi + 3]) <= 65504.f);
          px[qi] = f32_to_f16_bits(v[4 * qi]) | (f32_to_f16_bits(v[4 * qi + 1]) << 16);
          py[qi] = f32_to_f16_bits(v[4 * qi + 2]) | (f32_to_f16_bits(v[4 * qi + 3]) << 16);
        }
        const auto x02 = __builtin_amdgcn_permlane32_swap(px[0], px[2], false, false);
        const auto y02 = __builtin_amdgcn_permlane32_swap(py[0], py[2], false, false);
        const auto x13 = __builtin_amdgcn_permlane32_swap(px[1], px[3], false, false);
        const auto y13 = __builtin_amdgcn_permlane32_swap(py[1], py[3], false, false);
        if (m >= rows || nb >= N) continue;
        overflow |= ovf;
        uint16_t* dst = static_cast<uint16_t*>(Out) + (size_t)(row0 + m) * ldo + nb + 16 * fk;
        *reinterpret_cast<u32x4*>(dst) = u32x4{x02[0], y02[0], x02[1], y02[1]};
        *reinterpret_cast<u32x4*>(dst + 8) = u32x4{x13[0], y13[0], x13[1], y13[1]};
      }
    }
  } else {
#pragma unroll
  for (int b = 0; b < FM; ++b) {
    const int m = wm * WM + b * 32 + fr;
    if (m >= rows) continue;
#pragma unroll
    for (int a = 0; a < FN; ++a) {
#pragma unroll
      for (int qi = 0; qi < 4; ++qi) {
        const int n = n0 + wn * WN + a * 32 + 8 * qi + 4 * fk;
        const size_t o = (size_t)(row0 + m) * ldo + n;
#pragma unroll
        for (int ob = 0; ob < (gemm_part(MODE) ? 2 : 1); ++ob) {
          const f32x16 acc = ob ? acc1[DUAL ? a : 0][DUAL ? b : 0] : acc0[a][b];
          f32x4 v = {acc[4 * qi], acc[4 * qi + 1], acc[4 * qi + 2], acc[4 * qi + 3]};
          float* dst = static_cast<float*>(Out) + o + (ob ? up_off : 0);
          if (n + 3 < N && (ldo & 3) == 0) {
            if (bias) {
              v[0] += bias[n];
              v[1] += bias[n + 1];
              v[2] += bias[n + 2];
              v[3] += bias[n + 3];
            }
            *reinterpret_cast<f32x4*>(dst) = v;
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (n + q < N) dst[q] = v[q] + (bias ? bias[n + q] : 0.0f);
          }
        }
      }
    }
  }
  }
  if (overflow && flags) atomicOr(flags, DUAL ? (uint32_t)MOE_FLAG_H_RANGE : (uint32_t)MOE_FLAG_Y_RANGE);
}

// Small-expert tiles of at most kSkinnyRows token rows in the interleaved
// launches (bf16 gate/up and the down projection).  A 64-row MFMA tile runs
// 16 to 64 times the needed MFMA work on such a tile (clamped duplicate rows),
// and inside a power-limited interleaved launch its ping-pong schedule streams
// the weights at about 33 GB/s per compute unit; this tile streams about 55
// GB/s there, the rate of the unit's memory path (alone, at a higher clock,
// both reach about 50 GB/s, and about 7 TB/s together when every unit runs
// one).  Here the weights go from memory straight into registers in whole
// 128-byte lines (8
// rows x 8 lanes per wavefront load) and the vector ALUs form the dot
// products: v_dot2 (two products per lane and instruction, fp32 sums) on bf16
// pairs for gate/up and on fp16 pairs for the down projection, whose bf16
// weights are converted to fp16 by the conversion the MFMA tiles apply.
//
// Wave w owns output columns n0 + 32w .. n0 + 32w + 31 (all in range or all
// out: N is a multiple of 64).  Lane l takes 16-byte chunk l % 8 of every
// 64-element K segment of weight rows n0 + 32w + 8g + l / 8 (g = 0..3; of
// both matrices for gate/up) and of each token row, so it holds partial sums
// for 4 (or 2 x 4) weight rows x R token rows; the 8 lanes of a weight row
// then add theirs across lanes and lane 8j + 2g writes column
// n0 + 32w + 8g + j.  D segments of loads stay in flight.  Rows past t.rows
// (R = 4 for three rows) repeat the last row and are not stored.
constexpr int kSkinnyRows = 4;

constexpr bool skinny_mode(int MODE) { return MODE == kGateUp || MODE == kDown || MODE == kDownW16; }

template <int R, int MODE, int BNB>
__device__ __forceinline__ void skinny_tile(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ a_rows, int lda,
    const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1, long long strideB, int N, int K,
    void* __restrict__ Out, int ldo, uint32_t* __restrict__ flags, const MTile t, int ni, int kst0,
    int kstn, bool out_half) {
  static_assert(BNB == 256, "eight waves of 32 columns");
  constexpr bool DUAL = MODE == kGateUp;
  constexpr int NB = DUAL ? 2 : 1;
  constexpr int D = DUAL ? 4 : 6;
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cw = ni * BNB + 32 * wave;
  if (cw >= N || t.rows < 1 || kstn < 1) return;
  const int j = lane >> 3, c = lane & 7;
  // Buffer loads: one resource per weight matrix (the expert's, from the
  // block's first K segment) and per token row, a lane offset per row group,
  // and the segment's byte offset in a scalar register, so a load needs no
  // address registers of its own.  Every offset fits 32 bits (an expert's
  // matrix and a row hold fewer than 2^31 elements); reads past a resource's
  // end return zeros.
  const size_t k0 = (size_t)kst0 * kPingRowElems;
  const uint32_t wbytes = (uint32_t)(((size_t)N * K - k0) * 2);
  const __amdgpu_buffer_rsrc_t rw0 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(B0 + (size_t)t.expert * strideB + k0), 0, wbytes, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t rw1 = DUAL ? __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(B1 + (size_t)t.expert * strideB + k0), 0, wbytes, kBufferRsrcWord3) : rw0;
  const uint32_t xbytes = (uint32_t)(((size_t)K - k0) * 2);
  __amdgpu_buffer_rsrc_t rx[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int rr = t.row0 + min(r, t.rows - 1);
    const int row = __builtin_amdgcn_readfirstlane(a_rows ? a_rows[rr] : rr);
    rx[r] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(A + (size_t)row * lda + k0), 0, xbytes,
                                              kBufferRsrcWord3);
  }
  int wo[4];  // byte offsets below 2^32, passed as their 32-bit pattern
#pragma unroll
  for (int g = 0; g < 4; ++g)
    wo[g] = __builtin_bit_cast(int, ((uint32_t)(cw + 8 * g + j) * (uint32_t)K + 8u * c) * 2u);
  const int xo = 16 * c;
  u32x4 wv[D][NB][4];
  u32x4 xv[D][R];
  float acc[NB][4][R];
#pragma unroll
  for (int m = 0; m < NB; ++m)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[m][g][r] = 0.f;
  // weight lines are read once: non-temporal (aux bit 1)
#define MOE_SK_ISSUE(d_, seg_)                                                          \
  do {                                                                                  \
    const int so_ = (seg_) * (kPingRowElems * 2);                                       \
    _Pragma("unroll") for (int g = 0; g < 4; ++g) {                                     \
      wv[d_][0][g] = __builtin_amdgcn_raw_buffer_load_b128(rw0, wo[g], so_, 2);         \
      if constexpr (DUAL) wv[d_][NB - 1][g] = __builtin_amdgcn_raw_buffer_load_b128(rw1, wo[g], so_, 2); \
    }                                                                                   \
    _Pragma("unroll") for (int r = 0; r < R; ++r)                                       \
      xv[d_][r] = __builtin_amdgcn_raw_buffer_load_b128(rx[r], xo, so_, 0);             \
  } while (0)
#define MOE_SK_DOT(d_)                                                                  \
  do {                                                                                  \
    _Pragma("unroll") for (int m = 0; m < NB; ++m) {                                    \
      _Pragma("unroll") for (int g = 0; g < 4; ++g) {                                   \
        const u32x4 w_ = MODE == kDown ? bf16x8_to_f16x8(wv[d_][m][g]) : wv[d_][m][g];   \
        _Pragma("unroll") for (int r = 0; r < R; ++r) {                                 \
          _Pragma("unroll") for (int q = 0; q < 4; ++q) {                               \
            /* words copied out first: a bit_cast of a vector element reads */          \
            /* element 0 with this compiler */                                          \
            const uint32_t wq_ = w_[q], xq_ = xv[d_][r][q];                             \
            if constexpr (DUAL)                                                         \
              acc[m][g][r] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wq_), \
                  __builtin_bit_cast(bf16x2_t, xq_), acc[m][g][r], false);             \
            else                                                                        \
              acc[m][g][r] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, wq_),    \
                  __builtin_bit_cast(f16x2_t, xq_), acc[m][g][r], false);              \
          }                                                                             \
        }                                                                               \
      }                                                                                 \
    }                                                                                   \
  } while (0)
  // segments 0 .. D-1 in flight; each step multiplies one and issues the one D
  // ahead (clamped to the last: re-read lines, never used)
#pragma unroll
  for (int d = 0; d < D; ++d) MOE_SK_ISSUE(d, min(d, kstn - 1));
  const int full = kstn - kstn % D;
  for (int s = 0; s < full; s += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      // fences keep the scheduler from hoisting the next loads above the
      // products (longer live ranges, then waits for every load in flight)
      MOE_SK_DOT(d);
      __builtin_amdgcn_sched_barrier(0);
      MOE_SK_ISSUE(d, min(s + d + D, kstn - 1));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (d < kstn - full) MOE_SK_DOT(d);
  __builtin_amdgcn_s_waitcnt(0);  // drain the clamped loads before the block ends
#undef MOE_SK_DOT
#undef MOE_SK_ISSUE
  // The 8 lanes of a weight row add their partial sums, halving the values
  // each lane holds at every exchange: lanes c and c ^ 4 split the row groups
  // {0, 1} / {2, 3}, then c and c ^ 2 split those, then c and c ^ 1 add.  Lanes
  // c and c ^ 1 end with the same sum (fp addition commutes), of row group
  // g = c / 2 for even c.
  float res[NB][R];
  const bool hi4 = (c & 4) != 0, hi2 = (c & 2) != 0;
#pragma unroll
  for (int m = 0; m < NB; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float k0 = hi4 ? acc[m][2][r] : acc[m][0][r], k1 = hi4 ? acc[m][3][r] : acc[m][1][r];
      const float s0 = hi4 ? acc[m][0][r] : acc[m][2][r], s1 = hi4 ? acc[m][1][r] : acc[m][3][r];
      k0 += __shfl_xor(s0, 4);
      k1 += __shfl_xor(s1, 4);
      float k = hi2 ? k1 : k0;
      k += __shfl_xor(hi2 ? k0 : k1, 2);
      k += __shfl_xor(k, 1);
      res[m][r] = k;
    }
  if (c & 1) return;
  const int col = cw + 4 * c + j;   // row group c / 2: column cw + 8 (c / 2) + j
  bool overflow = false;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r >= t.rows) break;
    const size_t o = (size_t)(t.row0 + r) * ldo + col;
    if constexpr (DUAL) {
      const float h = silu_mul(res[0][r], res[NB - 1][r]);
      overflow |= !(fabsf(h) <= 65504.f);
      static_cast<uint16_t*>(Out)[o] = (uint16_t)f32_to_f16_bits(h);
    } else if (out_half) {
      overflow |= !(fabsf(res[0][r]) <= 65504.f);
      static_cast<uint16_t*>(Out)[o] = (uint16_t)f32_to_f16_bits(res[0][r]);
    } else {
      static_cast<float*>(Out)[o] = res[0][r];
    }
  }
  if (overflow && flags) atomicOr(flags, DUAL ? (uint32_t)MOE_FLAG_H_RANGE : (uint32_t)MOE_FLAG_Y_RANGE);
}

// One row-tile class per launch: block -> (row tile, column tile) by block_tile.
// ksplit > 1 splits K into that many ranges of whole 64-element stages; the
// blocks of range p write their partial sums to Out + p * part_elems (fp32
// outputs only), and the consumer adds the parts in order.
template <int BM, int BNB, int MODE, int NS, int NW>
__global__ __launch_bounds__(64 * NW) void k_gemm_mfma(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ a_rows, int lda,
    const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, long long strideB, int N, int K, void* __restrict__ Out,
    int ldo, const float* __restrict__ bias, const MTile* __restrict__ sched,
    const int32_t* __restrict__ count, int mslots, int ntiles, int static_rows,
    uint32_t* __restrict__ flags, const MxArgs mx, int ksplit, long long part_elems, int out_half,
    int group_m) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  int mi, nn;
  const int mtiles = sched ? min(*count, mslots) : (static_rows + BM - 1) / BM;
  if (!block_tile(mtiles, ntiles * ksplit, mi, nn, group_m)) return;
  const int part = nn % ksplit, ni = nn / ksplit;
  const int stages = K / kPingRowElems;
  const int kst0 = part * stages / ksplit, kst1 = (part + 1) * stages / ksplit;
  if (part) {
    Out = static_cast<float*>(Out) + part * part_elems;
    bias = nullptr;  // added once, by part 0
  }
  gemm_tile<BM, BNB, MODE, NS, NW>(smem, A, a_rows, lda, B0, B1, strideB, N, K, Out, ldo, bias, sched,
                                   static_rows, flags, mx, mi, ni, kst0, kst1 - kst0,
                                   gemm_part(MODE) ? ksplit * part_elems : 0, out_half != 0);
}

// Both row-tile classes of a skewed layer in one launch (8-wave blocks): the
// big-expert tiles (BM1 rows, MFMA-bound) and the small-expert tiles (BM2
// rows, weight-streaming, HBM-bound) are interleaved through the grid
// (block_tile2), so at any time some compute units stream weights while the
// others run MFMAs, instead of the two classes running one after the other.
// ksplit > 1 (fp32 outputs only) splits K of every tile of both classes as
// in k_gemm_mfma: part p of a tile writes its partial sums at Out + p *
// part_elems.
template <int BM1, int BNB1, int BM2, int BNB2, int MODE>
__global__ __launch_bounds__(512) void k_gemm_mfma2(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ a_rows, int lda,
    const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1, long long strideB, int N,
    int K, void* __restrict__ Out, int ldo, uint32_t* __restrict__ flags, const MxArgs mx,
    const MTile* __restrict__ sched1, const int32_t* __restrict__ count1, int mslots1,
    int ntiles1, const MTile* __restrict__ sched2, const int32_t* __restrict__ count2,
    int mslots2, int ntiles2, int ksplit, long long part_elems, int out_half, int group_m) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const int m1 = min(*count1, mslots1), m2 = min(*count2, mslots2);
  int cls, idx, mi, nn;
  if (!block_tile2(m1 * ntiles1 * ksplit, m2 * ntiles2 * ksplit, cls, idx)) return;
  if (cls == 0) tile_of(idx, m1, ntiles1 * ksplit, mi, nn, group_m);
  else tile_of(idx, m2, ntiles2 * ksplit, mi, nn, kGroupM);
  const int part = nn % ksplit, ni = nn / ksplit;
  const int stages = K / kPingRowElems;
  const int kst0 = part * stages / ksplit, kst1 = (part + 1) * stages / ksplit;
  if (part) Out = static_cast<float*>(Out) + part * part_elems;
  if (cls == 0) {
    gemm_tile<BM1, BNB1, MODE, 2, 8>(smem, A, a_rows, lda, B0, B1, strideB, N, K, Out, ldo, nullptr,
                                     sched1, 0, flags, mx, mi, ni, kst0, kst1 - kst0, 0, out_half != 0);
  } else {
    if constexpr (skinny_mode(MODE)) {
      const MTile t = sched2[mi];
      if (t.rows <= kSkinnyRows) {
        if (t.rows == 1)
          skinny_tile<1, MODE, BNB2>(A, a_rows, lda, B0, B1, strideB, N, K, Out, ldo, flags, t, ni, kst0,
                                     kst1 - kst0, out_half != 0);
        else if (t.rows == 2)
          skinny_tile<2, MODE, BNB2>(A, a_rows, lda, B0, B1, strideB, N, K, Out, ldo, flags, t, ni, kst0,
                                     kst1 - kst0, out_half != 0);
        else
          skinny_tile<4, MODE, BNB2>(A, a_rows, lda, B0, B1, strideB, N, K, Out, ldo, flags, t, ni, kst0,
                                     kst1 - kst0, out_half != 0);
        return;
      }
    }
    // small tiles of at most 32 rows run as 32-row tiles: the weight stream of
    // a small tile is bound by the LDS traffic of its stages, which a 32-row
    // tile cuts by about a quarter (one token fragment per wave instead of
    // weight fragments read by two wave rows)
    if constexpr (BM2 > 32) {
      if (sched2[mi].rows <= 32) {
        gemm_tile<32, BNB2, MODE, 2, 8>(smem, A, a_rows, lda, B0, B1, strideB, N, K, Out, ldo, nullptr,
                                        sched2, 0, flags, mx, mi, ni, kst0, kst1 - kst0, 0, out_half != 0);
        return;
      }
    }
    gemm_tile<BM2, BNB2, MODE, 2, 8>(smem, A, a_rows, lda, B0, B1, strideB, N, K, Out, ldo, nullptr,
                                     sched2, 0, flags, mx, mi, ni, kst0, kst1 - kst0, 0, out_half != 0);
  }
}

// fp32 grouped GEMM: 32x32 output tile (per B matrix), 2x2 outputs per thread,
// K step 16.  Used by fp32 layers, whose sizes make it latency-bound.
template <bool DUAL>
__global__ __launch_bounds__(256) void k_gemm_f32(const float* __restrict__ A,
                                                  const int32_t* __restrict__ a_rows, int lda,
                                                  const float* __restrict__ B0,
                                                  const float* __restrict__ B1,
                                                  long long strideB, int N, int K,
                                                  float* __restrict__ Out, int ldo,
                                                  const float* __restrict__ bias,
                                                  const MTile* __restrict__ sched,
                                                  const int32_t* __restrict__ count, int mslots,
                                                  int ntiles, int static_rows) {
  constexpr int TB = 32, TK = 16;
  int mi, ni;
  const int mtiles = sched ? min(*count, mslots) : (static_rows + TB - 1) / TB;
  if (!block_tile(mtiles, ntiles, mi, ni, kGroupM)) return;
  int expert = 0, row0, rows;
  if (sched) {
    const MTile t = sched[mi];
    expert = t.expert;
    row0 = t.row0;
    rows = t.rows;
  } else {
    row0 = mi * TB;
    if (row0 >= static_rows) return;
    rows = min(TB, static_rows - row0);
  }
  const int n0 = ni * TB;
  __shared__ float sA[TB][TK + 1], sB0[TB][TK + 1], sB1[DUAL ? TB : 1][TK + 1];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;  // outputs (ty*2+i, tx*2+j)
  const float* B0b = B0 + (size_t)expert * strideB;
  const float* B1b = DUAL ? B1 + (size_t)expert * strideB : nullptr;
  float c0[2][2] = {{0, 0}, {0, 0}}, c1[2][2] = {{0, 0}, {0, 0}};
  for (int k0 = 0; k0 < K; k0 += TK) {
    for (int i = tid; i < TB * TK; i += 256) {
      const int r = i / TK, k = i % TK;
      const int kk = k0 + k;
      const int ar = min(r, rows - 1);
      const int bn = min(n0 + r, N - 1);
      const size_t arow = a_rows ? (size_t)a_rows[row0 + ar] : (size_t)(row0 + ar);
      sA[r][k] = kk < K ? A[arow * lda + kk] : 0.f;
      sB0[r][k] = kk < K ? B0b[(size_t)bn * K + kk] : 0.f;
      if constexpr (DUAL) sB1[r][k] = kk < K ? B1b[(size_t)bn * K + kk] : 0.f;
    }
    __syncthreads();
    for (int k = 0; k < TK; ++k) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          c0[i][j] = fmaf(sA[ty * 2 + i][k], sB0[tx * 2 + j][k], c0[i][j]);
          if constexpr (DUAL) c1[i][j] = fmaf(sA[ty * 2 + i][k], sB1[tx * 2 + j][k], c1[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = ty * 2 + i;
    if (m >= rows) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + tx * 2 + j;
      if (n >= N) continue;
      float v;
      if (DUAL) v = silu_mul(c0[i][j], c1[i][j]);
      else v = c0[i][j] + (bias ? bias[n] : 0.0f);
      Out[(size_t)(row0 + m) * ldo + n] = v;
    }
  }
}

// SwiGLU over split-K partial sums: h[r][c] = silu(sum_p G_p[r][c]) *
// (sum_p U_p[r][c]) for rows r below *rows_dev (or static_rows), where part
// p of the gate sums is at parts + p * part_elems and part p of the up sums at
// parts + (nparts + p) * part_elems, rows of ld floats.  Parts are added in
// order; h is fp16 as in the fused epilogue (values outside its range set
// MOE_FLAG_H_RANGE).  One block per row and 1024 columns, four per thread.
__global__ __launch_bounds__(256) void k_swiglu_parts(const float* __restrict__ parts, int nparts,
                                                      long long part_elems, int N, int ld,
                                                      const int32_t* __restrict__ rows_dev,
                                                      int static_rows, uint16_t* __restrict__ h,
                                                      int ldh, uint32_t* __restrict__ flags) {
  const int r = blockIdx.x;
  const int rows = rows_dev ? *rows_dev : static_rows;
  if (r >= rows) return;
  const int c = (blockIdx.y * blockDim.x + threadIdx.x) * 4;
  if (c >= N) return;
  const float* g = parts + (size_t)r * ld + c;
  const float* u = g + (size_t)nparts * part_elems;
  f32x4 gs = *reinterpret_cast<const f32x4*>(g);
  f32x4 us = *reinterpret_cast<const f32x4*>(u);
  for (int p = 1; p < nparts; ++p) {
    gs += *reinterpret_cast<const f32x4*>(g + p * part_elems);
    us += *reinterpret_cast<const f32x4*>(u + p * part_elems);
  }
  const float h0 = silu_mul(gs[0], us[0]), h1 = silu_mul(gs[1], us[1]);
  const float h2 = silu_mul(gs[2], us[2]), h3 = silu_mul(gs[3], us[3]);
  const bool ovf = !(fabsf(h0) <= 65504.f && fabsf(h1) <= 65504.f && fabsf(h2) <= 65504.f &&
                     fabsf(h3) <= 65504.f);
  *reinterpret_cast<uint2*>(h + (size_t)r * ldh + c) =
      uint2{f32_to_f16_bits(h0) | (f32_to_f16_bits(h1) << 16), f32_to_f16_bits(h2) | (f32_to_f16_bits(h3) << 16)};
  if (ovf && flags) atomicOr(flags, (uint32_t)MOE_FLAG_H_RANGE);
}

// The MXFP8 form: h re-quantised per 32-column block as in the fused
// epilogue (block maximum -> E8M0 scale, E4M3 codes), codes [rows][N] and
// scale bytes at ((c / 128) * hs_stride + r) * 4 + (c / 32) % 4.  Thread t of
// a block owns columns 4t .. 4t+3, so a 32-column block is 8 consecutive
// lanes and its maximum takes three shuffles.
__global__ __launch_bounds__(256) void k_swiglu_parts_mx(const float* __restrict__ parts, int nparts,
                                                         long long part_elems, int N,
                                                         const int32_t* __restrict__ rows_dev,
                                                         int static_rows, uint8_t* __restrict__ h,
                                                         uint8_t* __restrict__ hsc, int hs_stride,
                                                         uint32_t* __restrict__ flags) {
  const int r = blockIdx.x;
  const int rows = rows_dev ? *rows_dev : static_rows;
  if (r >= rows) return;  // uniform over the block
  const int c = (blockIdx.y * blockDim.x + threadIdx.x) * 4;
  const bool live = c < N;  // N is a multiple of 128: whole 8-lane groups are live or not
  f32x4 gs = {0.f, 0.f, 0.f, 0.f}, us = {0.f, 0.f, 0.f, 0.f};
  if (live) {
    const float* g = parts + (size_t)r * N + c;
    const float* u = g + (size_t)nparts * part_elems;
    gs = *reinterpret_cast<const f32x4*>(g);
    us = *reinterpret_cast<const f32x4*>(u);
    for (int p = 1; p < nparts; ++p) {
      gs += *reinterpret_cast<const f32x4*>(g + p * part_elems);
      us += *reinterpret_cast<const f32x4*>(u + p * part_elems);
    }
  }
  float hv[4];
  float amax = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    hv[q] = silu_mul(gs[q], us[q]);
    amax = fmaxf(amax, fabsf(hv[q]));
  }
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if (!live) return;
  const uint32_t sb = mx_scale_byte(amax);
  const int sh = 127 - (int)sb;
  *reinterpret_cast<uint32_t*>(h + (size_t)r * N + c) =
      e4m3x4(ldexpf(hv[0], sh), ldexpf(hv[1], sh), ldexpf(hv[2], sh), ldexpf(hv[3], sh));
  if ((threadIdx.x & 7) == 0) {
    hsc[((size_t)(c >> 7) * hs_stride + r) * 4 + ((c >> 5) & 3)] = (uint8_t)sb;
    if (!(amax <= 3.402823466e38f) && flags) atomicOr(flags, (uint32_t)MOE_FLAG_H_RANGE);
  }
}

// Worst-case grid: every row-tile slot real; a multiple of 8 (one slot per XCD).
inline int grid_for(int mslots, int ntiles) {
  const long long g = (long long)mslots * ntiles;
  return (int)((g + 7) / 8 * 8);
}

// Launches k_gemm_mfma<BM, BNB, MODE>, raising the block's LDS limit when the
// two stages exceed the default 64 KiB.
template <int BM, int BNB, int MODE, int NS, int NW>
hipError_t launch_mfma(const void* A, const int32_t* a_rows, int lda, const void* B0,
                       const void* B1, int N, int K,
                       void* out, int ldo, const float* bias, const MTile* sched,
                       const int32_t* count, int mslots, int static_rows, uint32_t* flags,
                       hipStream_t st, const MxArgs mx = MxArgs{}, int ksplit = 1,
                       long long part_elems = 0, bool out_half = false, int group_m = kGroupM) {
  constexpr int lds = gemm_lds_bytes(BM, BNB, MODE, NS, NW);
  static_assert(lds <= 160 * 1024, "LDS");
  if constexpr (lds > 65536) {
    // raise the kernel's LDS limit once per device (setting it again is harmless,
    // so concurrent first calls may both set it)
    static std::atomic<uint64_t> set_on{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = 1ull << (dev & 63);
    if (!(set_on.load(std::memory_order_acquire) & bit)) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_mfma<BM, BNB, MODE, NS, NW>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      if (e != hipSuccess) return e;
      set_on.fetch_or(bit, std::memory_order_release);
    }
  }
  const int ntiles = (N + BNB - 1) / BNB;
  const dim3 grid(grid_for(mslots, ntiles * ksplit));
  hipLaunchKernelGGL((k_gemm_mfma<BM, BNB, MODE, NS, NW>), grid, dim3(64 * NW), lds, st,
                     static_cast<const uint16_t*>(A), a_rows, lda,
                     static_cast<const uint16_t*>(B0), static_cast<const uint16_t*>(B1),
                     (long long)N * K, N, K, out, ldo, bias,
                     sched, count, mslots, ntiles, static_rows, flags, mx, ksplit, part_elems, out_half ? 1 : 0,
                     group_m);
  return hipGetLastError();
}

// Raises a kernel's dynamic LDS limit once per device when it exceeds the
// default 64 KiB (setting it again is harmless, so concurrent first calls may
// both set it).
template <const void* (*KERNEL)()>
hipError_t raise_lds_limit(int lds, std::atomic<uint64_t>& set_on) {
  if (lds <= 65536) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (set_on.load(std::memory_order_acquire) & bit) return hipSuccess;
  e = hipFuncSetAttribute(KERNEL(), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  set_on.fetch_or(bit, std::memory_order_release);
  return hipSuccess;
}

template <int BM1, int BNB1, int BM2, int BNB2, int MODE>
const void* mfma2_kernel() {
  return reinterpret_cast<const void*>(&k_gemm_mfma2<BM1, BNB1, BM2, BNB2, MODE>);
}

// Launches k_gemm_mfma2: the big-tile class (schedule s1, count c1, at most
// ms1 row tiles) and the small-tile class (s2, c2, ms2) in one grid.
template <int BM1, int BNB1, int BM2, int BNB2, int MODE>
hipError_t launch_mfma2(const void* A, const int32_t* a_rows, int lda, const void* B0, const void* B1,
                        int N, int K, void* out, int ldo, uint32_t* flags, const MTile* s1,
                        const int32_t* c1, int ms1, const MTile* s2, const int32_t* c2, int ms2,
                        hipStream_t st, const MxArgs mx = MxArgs{}, int ksplit = 1,
                        long long part_elems = 0, bool out_half = false, int group_m = kGroupM) {
  constexpr int l1 = gemm_lds_bytes(BM1, BNB1, MODE, 2, 8), l2 = gemm_lds_bytes(BM2, BNB2, MODE, 2, 8);
  constexpr int l3 = gemm_lds_bytes(32, BNB2, MODE, 2, 8);  // small tiles of at most 32 rows
  constexpr int lds = (l1 > l2 ? l1 : l2) > l3 ? (l1 > l2 ? l1 : l2) : l3;
  static_assert(lds <= 160 * 1024, "LDS");
  static std::atomic<uint64_t> set_on{0};
  hipError_t e = raise_lds_limit<mfma2_kernel<BM1, BNB1, BM2, BNB2, MODE>>(lds, set_on);
  if (e != hipSuccess) return e;
  const int nt1 = (N + BNB1 - 1) / BNB1, nt2 = (N + BNB2 - 1) / BNB2;
  const dim3 grid(grid_for(ms1, nt1 * ksplit) + grid_for(ms2, nt2 * ksplit));
  if (grid.x == 0) return hipSuccess;
  hipLaunchKernelGGL((k_gemm_mfma2<BM1, BNB1, BM2, BNB2, MODE>), grid, dim3(512), lds, st,
                     static_cast<const uint16_t*>(A), a_rows, lda, static_cast<const uint16_t*>(B0),
                     static_cast<const uint16_t*>(B1), (long long)N * K, N, K, out, ldo, flags, mx, s1, c1,
                     ms1, nt1, s2, c2, ms2, nt2, ksplit, part_elems, out_half ? 1 : 0, group_m);
  return hipGetLastError();
}

}  // namespace

int gemm_tile_rows(int dtype, int bm_hint) {
  if (dtype == MOE_F32) return 32;
  return bm_hint >= 256 ? 256 : (bm_hint >= 128 ? 128 : 32);
}

hipError_t launch_gemm_gateup(int dtype, int bm, const void* A, const int32_t* a_rows, int lda,
                              const void* Bg, const void* Bu, int N, int K, void* h, int ldh,
                              const MTile* sched,
                              const int32_t* count, int max_tiles, int static_rows,
                              uint32_t* flags, hipStream_t st) {
  const long long strideB = (long long)N * K;
  if (dtype == MOE_F32) {
    const int mslots = sched ? max_tiles : (static_rows + 31) / 32;
    const int ntiles = (N + 31) / 32;
    if (mslots == 0) return hipSuccess;
    hipLaunchKernelGGL(k_gemm_f32<true>, dim3(grid_for(mslots, ntiles)), dim3(256), 0, st,
                       static_cast<const float*>(A), a_rows, lda, static_cast<const float*>(Bg),
                       static_cast<const float*>(Bu), strideB, N, K, static_cast<float*>(h), ldh,
                       nullptr, sched, count, mslots, ntiles, static_rows);
    return hipGetLastError();
  }
  const int mslots = sched ? max_tiles : (static_rows + bm - 1) / bm;
  if (mslots == 0) return hipSuccess;
  if (bm == 256)
    return launch_mfma<256, 128, kGateUp, 2, 8>(A, a_rows, lda, Bg, Bu, N, K, h, ldh, nullptr, sched, count,
                                          mslots, static_rows, flags, st);
  if (bm == 128)
    return launch_mfma<128, 128, kGateUp, 2, 8>(A, a_rows, lda, Bg, Bu, N, K, h, ldh, nullptr, sched, count,
                                          mslots, static_rows, flags, st);
  // 32-row tiles (small experts, decode): 8-wave blocks of 32 x 256, which
  // stream the weights faster than 4-wave 32 x 128 blocks (measured 0.29 vs
  // 0.35 ms on the Mixtral-shaped decode layer)
  if (bm != 32) return hipErrorInvalidValue;
  return launch_mfma<32, 256, kGateUp, 2, 8>(A, a_rows, lda, Bg, Bu, N, K, h, ldh, nullptr, sched, count,
                                             mslots, static_rows, flags, st);
}

hipError_t launch_gemm_gateup_parts(const void* A, const int32_t* a_rows, int lda, const void* Bg,
                                    const void* Bu, int N, int K, float* parts, const MTile* sched,
                                    const int32_t* count, int max_tiles, int static_rows, int ksplit,
                                    long long part_elems, hipStream_t st) {
  const int mslots = sched ? max_tiles : (static_rows + 31) / 32;
  if (mslots == 0) return hipSuccess;
  return launch_mfma<32, 256, kGateUpPart, 2, 8>(A, a_rows, lda, Bg, Bu, N, K, parts, N, nullptr, sched, count,
                                                 mslots, static_rows, nullptr, st, MxArgs{}, ksplit, part_elems);
}

hipError_t launch_swiglu_parts(const float* parts, int nparts, long long part_elems, int N,
                               const int32_t* rows_dev, int static_rows, int max_rows, void* h, int ldh,
                               uint32_t* flags, hipStream_t st) {
  if (max_rows <= 0) return hipSuccess;
  if (N % 4) return hipErrorInvalidValue;
  const dim3 grid(max_rows, (N + 1023) / 1024);
  hipLaunchKernelGGL(k_swiglu_parts, grid, dim3(256), 0, st, parts, nparts, part_elems, N, N, rows_dev,
                     static_rows, static_cast<uint16_t*>(h), ldh, flags);
  return hipGetLastError();
}

namespace {
// The down projection on fp16 weights: the tile configurations of kDown.
hipError_t launch_down_w16(int bm, const void* A, int lda, const void* B, int N, int K, void* Y, int ldy,
                           const MTile* sched, const int32_t* count, int mslots, int static_rows, hipStream_t st,
                           int ksplit, long long part_elems, bool y_half, uint32_t* flags) {
  if (bm == 256)
    return launch_mfma<256, 256, kDownW16, 2, 8>(A, nullptr, lda, B, nullptr, N, K, Y, ldy, nullptr, sched, count,
                                                 mslots, static_rows, flags, st, MxArgs{}, ksplit, part_elems,
                                                 y_half);
  if (bm == 128)
    return launch_mfma<128, 128, kDownW16, 2, 8>(A, nullptr, lda, B, nullptr, N, K, Y, ldy, nullptr, sched, count,
                                                 mslots, static_rows, flags, st, MxArgs{}, ksplit, part_elems,
                                                 y_half);
  if (bm != 32) return hipErrorInvalidValue;
  if (K >= kDown8MinK)
    return launch_mfma<32, 256, kDownW16, 2, 8>(A, nullptr, lda, B, nullptr, N, K, Y, ldy, nullptr, sched, count,
                                                mslots, static_rows, flags, st, MxArgs{}, ksplit, part_elems,
                                                y_half);
  if ((long long)mslots * ((N + 127) / 128) <= 1024)
    return launch_mfma<32, 128, kDownW16, 6, 4>(A, nullptr, lda, B, nullptr, N, K, Y, ldy, nullptr, sched, count,
                                                mslots, static_rows, flags, st, MxArgs{}, ksplit, part_elems,
                                                y_half);
  return launch_mfma<32, 128, kDownW16, 4, 4>(A, nullptr, lda, B, nullptr, N, K, Y, ldy, nullptr, sched, count,
                                              mslots, static_rows, flags, st, MxArgs{}, ksplit, part_elems, y_half);
}

// bf16 -> fp16 of n elements, with the conversion kDown applies to its
// weights while staging them (so a layer on converted weights computes the
// same products); eight elements per thread, the tail one by one.
__global__ __launch_bounds__(256) void k_bf16_to_f16(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                     long long n) {
  const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i + 8 <= n) {
    *reinterpret_cast<u32x4*>(dst + i) = bf16x8_to_f16x8(*reinterpret_cast<const u32x4*>(src + i));
  } else {
    for (long long j = i; j < n; ++j) {
      const uint32_t w = bf16x2_to_f16x2((uint32_t)src[j]);
      dst[j] = (uint16_t)(w & 0xFFFFu);
    }
  }
}
}  // namespace

hipError_t launch_bf16_to_f16(const void* src, void* dst, long long n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const long long blocks = (n + 2047) / 2048;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_bf16_to_f16, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<const uint16_t*>(src),
                     static_cast<uint16_t*>(dst), n);
  return hipGetLastError();
}

hipError_t launch_gemm_plain(int dtype, int bm, bool a_is_h, const void* A, int lda,
                             const void* B, int N, int K, const float* bias, void* Y, int ldy,
                             const MTile* sched, const int32_t* count, int max_tiles,
                             int static_rows, hipStream_t st, int ksplit, long long part_elems,
                             bool y_half, uint32_t* flags, bool w16) {
  const long long strideB = (long long)N * K;
  if (y_half && (dtype != MOE_BF16 || !a_is_h || ksplit != 1 || bias)) return hipErrorInvalidValue;
  if (w16 && (dtype != MOE_BF16 || !a_is_h)) return hipErrorInvalidValue;
  if (dtype == MOE_F32) {
    if (ksplit > 1) return hipErrorInvalidValue;  // the fp32 kernel does not split K
    const int mslots = sched ? max_tiles : (static_rows + 31) / 32;
    const int ntiles = (N + 31) / 32;
    if (mslots == 0) return hipSuccess;
    hipLaunchKernelGGL(k_gemm_f32<false>, dim3(grid_for(mslots, ntiles)), dim3(256), 0, st,
                       static_cast<const float*>(A), nullptr, lda, static_cast<const float*>(B), nullptr,
                       strideB, N, K, static_cast<float*>(Y), ldy, bias, sched, count, mslots, ntiles,
                       static_rows);
    return hipGetLastError();
  }
  const int mslots = sched ? max_tiles : (static_rows + bm - 1) / bm;
  if (mslots == 0) return hipSuccess;
  if (a_is_h && w16)
    return launch_down_w16(bm, A, lda, B, N, K, Y, ldy, sched, count, mslots, static_rows, st, ksplit, part_elems,
                           y_half, flags);
  if (a_is_h) {
    if (bm == 256)
      return launch_mfma<256, 256, kDown, 2, 8>(A, nullptr, lda, B, nullptr, N, K, Y, ldy, nullptr, sched, count,
                                          mslots, static_rows, flags, st, MxArgs{}, ksplit, part_elems, y_half);
    if (bm == 128)
      return launch_mfma<128, 128, kDown, 2, 8>(A, nullptr, lda, B, nullptr, N, K, Y, ldy, nullptr, sched, count,
                                          mslots, static_rows, flags, st, MxArgs{}, ksplit, part_elems, y_half);
    if (bm != 32) return hipErrorInvalidValue;
    // K of at least 2048: 8-wave 32 x 256 blocks, as for gate/up (Mixtral-
    // shaped decode down 0.181 -> 0.139 ms); shorter K keeps the 4-wave
    // 32 x 128 blocks (I = 768: 0.025 against 0.030 ms)
    if (K >= kDown8MinK)
      return launch_mfma<32, 256, kDown, 2, 8>(A, nullptr, lda, B, nullptr, N, K, Y, ldy, nullptr, sched,
                                               count, mslots, static_rows, flags, st, MxArgs{}, ksplit,
                                               part_elems, y_half);
    // few blocks (decode-sized layers): a deeper ring keeps more weight bytes
    // in flight per compute unit
    if ((long long)mslots * ((N + 127) / 128) <= 1024)
      return launch_mfma<32, 128, kDown, 6, 4>(A, nullptr, lda, B, nullptr, N, K, Y, ldy, nullptr, sched,
                                               count, mslots, static_rows, flags, st, MxArgs{}, ksplit,
                                               part_elems, y_half);
    return launch_mfma<32, 128, kDown, 4, 4>(A, nullptr, lda, B, nullptr, N, K, Y, ldy, nullptr, sched, count,
                                       mslots, static_rows, flags, st, MxArgs{}, ksplit, part_elems, y_half);
  }
  if (bm == 128)
    return launch_mfma<128, 128, kPlain, 2, 8>(A, nullptr, lda, B, nullptr, N, K, Y, ldy, bias, sched, count,
                                         mslots, static_rows, nullptr, st, MxArgs{}, ksplit, part_elems);
  if (bm != 32) return hipErrorInvalidValue;
  return launch_mfma<32, 128, kPlain, 4, 4>(A, nullptr, lda, B, nullptr, N, K, Y, ldy, bias, sched, count,
                                      mslots, static_rows, nullptr, st, MxArgs{}, ksplit, part_elems);
}

// MXFP8 gate/up + SwiGLU: A = E4M3 token rows (K = H codes each, gathered
// through a_rows when given; scales sa, stride sa_stride), Bg/Bu = E4M3 weights
// [E][N][K] (scales stride sb_stride = E * N); h = MXFP8 codes [rows][N] with
// scales hsc (stride hs_stride).  bm: 256, 128 or 32 (the 32-row tiles span
// 256 weight rows so that eight wavefronts still split the columns).
hipError_t launch_gemm_gateup_mx(int bm, const void* A, const int32_t* a_rows, const uint8_t* sa,
                                 int sa_stride, const void* Bg, const uint8_t* sbg, const void* Bu,
                                 const uint8_t* sbu, int sb_stride, int N, int K, void* h,
                                 uint8_t* hsc, int hs_stride, const MTile* sched,
                                 const int32_t* count, int max_tiles, int static_rows,
                                 uint32_t* flags, hipStream_t st, bool sa_direct) {
  const int mslots = sched ? max_tiles : (static_rows + bm - 1) / bm;
  if (mslots == 0) return hipSuccess;
  const MxArgs mx{sa, sbg, sbu, hsc, sa_stride, sb_stride, hs_stride, sa_direct ? 1 : 0};
  const int K2 = K / 2;  // 16-bit units
  if (bm == 256)
    return launch_mfma<256, 128, kGateUpMX, 2, 8>(A, a_rows, K2, Bg, Bu, N, K2, h, N, nullptr, sched,
                                                  count, mslots, static_rows, flags, st, mx);
  if (bm == 128)
    return launch_mfma<128, 128, kGateUpMX, 2, 8>(A, a_rows, K2, Bg, Bu, N, K2, h, N, nullptr, sched,
                                                  count, mslots, static_rows, flags, st, mx);
  if (bm != 32) return hipErrorInvalidValue;
  return launch_mfma<32, 256, kGateUpMX, 2, 8>(A, a_rows, K2, Bg, Bu, N, K2, h, N, nullptr, sched,
                                               count, mslots, static_rows, flags, st, mx);
}

hipError_t launch_gemm_gateup_mx_parts(const void* A, const int32_t* a_rows, const uint8_t* sa,
                                       int sa_stride, const void* Bg, const uint8_t* sbg, const void* Bu,
                                       const uint8_t* sbu, int sb_stride, int N, int K, float* parts,
                                       const MTile* sched, const int32_t* count, int max_tiles,
                                       int static_rows, int ksplit, long long part_elems, hipStream_t st,
                                       bool sa_direct) {
  const int mslots = sched ? max_tiles : (static_rows + 31) / 32;
  if (mslots == 0) return hipSuccess;
  const MxArgs mx{sa, sbg, sbu, nullptr, sa_stride, sb_stride, 0, sa_direct ? 1 : 0};
  const int K2 = K / 2;  // 16-bit units
  return launch_mfma<32, 256, kGateUpMXPart, 2, 8>(A, a_rows, K2, Bg, Bu, N, K2, parts, N, nullptr, sched,
                                                   count, mslots, static_rows, nullptr, st, mx, ksplit,
                                                   part_elems);
}

hipError_t launch_swiglu_parts_mx(const float* parts, int nparts, long long part_elems, int N,
                                  const int32_t* rows_dev, int static_rows, int max_rows, void* h,
                                  uint8_t* hsc, int hs_stride, uint32_t* flags, hipStream_t st) {
  if (max_rows <= 0) return hipSuccess;
  if (N % 128) return hipErrorInvalidValue;
  const dim3 grid(max_rows, (N + 1023) / 1024);
  hipLaunchKernelGGL(k_swiglu_parts_mx, grid, dim3(256), 0, st, parts, nparts, part_elems, N, rows_dev,
                     static_rows, static_cast<uint8_t*>(h), hsc, hs_stride, flags);
  return hipGetLastError();
}

// MXFP8 down projection: A = MXFP8 h rows [rows][K] (scales hsc, stride
// hs_stride), B = E4M3 weights [E][N][K] (scales sb, stride sb_stride = E * N);
// Y fp32 [rows][ldy].
hipError_t launch_gemm_down_mx(int bm, const void* A, const uint8_t* hsc, int hs_stride,
                               const void* B, const uint8_t* sb, int sb_stride, int N, int K,
                               void* Y, int ldy, const MTile* sched, const int32_t* count,
                               int max_tiles, int static_rows, hipStream_t st, int ksplit,
                               long long part_elems, bool y_half, uint32_t* flags) {
  const int mslots = sched ? max_tiles : (static_rows + bm - 1) / bm;
  if (mslots == 0) return hipSuccess;
  if (y_half && ksplit != 1) return hipErrorInvalidValue;
  const MxArgs mx{hsc, sb, nullptr, nullptr, hs_stride, sb_stride, 0};
  const int K2 = K / 2;
  if (bm == 256)
    return launch_mfma<256, 256, kDownMX, 2, 8>(A, nullptr, K2, B, nullptr, N, K2, Y, ldy, nullptr,
                                                sched, count, mslots, static_rows, flags, st, mx, 1, 0, y_half);
  if (bm == 128)
    return launch_mfma<128, 128, kDownMX, 2, 8>(A, nullptr, K2, B, nullptr, N, K2, Y, ldy, nullptr,
                                                sched, count, mslots, static_rows, flags, st, mx, 1, 0, y_half);
  if (bm != 32) return hipErrorInvalidValue;
  return launch_mfma<32, 256, kDownMX, 2, 8>(A, nullptr, K2, B, nullptr, N, K2, Y, ldy, nullptr,
                                             sched, count, mslots, static_rows, flags, st, mx, ksplit,
                                             part_elems, y_half);
}

// Both row-tile classes of a layer in one launch (big: 256-row tiles,
// small: 32-row tiles, both 8-wave blocks); bf16 layers.
hipError_t launch_gemm_gateup2(const void* A, const int32_t* a_rows, int lda, const void* Bg,
                               const void* Bu, int N, int K, void* h, int ldh, const MTile* sb,
                               const int32_t* cb, int mb, const MTile* ss, const int32_t* cs, int ms,
                               uint32_t* flags, hipStream_t st) {
  return launch_mfma2<256, 128, kMergedSmallRows, 256, kGateUp>(A, a_rows, lda, Bg, Bu, N, K, h, ldh, flags, sb, cb, mb,
                                                  ss, cs, ms, st);
}

hipError_t launch_gemm_down2(const void* A, int lda, const void* B, int N, int K, void* Y, int ldy,
                             const MTile* sb, const int32_t* cb, int mb, const MTile* ss,
                             const int32_t* cs, int ms, hipStream_t st, int ksplit,
                             long long part_elems, bool y_half, uint32_t* flags, bool w16) {
  if (y_half && ksplit != 1) return hipErrorInvalidValue;
  if (w16)
    return launch_mfma2<256, 256, kMergedSmallRows, 256, kDownW16>(A, nullptr, lda, B, nullptr, N, K, Y, ldy, flags,
                                                                   sb, cb, mb, ss, cs, ms, st, MxArgs{}, ksplit,
                                                                   part_elems, y_half);
  return launch_mfma2<256, 256, kMergedSmallRows, 256, kDown>(A, nullptr, lda, B, nullptr, N, K, Y, ldy, flags, sb, cb,
                                                mb, ss, cs, ms, st, MxArgs{}, ksplit, part_elems, y_half);
}

hipError_t launch_gemm_gateup_mx2(const void* A, const int32_t* a_rows, const uint8_t* sa, int sa_stride,
                                  const void* Bg, const uint8_t* sbg, const void* Bu, const uint8_t* sbu,
                                  int sb_stride, int N, int K, void* h, uint8_t* hsc, int hs_stride,
                                  const MTile* sb, const int32_t* cb, int mb, const MTile* ss,
                                  const int32_t* cs, int ms, uint32_t* flags, hipStream_t st,
                                  bool sa_direct) {
  const MxArgs mx{sa, sbg, sbu, hsc, sa_stride, sb_stride, hs_stride, sa_direct ? 1 : 0};
  return launch_mfma2<256, 128, kMergedSmallRows, 256, kGateUpMX>(A, a_rows, K / 2, Bg, Bu, N, K / 2, h, N, flags, sb, cb,
                                                    mb, ss, cs, ms, st, mx);
}

hipError_t launch_gemm_down_mx2(const void* A, const uint8_t* hsc, int hs_stride, const void* B,
                                const uint8_t* sb_w, int sb_stride, int N, int K, void* Y, int ldy,
                                const MTile* sb, const int32_t* cb, int mb, const MTile* ss,
                                const int32_t* cs, int ms, hipStream_t st, int ksplit,
                                long long part_elems, bool y_half, uint32_t* flags) {
  if (y_half && ksplit != 1) return hipErrorInvalidValue;
  const MxArgs mx{hsc, sb_w, nullptr, nullptr, hs_stride, sb_stride, 0};
  return launch_mfma2<256, 256, kMergedSmallRows, 256, kDownMX>(A, nullptr, K / 2, B, nullptr, N, K / 2, Y, ldy, flags, sb,
                                                  cb, mb, ss, cs, ms, st, mx, ksplit, part_elems, y_half);
}

}  // namespace moe
