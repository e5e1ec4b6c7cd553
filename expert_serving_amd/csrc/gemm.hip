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
// bf16 kernel (gfx950):
//   * v_mfma_f32_16x16x32_bf16, fp32 accumulation;
//   * the weight tile is the MFMA A operand and the token tile the B
//     operand, so each lane's 4 accumulators are 4 consecutive output
//     columns of one token row (8-byte bf16 / 16-byte fp32 stores);
//   * block = 4 wavefronts in a 2x2 grid; K step 64; LDS tiles [rows][64] with
//     16-byte chunks XOR-swizzled by row; the next K step is prefetched into
//     registers while the current one is multiplied;
//   * gate/up variant: one block computes the same column range of X.Wg^T
//     and X.Wu^T and applies SwiGLU in the epilogue (h never exists unfused);
//   * block -> tile map: blocks are dealt round-robin to the 8 XCDs, so block
//     b is remapped to give each XCD a contiguous range of logical tiles, and
//     logical tiles sweep groups of kGroupM row tiles across all column tiles
//     so the XCD's L2 serves both the token rows and the weight rows.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBK = 64;
constexpr int kGroupM = 8;
constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b + (((b >> 16) & 1u) + 0x7FFFu)) >> 16;
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

// Logical tile of this block.  Returns false when the block has no tile.
__device__ __forceinline__ bool block_tile(int mslots, int ntiles, int& m, int& n) {
  const int b = blockIdx.x;
  const int per_xcd = gridDim.x >> 3;  // gridDim.x is a multiple of 8
  const int L = (b & 7) * per_xcd + (b >> 3);
  const int per_group = kGroupM * ntiles;
  const int g = L / per_group;
  const int r = L - g * per_group;
  n = r / kGroupM;
  m = g * kGroupM + (r - n * kGroupM);
  return m < mslots && n < ntiles;
}

// Kernel modes.
//   kGateUp: A = bf16 token rows, B0/B1 = bf16 gate/up weights;
//            out h (fp16) = silu(A.B0^T) * (A.B1^T)
//   kDown:   A = fp16 h rows, B0 = bf16 down weights converted to fp16 while
//            staged into LDS (exact for |w| in fp16's normal range);
//            out y (fp32) = A.B0^T
//   kPlain:  A = bf16 rows, B0 = bf16 weights; out fp32 = A.B0^T + bias
enum GemmMode { kGateUp = 0, kDown = 1, kPlain = 2 };

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
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (MODE == kDown)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int BM, int BN, int MODE>
__global__ __launch_bounds__(kThreads, 2) void k_gemm_mfma(
    const uint16_t* __restrict__ A, int lda, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, long long strideB, int N, int K, void* __restrict__ Out,
    int ldo, const float* __restrict__ bias, const MTile* __restrict__ sched,
    const int32_t* __restrict__ count, int mslots, int ntiles, int static_rows,
    uint32_t* __restrict__ flags) {
  constexpr bool DUAL = MODE == kGateUp;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int A_LD = BM * 8 / kThreads;  // 16-byte chunks per thread
  constexpr int B_LD = BN * 8 / kThreads;
  static_assert(FM >= 1 && FN >= 1 && A_LD >= 1 && B_LD >= 1, "tile too small");

  int mi, ni;
  if (!block_tile(mslots, ntiles, mi, ni)) return;
  int expert = 0, row0, rows;
  if (sched) {
    if (mi >= *count) return;
    const MTile t = sched[mi];
    expert = t.expert;
    row0 = t.row0;
    rows = t.rows;
  } else {
    row0 = mi * BM;
    if (row0 >= static_rows) return;
    rows = min(BM, static_rows - row0);
  }
  const int n0 = ni * BN;

  __shared__ __attribute__((aligned(16))) uint16_t sA[BM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t sB0[BN * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t sB1[DUAL ? BN * kBK : 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int lc = tid & 7;   // 16-byte chunk of a 64-wide K row
  const int lr = tid >> 3;  // first row this thread loads

  const uint16_t* Ab = A + (size_t)row0 * lda;
  const uint16_t* B0b = B0 + (size_t)expert * strideB;
  const uint16_t* B1b = DUAL ? B1 + (size_t)expert * strideB : nullptr;

  // per-thread global source offsets (rows clamped into range), in elements
  int oa[A_LD], ob[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) oa[i] = min(lr + 32 * i, rows - 1) * lda + lc * 8;
#pragma unroll
  for (int i = 0; i < B_LD; ++i) ob[i] = min(n0 + lr + 32 * i, N - 1) * K + lc * 8;

  u32x4 ra[A_LD], rb0[B_LD], rb1[DUAL ? B_LD : 1];
#define MOE_GLOAD(k0)                                                                  \
  do {                                                                                 \
    _Pragma("unroll") for (int i = 0; i < A_LD; ++i)                                   \
        ra[i] = *reinterpret_cast<const u32x4*>(Ab + oa[i] + (k0));                    \
    _Pragma("unroll") for (int i = 0; i < B_LD; ++i)                                   \
        rb0[i] = *reinterpret_cast<const u32x4*>(B0b + ob[i] + (k0));                  \
    if constexpr (DUAL) {                                                              \
      _Pragma("unroll") for (int i = 0; i < B_LD; ++i)                                 \
          rb1[i] = *reinterpret_cast<const u32x4*>(B1b + ob[i] + (k0));                \
    }                                                                                  \
  } while (0)

  f32x4 acc0[FN][FM];
  f32x4 acc1[DUAL ? FN : 1][DUAL ? FM : 1];
#pragma unroll
  for (int a = 0; a < FN; ++a)
#pragma unroll
    for (int b = 0; b < FM; ++b) {
      acc0[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (DUAL) acc1[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  const int fr = lane & 15;   // row of a 16-row fragment this lane feeds
  const int fk = lane >> 4;   // which 8-element K chunk (of 4) this lane feeds

  MOE_GLOAD(0);
  for (int k0 = 0; k0 < K; k0 += kBK) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int r = lr + 32 * i;
      *reinterpret_cast<u32x4*>(sA + r * kBK + ((lc ^ (r & 7)) << 3)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int r = lr + 32 * i;
      const u32x4 v = MODE == kDown ? bf16x8_to_f16x8(rb0[i]) : rb0[i];
      *reinterpret_cast<u32x4*>(sB0 + r * kBK + ((lc ^ (r & 7)) << 3)) = v;
      if constexpr (DUAL) *reinterpret_cast<u32x4*>(sB1 + r * kBK + ((lc ^ (r & 7)) << 3)) = rb1[i];
    }
    __syncthreads();
    if (k0 + kBK < K) MOE_GLOAD(k0 + kBK);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = kk * 4 + fk;
      u32x4 xa[FM], wb0[FN], wb1[DUAL ? FN : 1];
#pragma unroll
      for (int b = 0; b < FM; ++b) {
        const int r = wm * WM + b * 16 + fr;
        xa[b] = *reinterpret_cast<const u32x4*>(sA + r * kBK + ((c ^ (r & 7)) << 3));
      }
#pragma unroll
      for (int a = 0; a < FN; ++a) {
        const int r = wn * WN + a * 16 + fr;
        wb0[a] = *reinterpret_cast<const u32x4*>(sB0 + r * kBK + ((c ^ (r & 7)) << 3));
        if constexpr (DUAL)
          wb1[a] = *reinterpret_cast<const u32x4*>(sB1 + r * kBK + ((c ^ (r & 7)) << 3));
      }
#pragma unroll
      for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int b = 0; b < FM; ++b) {
          acc0[a][b] = mfma16<MODE>(wb0[a], xa[b], acc0[a][b]);
          if constexpr (DUAL) acc1[a][b] = mfma16<MODE>(wb1[a], xa[b], acc1[a][b]);
        }
    }
    __syncthreads();
  }
#undef MOE_GLOAD

  // epilogue: lane holds output columns n..n+3 of token row m
  bool overflow = false;
#pragma unroll
  for (int a = 0; a < FN; ++a) {
    const int n = n0 + wn * WN + a * 16 + fk * 4;
#pragma unroll
    for (int b = 0; b < FM; ++b) {
      const int m = wm * WM + b * 16 + fr;
      if (m >= rows) continue;
      const size_t o = (size_t)(row0 + m) * ldo + n;
      if constexpr (DUAL) {
        if (n + 3 < N) {
          const f32x4 g = acc0[a][b], u = acc1[a][b];
          const float h0 = silu_mul(g[0], u[0]), h1 = silu_mul(g[1], u[1]);
          const float h2 = silu_mul(g[2], u[2]), h3 = silu_mul(g[3], u[3]);
          overflow |= !(fabsf(h0) <= 65504.f && fabsf(h1) <= 65504.f && fabsf(h2) <= 65504.f &&
                        fabsf(h3) <= 65504.f);
          u32x2 pk;
          pk[0] = f32_to_f16_bits(h0) | (f32_to_f16_bits(h1) << 16);
          pk[1] = f32_to_f16_bits(h2) | (f32_to_f16_bits(h3) << 16);
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(Out) + o) = pk;
        }
      } else {
        f32x4 v = acc0[a][b];
        float* dst = static_cast<float*>(Out) + o;
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
  if constexpr (DUAL) {
    if (overflow && flags) atomicOr(flags, (uint32_t)MOE_FLAG_H_RANGE);
  }
}

// fp32 grouped GEMM: 32x32 output tile (per B matrix), 2x2 outputs per thread,
// K step 16.  Used by fp32 layers, whose sizes make it latency-bound.
template <bool DUAL>
__global__ __launch_bounds__(256) void k_gemm_f32(const float* __restrict__ A, int lda,
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
  if (!block_tile(mslots, ntiles, mi, ni)) return;
  int expert = 0, row0, rows;
  if (sched) {
    if (mi >= *count) return;
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
      sA[r][k] = kk < K ? A[(size_t)(row0 + ar) * lda + kk] : 0.f;
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

inline int grid_for(int mslots, int ntiles) {
  const int groups = (mslots + kGroupM - 1) / kGroupM;
  const int g = groups * kGroupM * ntiles;
  return (g + 7) / 8 * 8;
}

}  // namespace

hipError_t launch_gemm_gateup(int dtype, int bm, const void* A, int lda, const void* Bg,
                              const void* Bu, int N, int K, void* h, int ldh, const MTile* sched,
                              const int32_t* count, int max_tiles, int static_rows,
                              uint32_t* flags, hipStream_t st) {
  const long long strideB = (long long)N * K;
  if (dtype == MOE_F32) {
    const int mslots = sched ? max_tiles : (static_rows + 31) / 32;
    const int ntiles = (N + 31) / 32;
    if (mslots == 0) return hipSuccess;
    hipLaunchKernelGGL(k_gemm_f32<true>, dim3(grid_for(mslots, ntiles)), dim3(256), 0, st,
                       static_cast<const float*>(A), lda, static_cast<const float*>(Bg),
                       static_cast<const float*>(Bu), strideB, N, K, static_cast<float*>(h), ldh,
                       nullptr, sched, count, mslots, ntiles, static_rows);
    return hipGetLastError();
  }
  constexpr int BN = 128;
  const int ntiles = (N + BN - 1) / BN;
  const int mslots = sched ? max_tiles : (static_rows + bm - 1) / bm;
  if (mslots == 0) return hipSuccess;
  const dim3 grid(grid_for(mslots, ntiles));
#define MOE_GU(BM)                                                                               \
  hipLaunchKernelGGL((k_gemm_mfma<BM, BN, kGateUp>), grid, dim3(kThreads), 0, st,               \
                     static_cast<const uint16_t*>(A), lda, static_cast<const uint16_t*>(Bg),     \
                     static_cast<const uint16_t*>(Bu), strideB, N, K, h, ldh, nullptr, sched,    \
                     count, mslots, ntiles, static_rows, flags)
  if (bm == 128) MOE_GU(128);
  else MOE_GU(32);
#undef MOE_GU
  return hipGetLastError();
}

hipError_t launch_gemm_plain(int dtype, int bm, bool a_is_h, const void* A, int lda,
                             const void* B, int N, int K, const float* bias, float* Y, int ldy,
                             const MTile* sched, const int32_t* count, int max_tiles,
                             int static_rows, hipStream_t st) {
  const long long strideB = (long long)N * K;
  if (dtype == MOE_F32) {
    const int mslots = sched ? max_tiles : (static_rows + 31) / 32;
    const int ntiles = (N + 31) / 32;
    if (mslots == 0) return hipSuccess;
    hipLaunchKernelGGL(k_gemm_f32<false>, dim3(grid_for(mslots, ntiles)), dim3(256), 0, st,
                       static_cast<const float*>(A), lda, static_cast<const float*>(B), nullptr,
                       strideB, N, K, Y, ldy, bias, sched, count, mslots, ntiles, static_rows);
    return hipGetLastError();
  }
  constexpr int BN = 128;
  const int ntiles = (N + BN - 1) / BN;
  const int mslots = sched ? max_tiles : (static_rows + bm - 1) / bm;
  if (mslots == 0) return hipSuccess;
  const dim3 grid(grid_for(mslots, ntiles));
#define MOE_PL(BM, MODE)                                                                         \
  hipLaunchKernelGGL((k_gemm_mfma<BM, BN, MODE>), grid, dim3(kThreads), 0, st,                  \
                     static_cast<const uint16_t*>(A), lda, static_cast<const uint16_t*>(B),      \
                     nullptr, strideB, N, K, Y, ldy, bias, sched, count, mslots, ntiles,         \
                     static_rows, nullptr)
  if (a_is_h) {
    if (bm == 128) MOE_PL(128, kDown);
    else MOE_PL(32, kDown);
  } else {
    if (bm == 128) MOE_PL(128, kPlain);
    else MOE_PL(32, kPlain);
  }
#undef MOE_PL
  return hipGetLastError();
}

}  // namespace moe
