// Compression back to rank r, one wavefront per unit, with the core matrices in registers
// (16-bit factors, bf16 or fp16, r <= 32, r + T <= 64).
//
// Method: pages titled "Shallow Encoding Emits Deep Memories" (SEED architecture: every T
// steps the rank r + T factors are truncated back to rank r by a Gram / QR step and a truncated
// SVD of the small core). The factored reduction is the same as in compress.hip:
//   G_U = U~^T U~, G_V = V~^T V~ of the decay-balanced columns; pivoted Cholesky G_U ~ L L^T;
//   core B = L^T G_V L, whose eigenvalues are sigma_i^2 of U~ V~^T; with its r leading
//   eigenvectors Y and eigenvalues lambda, V' = V~ L Y lambda^(-1/4) and U' = M V' lambda^(-1/2)
//   (M = U~ V~^T, so U' V'^T = M times the projector on the kept right singular directions).
//
// Layout on gfx950: one 64-lane wavefront per unit, lane i owning row i of every N x N core
// matrix (N = 64: 64 registers, two 32-wide vectors so that a wave-uniform index reaches a
// register through the indirect-register mode; N = 32 when r + T <= 32: lanes i and i + 32
// both hold row i). MFMA tiles move in and out of that layout with v_permlane32_swap: a
// 32 x 32 accumulator tile keeps one column per lane pair (l, l + 32), and swapping the upper
// half of tile (I, 0) with the lower half of tile (I, 1) leaves every lane with its own column;
// for a symmetric matrix that is its row.
//
//   Grams                 MFMA 32x32x16 bf16 (fp16) straight from the stored columns (fp32
//                         sums);
//   pivoted Cholesky      no row swaps: the L column of step s lands in column p_s of its LDS
//                         copy, so L is held as L P^T (the core below is permuted alike,
//                         which changes neither its eigenvalues nor X_V);
//   B = L^T G_V L         MFMA 32x32x2 fp32, G_V and then L^T G_V from registers, L from LDS;
//   eigenpairs of B       Householder tridiagonalisation in registers (reflectors kept in the
//                         registers they zero), the r largest eigenvalues by Sturm counts
//                         (a 64-point grid shared by all, then trisection), one
//                         eigenvector per eigenvalue from a twisted factorisation (computed on
//                         both lanes of the pair, each keeping the even or the odd entries),
//                         modified Gram-Schmidt, back-transformation by the reflectors;
//   X_V, V', U'           MFMA 32x32x2 fp32 (the rows of a factor tile interleaved, d = NT i +
//                         I, so that each lane loads NT consecutive elements of a column);
//                         W = V_s^T V' by MFMA 32x32x16 bf16 (fp16) on the rounded V' that is
//                         stored,
//                         so that U' = M V' / sigma holds for the stored pair;
//   lazy sink             a = (slot-0 decay) a_0 + U_s f (f_j: column j's sink coefficient
//                         times its decay scale), accumulated on the A operands of the U'
//                         product (no separate pass over the columns).
// Stochastic rounding of the stored factors is a separate instance of the kernel.
// LDS holds L (N x (N + 1) fp32) and a few vectors: about 19.5 KB for N = 64, so eight units
// share a CU (two waves per SIMD), and 6 KB for N = 32 (three waves per SIMD).
#include <float.h>

#include "common.hpp"
#include "kernels.hpp"

namespace seed {

namespace cw {

// N is the padded column count of the core, 64 or 32 (r + T <= 32). With N = 32, lanes c and
// c + 32 hold the same row c, so that the MFMA tiles and the lane-pair phases keep their
// 64-lane form; sums over rows then stop at 32 lanes.
constexpr int RX = 32;          // maximum rank on this path
constexpr int kGrid = 64;       // points of the shared Sturm grid (one per lane)
constexpr int NSEC = 11;        // trisection steps after the 64-point grid (65 * 3^11 ~ 1.15e7)
constexpr float kPivTol = 1e-7f;
constexpr float kReduceFloor = 1e-30f;  // squared column norm below which no reflector is built
// Eigenvalues of the core below kEigFloor times the largest give zero columns. The fp32 core
// resolves no finer: B carries fp32 rounding of about 1e-7 of its norm, and the Sturm search
// stops at about 1e-7 of its Gershgorin range. Below that, the computed eigenvalue can sit far
// above the direction's true Rayleigh quotient, and the computed vector keeps rounding-level
// components along the dominant directions; V' = V L y lambda^(-1/4) then points mostly along
// a dominant direction, and U' = M V' / sigma adds that direction a second time (seen on
// Mamba-2 states whose column decays span 16 orders of magnitude). Dropping them costs at most
// r * kEigFloor of the content's energy.
constexpr float kEigFloor = 1e-6f;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x32 __attribute__((ext_vector_type(32)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// MFMA 32x32x16 over the 16-bit factor format (1 = bf16, 2 = fp16), fp32 accumulation.
template <int FDT> struct Mf16;
template <> struct Mf16<1> {
  using V8 = bf16x8;
  using E = __bf16;
  static __device__ __forceinline__ f32x16 mfma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mf16<2> {
  using V8 = f16x8;
  using E = _Float16;
  static __device__ __forceinline__ f32x16 mfma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// A 64 x 64 matrix held one row per lane: register c of lane i is element (i, c), kept in two
// local 32-wide vectors NAME_lo, NAME_hi. The index is a compile-time constant after unrolling
// or wave-uniform (indirect register access). The matrices stay plain locals touched only
// through these macros, so that they live in registers; helpers pass them by value.
#define MGET(M, c) ((c) < 32 ? M##_lo[(c) & 31] : M##_hi[(c) & 31])
#define MSET(M, c, v)             \
  do {                            \
    if ((c) < 32)                 \
      M##_lo[(c) & 31] = (v);     \
    else                          \
      M##_hi[(c) & 31] = (v);     \
  } while (0)

struct M64 {
  f32x32 lo, hi;
};

__device__ __forceinline__ void swap32(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}

__device__ __forceinline__ float swap16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The value held by lane ^ 32.
__device__ __forceinline__ float partner(float v) {
  float x = v, y = v;
  swap32(x, y);
  return (threadIdx.x & 32) ? x : y;
}

__device__ __forceinline__ float wsum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  v = swap16_sum(v);
  float x = v, y = v;
  swap32(x, y);
  return x + y;
}

// Sum over each 32-lane half (both halves get their own).
__device__ __forceinline__ float hsum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  return swap16_sum(v);
}

// Sum over the rows of an N-wide core: all 64 lanes, or one copy of the 32 rows.
template <int N>
__device__ __forceinline__ float rsum(float v) {
  if constexpr (N == 64) return wsum(v);
  else return hsum(v);
}

__device__ __forceinline__ float wmax(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  float x = v, y = v;
  swap32(x, y);
  return fmaxf(x, y);
}

__device__ __forceinline__ float wmin(float v) { return -wmax(-v); }

// Maximum over the wave of non-negative int keys (the bit patterns of non-negative floats
// order like the floats).
template <int CTRL>
__device__ __forceinline__ int dppi(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ int wmax_key(int v) {
  v = max(v, dppi<0xB1>(v));
  v = max(v, dppi<0x4E>(v));
  v = max(v, dppi<0x141>(v));
  v = max(v, dppi<0x140>(v));
  {
    const auto r = __builtin_amdgcn_permlane16_swap(static_cast<unsigned>(v), static_cast<unsigned>(v), false, false);
    v = max(static_cast<int>(r[0]), static_cast<int>(r[1]));
  }
  const auto r = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(v), static_cast<unsigned>(v), false, false);
  return max(static_cast<int>(r[0]), static_cast<int>(r[1]));
}

// The same value through an identity DPP move, which the compiler cannot see through: loops
// that compare constant indices with a lane-varying index each get their own copy, so that
// their comparison masks are not kept alive from one loop to the next.
__device__ __forceinline__ int opaque(int v) { return __builtin_amdgcn_mov_dpp(v, 0xE4, 0xF, 0xF, false); }

// A value every lane holds (a wave reduction's result), moved to a scalar register so that the
// compiler treats branches on it as uniform.
__device__ __forceinline__ float uni(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

__device__ __forceinline__ float bcast(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// A pivot of a shifted factorisation that is zero or tiny is replaced by -kPivFloor (B is
// scaled to entries <= 1, so the replacement is far below any meaningful pivot).
constexpr float kPivFloor = 1e-30f;
__device__ __forceinline__ float nz(float x) { return fabsf(x) < kPivFloor ? -kPivFloor : x; }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int j = 0; j < 16; ++j) z[j] = 0.f;
  return z;
}

// Accumulator tiles t[I][J] of an N x N product P -> lane L, register rho = P[rho][L] (N = 32:
// P[rho][L % 32] on both lanes of a pair).
template <int N>
__device__ __forceinline__ M64 tiles_to_rows(const f32x16 (&t)[2][2]) {
  f32x32 R_lo, R_hi;
  if constexpr (N == 32) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      float x = t[0][0][j], y = t[0][0][j];
      swap32(x, y);
      const int rho = 8 * (j >> 2) + (j & 3);
      R_lo[rho] = x;
      R_lo[rho + 4] = y;
    }
    return M64{R_lo, R_lo};
  }
#pragma unroll
  for (int I = 0; I < 2; ++I) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      float x = t[I][0][j], y = t[I][1][j];
      swap32(x, y);
      const int rho = 32 * I + 8 * (j >> 2) + (j & 3);
      MSET(R, rho, x);
      MSET(R, rho + 4, y);
    }
  }
  return M64{R_lo, R_hi};
}

// MFMA 32x32x2 operands of K-step s (k = 2s + lane / 32) from a row-per-lane matrix X: .x
// serves row (or column) block 0, .y block 1; as A they give X, as B they give X^T. With
// N = 32 both lanes of a pair hold the same row, so the same swap leaves element k of it in .x
// (selecting it by lane half instead would become a lane-varying register index).
template <int N>
__device__ __forceinline__ float2 rows_operand(const f32x32 X_lo, const f32x32 X_hi, int s) {
  float x = MGET(X, 2 * s), y = MGET(X, 2 * s + 1);
  swap32(x, y);
  return make_float2(x, y);
}

// One 32-row accumulator tile (rows 32 I + 8 q + 4 h + t, column lane % 32) -> MFMA 32x32x2 B
// operands: out[16 I + 4 q + {0, 2, 1, 3}] hold rows 2 s + h of that column.
template <int NO>
__device__ __forceinline__ void tile_to_kops(const f32x16& acc, int I, float (&out)[NO]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float x0 = acc[4 * q + 0], y0 = acc[4 * q + 1];
    swap32(x0, y0);
    float x1 = acc[4 * q + 2], y1 = acc[4 * q + 3];
    swap32(x1, y1);
    out[16 * I + 4 * q + 0] = x0;
    out[16 * I + 4 * q + 2] = y0;
    out[16 * I + 4 * q + 1] = x1;
    out[16 * I + 4 * q + 3] = y1;
  }
}

template <int N>
struct Smem {
  alignas(16) float Lp[N * (N + 1)];  // row stride N + 1 (odd: row and column reads both conflict-free)
  alignas(16) float bvw[2 * N];    // broadcast vectors (v, w); the second vector of a pair
  alignas(16) float y2[2 * N];     // Gram-Schmidt / back-transformation: one vector, even then odd entries
  alignas(16) float dg[N];
  alignas(16) float e[N];
  alignas(16) float e2[N];
  alignas(16) float tau[N];
  alignas(16) float bal[N];
  alignas(16) float ibal[N];
  alignas(16) float colsc[N];
  alignas(16) float cf[N];         // sink fold coefficients, column j at (j % 2) N / 2 + j / 2
  alignas(16) float gam[128];
};

// Gram of the stored columns 0..m-1 (rows of length D, bf16), as row-per-lane registers. With
// ROWSCALE the A operand carries gam^2 along d (KDA's per-channel lazy decay). The column reads
// are issued first, all of them (gram_load; the caller issues both factors' before either
// product), and masked at their use: issued a few at a time beside the MFMAs, each group waited
// for a memory round trip of its own.
template <int D, int N>
struct GramLoads {
  uint4 u0[D / 16], u1[N == 64 ? D / 16 : 1];
};

template <int D, int N>
__device__ __forceinline__ void gram_load(const uint16_t* __restrict__ base, const int m, GramLoads<D, N>& L) {
  const int lane = threadIdx.x;
  const int c0 = lane & 31, kh = lane >> 5;
  const bool ok0 = c0 < m, ok1 = N == 64 && c0 + 32 < m;
  const uint16_t* p0 = base + (ok0 ? c0 : 0) * D + 8 * kh;
  const uint16_t* p1 = base + (ok1 ? c0 + 32 : 0) * D + 8 * kh;
#pragma unroll
  for (int k = 0; k < D / 16; ++k) {
    L.u0[k] = *reinterpret_cast<const uint4*>(p0 + 16 * k);
    if constexpr (N == 64) L.u1[k] = *reinterpret_cast<const uint4*>(p1 + 16 * k);
  }
}

template <int D, bool ROWSCALE, int N, int FDT>
__device__ __forceinline__ M64 gram(const GramLoads<D, N>& L, const int m, const float* __restrict__ gam) {
  using MF = Mf16<FDT>;
  using V8 = typename MF::V8;
  const int lane = threadIdx.x;
  const int c0 = lane & 31, kh = lane >> 5;
  const bool ok0 = c0 < m, ok1 = N == 64 && c0 + 32 < m;
  f32x16 t[2][2] = {{zero16(), zero16()}, {zero16(), zero16()}};
#pragma unroll
  for (int k = 0; k < D / 16; ++k) {
    const int k0 = 16 * k;
    uint4 u0 = L.u0[k];
    uint4 u1 = make_uint4(0u, 0u, 0u, 0u);
    if constexpr (N == 64) u1 = L.u1[k];
    if (!ok0) u0 = make_uint4(0u, 0u, 0u, 0u);
    if (!ok1) u1 = make_uint4(0u, 0u, 0u, 0u);
    const V8 b0 = __builtin_bit_cast(V8, u0);
    const V8 b1 = __builtin_bit_cast(V8, u1);
    V8 a0 = b0, a1 = b1;
    if constexpr (ROWSCALE) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float gj = gam[k0 + 8 * kh + j];
        a0[j] = static_cast<typename MF::E>(static_cast<float>(b0[j]) * gj * gj);
        a1[j] = static_cast<typename MF::E>(static_cast<float>(b1[j]) * gj * gj);
      }
    }
    t[0][0] = MF::mfma(a0, b0, t[0][0]);
    if constexpr (N == 64) {
      t[0][1] = MF::mfma(a0, b1, t[0][1]);
      t[1][0] = MF::mfma(a1, b0, t[1][0]);
      t[1][1] = MF::mfma(a1, b1, t[1][1]);
    }
  }
  return tiles_to_rows<N>(t);
}

// P = X * Lp (X row-per-lane in registers, Lp in LDS) -> P^T row-per-lane.
template <int N>
__device__ __forceinline__ M64 times_L(const f32x32 X_lo, const f32x32 X_hi, const float* __restrict__ Lp) {
  constexpr int LDL = N + 1;
  const int lane = threadIdx.x;
  const int c = lane & 31, kh = lane >> 5;
  f32x16 t[2][2] = {{zero16(), zero16()}, {zero16(), zero16()}};
#pragma unroll
  for (int s = 0; s < N / 2; ++s) {
    const float2 a = rows_operand<N>(X_lo, X_hi, s);
    const float a0 = a.x, a1 = a.y;
    const float b0 = Lp[(2 * s + kh) * LDL + c];
    t[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, t[0][0], 0, 0, 0);
    if constexpr (N == 64) {
      const float b1 = Lp[(2 * s + kh) * LDL + 32 + c];
      t[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, t[0][1], 0, 0, 0);
      t[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, t[1][0], 0, 0, 0);
      t[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, t[1][1], 0, 0, 0);
    }
  }
  return tiles_to_rows<N>(t);
}

// The column reads of factor_times, issued by the caller ahead of the product (all of them at
// once, and as early as registers allow: issued four at a time beside the MFMAs, each group
// waited for a memory round trip of its own). Lane (c, kh) reads the NT elements d = NT c ..
// NT c + NT - 1 of column 2 s + kh for every K-step s (column 0 stands in past m; it is masked at
// its use).
template <int D, int N>
struct FactorLoads {
  uint32_t raw[N / 2][D / 64];
};

template <int D, int N>
__device__ __forceinline__ void factor_load(const uint16_t* __restrict__ base, const int m, FactorLoads<D, N>& L) {
  constexpr int NT = D / 32;
  static_assert(NT == 2 || NT == 4, "d of 64 or 128");
  const int lane = threadIdx.x;
  const int c = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int s = 0; s < N / 2; ++s) {
    const int col = 2 * s + kh;
    const uint16_t* p = base + (col < m ? col : 0) * D + NT * c;
    if constexpr (NT == 4) {
      const uint2 u = *reinterpret_cast<const uint2*>(p);
      L.raw[s][0] = u.x;
      L.raw[s][1] = u.y;
    } else {
      L.raw[s][0] = *reinterpret_cast<const uint32_t*>(p);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Y = F X for F (D x 64: the stored bf16 columns 0..m-1 of a factor) and X given as MFMA
// 32x32x2 B operands (rows 2 s + lane / 32 of column lane % 32). With NT = D / 32 tiles, row i
// of tile I is d = NT i + I, so that one lane's A operands of a column are NT consecutive
// elements (one load per K-step). Output: y[I][j] is Y[d][lane % 32] with
// d = NT (8 (j / 4) + 4 (lane / 32) + j % 4) + I.
// With FOLD, the same A operands also give F f for the vector f (cf: f_j at (j % 2) N / 2 + j / 2):
// fold[I] is lane half lane / 32's share of (F f)[NT (lane % 32) + I] (the other half's share is
// in the partner lane). L holds the columns' reads, issued by factor_load.
template <int D, int N, int FDT, bool FOLD = false>
__device__ __forceinline__ void factor_times(const FactorLoads<D, N>& L, const int m, const float (&xop)[N / 2],
                                             f32x16 (&y)[D / 32], const float* __restrict__ cf = nullptr,
                                             float* fold = nullptr) {
  constexpr int NT = D / 32;
  const int lane = threadIdx.x;
  const int kh = lane >> 5;
#pragma unroll
  for (int I = 0; I < NT; ++I) y[I] = zero16();
  if constexpr (FOLD) {
#pragma unroll
    for (int I = 0; I < NT; ++I) fold[I] = 0.f;
  }
#pragma unroll
  for (int s4 = 0; s4 < N / 8; ++s4) {
    float4 f4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (FOLD) f4 = *reinterpret_cast<const float4*>(cf + kh * (N / 2) + 4 * s4);
    const float fs[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
    for (int s1 = 0; s1 < 4; ++s1) {
      const int s = 4 * s4 + s1;
      const int col = 2 * s + kh;
      const bool ok = col < m;
      uint32_t w[2];
      w[0] = ok ? L.raw[s][0] : 0u;
      w[1] = (NT == 4 && ok) ? L.raw[s][NT / 2 - 1] : 0u;
#pragma unroll
      for (int I = 0; I < NT; ++I) {
        const uint32_t wi = w[I >> 1];
        const float a = (I & 1) ? hi16<FDT>(wi) : lo16<FDT>(wi);
        y[I] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, xop[s], y[I], 0, 0, 0);
        if constexpr (FOLD) fold[I] = fmaf(fs[s1], a, fold[I]);
      }
    }
  }
}

// The Sturm count at shift x: the number of eigenvalues of the tridiagonal (dg, e2 = e^2) below
// x. e2 is floored at FLT_MIN, so a zero pivot gives an infinite next pivot of the opposite sign
// (IEEE arithmetic) instead of NaN; pivots are counted by their sign bit, so that +0 followed by
// -inf and -0 followed by +inf count once each. The tridiagonal comes in registers (every lane
// holds all of it): read from LDS inside the recurrence, each pair of steps waited for an LDS
// round trip.
template <int N>
__device__ __forceinline__ int sturm1(const float (&dg)[N], const float (&e2)[N], const float x) {
  float q = dg[0] - x;
  uint32_t n = __float_as_uint(q) >> 31;
#pragma unroll
  for (int i = 1; i < N; ++i) {
    q = (dg[i] - x) - e2[i - 1] * __builtin_amdgcn_rcpf(q);
    n += __float_as_uint(q) >> 31;
  }
  return static_cast<int>(n);
}

}  // namespace cw

// The draws of one group of eight elements, as a call: inlined sixteen times per factor it
// pushed the stochastic-rounding kernel past the instruction cache.
__device__ __noinline__ uint4 sr_group_call(uint32_t rng_key, uint32_t site, int slot, int64_t unit,
                                            uint32_t window, int elem) {
  return sr_group(rng_key, site, 0u, slot, unit, window, elem);
}

template <int DK, int DV, bool DIAG, int N, int FDT, bool SR>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(N == 64 ? 2 : 3))) void k_compress_wave(const CompressArgs A) {
  using namespace cw;
  static_assert(N == 64 || N == 32, "core width");
  constexpr int LDL = N + 1;  // LDS row stride of L
  __shared__ Smem<N> S;
  const int lane = threadIdx.x;
  const int h = lane >> 5, c32 = lane & 31;
  const int row = N == 64 ? lane : c32;  // the core row this lane holds
  int64_t unit = blockIdx.x;
  if (A.list != nullptr) {   // list mode: the unit this block compresses (an index out of range: none)
    unit = A.list[blockIdx.x];
    if (unit < 0 || unit >= A.units) return;
  }
  const int r = A.rank, C = A.slots;
  float* __restrict__ sc = A.scale + unit * A.scale_len;
  int m = A.m;
  // spectrum mode (the diagnostic of seed_state_spectrum): every unit at its own column count,
  // the eigenvalues written out, the state left untouched
  float* __restrict__ spec = A.spectrum;
  if (spec != nullptr) {
    const uint32_t mu = __float_as_uint(sc[A.m_off]);
    m = mu > static_cast<uint32_t>(C) ? C : static_cast<int>(mu);
    if (m == 0) {
      if (lane <= RX) spec[unit * (RX + 1) + lane] = 0.f;
      return;
    }
  } else if (A.ragged) {
    // only the units whose own column count reached A.m (and holds columns beyond r)
    const int mu = static_cast<int>(__float_as_uint(sc[A.m_off]));
    if (mu < A.m || mu <= r || mu > C) return;
    m = mu;
  }
  uint16_t* __restrict__ Ub = reinterpret_cast<uint16_t*>(A.U) + unit * static_cast<int64_t>(C) * DK;
  uint16_t* __restrict__ Vb = reinterpret_cast<uint16_t*>(A.V) + unit * static_cast<int64_t>(C) * DV;
  // the unit's compression-window count (stochastic rounding's counter; one more at the end)
  const uint32_t window = __float_as_uint(sc[A.win_off]);
  // stochastic rounding is a separate instance: the nearest-rounding kernel carries none of its
  // code (a larger kernel misses the instruction cache more often)
  constexpr bool sr = SR;

  // ---- column scales (lazy decay), KDA's channel scales ----------------------------------------
  float csc;
  if constexpr (DIAG) {
    for (int i = lane; i < DK; i += 64) S.gam[i] = sc[i];
    csc = row < m ? 1.f : 0.f;
  } else {
    csc = row < m ? sc[row < r ? 0 : 1 + row - r] : 0.f;
  }
  S.colsc[row] = csc;
  // ---- the lazy sink: a = (slot-0 decay) a_0 + sum_{j >= r} c_j (true column j) (KDA:
  // Gamma . (a_0 + sum_j c_j U_j)). The sum U_s f, f_j = c_j (column scale j), rides on the
  // A operands of the U' product below (the same column reads); here only f goes to LDS.
  {
    const float f = row >= r && row < m ? sc[A.coef_off + row - r] * csc : 0.f;
    S.cf[(row & 1) * (N / 2) + (row >> 1)] = f;
  }
  wave_lds_sync();



  // ---- Grams of the stored columns -------------------------------------------------------------
  f32x32 GU_lo, GU_hi, GV_lo, GV_hi;
  {
    GramLoads<DK, N> lu;
    GramLoads<DV, N> lv;
    gram_load<DK, N>(Ub, m, lu);
    gram_load<DV, N>(Vb, m, lv);
    __builtin_amdgcn_sched_barrier(0);
    const M64 gu = gram<DK, DIAG, N, FDT>(lu, m, S.gam);
    const M64 gv = gram<DV, false, N, FDT>(lv, m, nullptr);
    GU_lo = gu.lo; GU_hi = gu.hi; GV_lo = gv.lo; GV_hi = gv.hi;
  }

  // ---- balance each column pair, folding the decay scale in -----------------------------------
  float du = 0.f, dv = 0.f;
#pragma unroll
  for (int c = 0; c < N; ++c) {
    if (row == c) { du = MGET(GU, c); dv = MGET(GV, c); }
  }
  float bal = 0.f, ibal = 0.f;
  if (du > 0.f && dv > 0.f && csc > 0.f) {
    const float qu = sqrtf(sqrtf(du)), qv = sqrtf(sqrtf(dv)), sq = sqrtf(csc);
    bal = sq * qv / qu;
    ibal = sq * qu / qv;
  }
  S.bal[row] = bal;
  S.ibal[row] = ibal;
  wave_lds_sync();
#pragma unroll
  for (int c4 = 0; c4 < N / 4; ++c4) {
    const float4 b4 = reinterpret_cast<const float4*>(S.bal)[c4];
    const float4 i4 = reinterpret_cast<const float4*>(S.ibal)[c4];
    const float bb[4] = {b4.x, b4.y, b4.z, b4.w}, ii[4] = {i4.x, i4.y, i4.z, i4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = 4 * c4 + e;
      MSET(GU, c, MGET(GU, c) * (bal * bb[e]));
      MSET(GV, c, MGET(GV, c) * (ibal * ii[e]));
    }
  }

  // ---- pivoted Cholesky of G_U (L column s into column p_s of the LDS copy) --------------------
  // In panels of kPanel steps. Within a panel the Gram is not updated: the pivot search needs
  // only the diagonal d (kept exactly, d -= l^2), and the pivot column is corrected for the
  // panel's earlier columns (kept one entry per lane in lp) by one readlane and one FMA each.
  // At the end of a panel its columns update the whole Gram at once, G -= Lp Lp^T, by MFMA
  // 32x32x2 (two columns per K-step, one 32-row tile block at a time, subtracted row by row).
  // A step thus reads no broadcast vector from LDS, which is what a rank-one update per step
  // waited on.
  float d = du * (bal * bal);
  uint64_t chosen = 0;
  {
    constexpr int kPanel = 8;
    const float tol = uni(kPivTol * wmax(d));
    bool done = !(tol > 0.f);
    for (int pb = 0; pb < N / kPanel && !done; ++pb) {  // uniform
      float lp[kPanel];
#pragma unroll
      for (int k = 0; k < kPanel; ++k) lp[k] = 0.f;
#pragma unroll
      for (int k = 0; k < kPanel; ++k) {
        if (done) break;  // uniform
        const bool was = (chosen >> row) & 1ull;
        // d is finite; with N = 32 the pivot is taken among lanes 0..31 (lanes 32.. hold copies)
        const int key = (!was && d > 0.f && (N == 64 || lane < 32)) ? __float_as_int(d) : -1;
        const int kmax = __builtin_amdgcn_readfirstlane(wmax_key(key));
        const float vmax = __int_as_float(kmax);
        if (kmax < 0 || !(vmax > tol)) {  // uniform
          done = true;
          break;
        }
        const uint64_t hit = __ballot(key == kmax);
        const int p = __builtin_amdgcn_readfirstlane(static_cast<int>(__builtin_ctzll(hit)));
        const float rp = __builtin_amdgcn_rsqf(vmax);
        const float piv = vmax * rp;
        float col = MGET(GU, p);
#pragma unroll
        for (int k2 = 0; k2 < k; ++k2) col = fmaf(-lp[k2], bcast(lp[k2], p), col);
        float l = was ? 0.f : col * rp;
        if (row == p) l = piv;
        S.Lp[row * LDL + p] = l;
        lp[k] = l;
        d -= l * l;
        chosen |= 1ull << p;
      }
      if (done) break;  // uniform: the Gram is not needed once the factorisation stops
#pragma unroll
      for (int I = 0; I < N / 32; ++I) {
        f32x16 t[2] = {zero16(), zero16()};
#pragma unroll
        for (int s2 = 0; s2 < kPanel / 2; ++s2) {
          float x = lp[2 * s2], y = lp[2 * s2 + 1];
          swap32(x, y);   // .x: rows of block 0, .y: block 1 (as rows_operand)
          const float aI = I == 0 ? x : y;
          t[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(aI, x, t[0], 0, 0, 0);
          if constexpr (N == 64) t[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(aI, y, t[1], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int rho = 32 * I + 8 * (j >> 2) + (j & 3);
          if constexpr (N == 64) {
            float x = t[0][j], y = t[1][j];
            swap32(x, y);
            MSET(GU, rho, MGET(GU, rho) - x);
            MSET(GU, rho + 4, MGET(GU, rho + 4) - y);
          } else {
            float x = t[0][j], y = t[0][j];
            swap32(x, y);
            MSET(GU, rho, MGET(GU, rho) - x);
            MSET(GU, rho + 4, MGET(GU, rho + 4) - y);
          }
        }
      }
    }
  }
  const int k = __builtin_popcountll(chosen);
  // columns never chosen (Schur residue below the tolerance) are zero in L
#pragma unroll
  for (int c = 0; c < N; ++c) {
    if (!((chosen >> c) & 1ull)) S.Lp[row * LDL + c] = 0.f;
  }
  wave_lds_sync();

  // ---- core B = L^T G_V L (in pivot-column order) ------------------------------------------------
  f32x32 Bm_lo, Bm_hi;
  {
    const M64 rt = times_L<N>(GV_lo, GV_hi, S.Lp);   // (G_V L)^T = L^T G_V, row per lane
    const M64 bt = times_L<N>(rt.lo, rt.hi, S.Lp);   // (L^T G_V L)^T, symmetric up to rounding
    Bm_lo = bt.lo; Bm_hi = bt.hi;
  }
  // The eigen phase works on B / bs (bs = largest |entry|): entries of order one keep every
  // intermediate (reflector norms, pivots of the shifted factorisations) far from the denormal
  // range, where the hardware reciprocal flushes to zero. Eigenvalues are scaled back below.
  float bs;
  {
    float mx = 0.f;
#pragma unroll
    for (int c = 0; c < N; ++c) mx = fmaxf(mx, fabsf(MGET(Bm, c)));
    bs = uni(wmax(mx));
    const float ibs = bs > 0.f ? 1.f / bs : 0.f;
#pragma unroll
    for (int c = 0; c < N; ++c) MSET(Bm, c, MGET(Bm, c) * ibs);
  }

  // ---- Householder tridiagonalisation, the reflectors kept in the registers they zero ---------
  // From step 8 qt on, v and w vanish on rows (and registers) below 8 qt, so block qt of the
  // steps works on registers 8 qt.. only.
#pragma unroll
  for (int qt = 0; qt < N / 8; ++qt) {
    const int c0 = 2 * qt;                       // first float4 block of registers touched
    for (int j = 8 * qt; j < (qt == N / 8 - 1 ? N - 2 : 8 * qt + 8); ++j) {
      const float colj = MGET(Bm, j);
      const bool tr = row > j;
      const float x = tr ? colj : 0.f;
      const float sig = uni(rsum<N>(x * x));
      const float x0 = bcast(x, j + 1);
      const float djj = bcast(colj, j);
      float t = 0.f, ej = x0, v = x;
      // below the floor the column is already reduced (B is scaled to entries <= 1)
      if (sig - x0 * x0 > 1e-30f * sig && sig > kReduceFloor) {  // uniform
        const float sr = __builtin_amdgcn_sqrtf(sig);   // v_sqrt_f32 (1 ulp; sig > 1e-30)
        const float al = x0 >= 0.f ? -sr : sr;
        const float v0 = x0 - al;
        t = 2.f * __builtin_amdgcn_rcpf(sig - x0 * x0 + v0 * v0);
        ej = al;
        v = (row == j + 1) ? v0 : x;
      }
      MSET(Bm, j, v);
      if (lane == 0) { S.dg[j] = djj; S.e[j] = ej; S.tau[j] = t; }
      if (t == 0.f) continue;  // uniform
      S.bvw[row] = v;
      wave_lds_sync();
      // every read of a step is issued before its arithmetic: the broadcast reads are what a
      // step waits on, and v is kept in registers for the update
      float4 vb[N / 4];
#pragma unroll
      for (int c4 = c0; c4 < N / 4; ++c4) vb[c4] = reinterpret_cast<const float4*>(S.bvw)[c4];
      __builtin_amdgcn_sched_barrier(0);
      float p4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c4 = c0; c4 < N / 4; ++c4) {
        const float4 b4 = vb[c4];
        p4[0] += MGET(Bm, 4 * c4 + 0) * b4.x;
        p4[1] += MGET(Bm, 4 * c4 + 1) * b4.y;
        p4[2] += MGET(Bm, 4 * c4 + 2) * b4.z;
        p4[3] += MGET(Bm, 4 * c4 + 3) * b4.w;
      }
      float p = (p4[0] + p4[1]) + (p4[2] + p4[3]);
      p = tr ? p * t : 0.f;
      const float K = 0.5f * t * uni(rsum<N>(p * v));
      const float w = tr ? p - K * v : 0.f;
      (S.bvw + N)[row] = w;
      wave_lds_sync();
      float4 wb[N / 4];
#pragma unroll
      for (int c4 = c0; c4 < N / 4; ++c4) wb[c4] = reinterpret_cast<const float4*>((S.bvw + N))[c4];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c4 = c0; c4 < N / 4; ++c4) {
        const float4 b4 = vb[c4];
        const float4 w4 = wb[c4];
        const float bb[4] = {b4.x, b4.y, b4.z, b4.w}, ww[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = 4 * c4 + e;
          MSET(Bm, c, fmaf(-w, bb[e], fmaf(-v, ww[e], MGET(Bm, c))));
        }
      }
      wave_lds_sync();
    }
  }
  {
    // the last 2 x 2 block (readlane outside any branch: every lane active)
    const float b62 = MGET(Bm, N - 2), b63 = MGET(Bm, N - 1);
    const float d62 = bcast(b62, N - 2), d63 = bcast(b63, N - 1), e62 = bcast(b63, N - 2);
    if (lane == 0) {
      S.dg[N - 2] = d62;
      S.dg[N - 1] = d63;
      S.e[N - 2] = e62;
      S.e[N - 1] = 0.f;
      S.tau[N - 2] = 0.f;
      S.tau[N - 1] = 0.f;
    }
  }
  wave_lds_sync();

  // ---- the rr largest eigenvalues by Sturm-count multisection --------------------------------------
  const int rr = spec != nullptr ? (RX < k ? RX : k) : (r < k ? r : k);
  float lam;
  {
    const float di = S.dg[row], ei = S.e[row], em = row > 0 ? S.e[row - 1] : 0.f;
    S.e2[row] = fmaxf(ei * ei, FLT_MIN);
    float lo = wmin(di - fabsf(em) - fabsf(ei));
    float hi = wmax(di + fabsf(em) + fabsf(ei));
    const float pad = 1e-6f * fmaxf(fabsf(lo), fabsf(hi)) + FLT_MIN;
    lo -= pad;
    hi += pad;
    wave_lds_sync();
    // the whole tridiagonal in registers for the Sturm recurrences (this phase has them free)
    float dgr[N], e2r[N];
#pragma unroll
    for (int c4 = 0; c4 < N / 4; ++c4) {
      const float4 d4 = reinterpret_cast<const float4*>(S.dg)[c4];
      const float4 f4 = reinterpret_cast<const float4*>(S.e2)[c4];
      dgr[4 * c4] = d4.x; dgr[4 * c4 + 1] = d4.y; dgr[4 * c4 + 2] = d4.z; dgr[4 * c4 + 3] = d4.w;
      e2r[4 * c4] = f4.x; e2r[4 * c4 + 1] = f4.y; e2r[4 * c4 + 2] = f4.z; e2r[4 * c4 + 3] = f4.w;
    }
    const int target = N - 1 - c32;  // the c32-th largest is the (N - 1 - c32)-th smallest
    {
      // first bracket from a shared grid of 64 points (one per lane, increasing with the lane):
      // the points with at most t eigenvalues below them are a prefix of the grid. One count
      // per lane here and then eleven trisection steps reach a finer bracket than two counts
      // per lane and ten steps, for one count less.
      const float step = (hi - lo) * (1.f / static_cast<float>(kGrid + 1));
      const float x1 = lo + static_cast<float>(lane + 1) * step;
      const int n1 = sturm1<N>(dgr, e2r, x1);
      float nlo = lo, nhi = hi;
      for (int g = 0; g < rr; ++g) {
        const int t = N - 1 - g;
        const int cnt = __builtin_popcountll(__ballot(n1 <= t));
        const float glo = cnt > 0 ? lo + static_cast<float>(cnt) * step : lo;
        const float ghi = cnt < kGrid ? lo + static_cast<float>(cnt + 1) * step : hi;
        if (c32 == g) { nlo = glo; nhi = ghi; }
      }
      lo = nlo;
      hi = nhi;
    }
    // trisection: the two interior points of the bracket, one Sturm count per lane (lane half h
    // probes point h + 1). Per Sturm count it narrows the bracket the most of the k-sections a
    // lane pair can run (a factor 3 for one count per lane; 5-section gives 5 for two), and the
    // phase is bound by the issue of the counts.
    for (int it = 0; it < NSEC; ++it) {
      const float step = (hi - lo) * (1.f / 3.f);
      const float x = lo + static_cast<float>(h + 1) * step;
      const int n = sturm1<N>(dgr, e2r, x);
      const float clo = n <= target ? x : -FLT_MAX;
      const float chi = n > target ? x : FLT_MAX;
      lo = fmaxf(lo, fmaxf(clo, partner(clo)));
      hi = fminf(hi, fminf(chi, partner(chi)));
    }
    lam = 0.5f * (lo + hi);
  }
  if (spec != nullptr) {
    // the RX largest eigenvalues of B (sigma_i^2 of U V^T; zero past the core's rank), then
    // their total, the trace (Householder keeps it: the sum of the tridiagonal's diagonal)
    float tr = S.dg[row];   // rows of unchosen pivots are zero
    tr = N == 64 ? wave_sum(tr) : group_sum<32>(tr);
    if (lane < RX) spec[unit * (RX + 1) + lane] = c32 < rr ? fmaxf(lam, 0.f) * bs : 0.f;
    if (lane == 0) spec[unit * (RX + 1) + RX] = fmaxf(tr, 0.f) * bs;
    return;
  }

  // eigenvalue floor: eigenvalues below the core's resolution give zero columns. They are the
  // trailing ones (lane c32 holds the c32-th largest), so the live ones are the first rl.
  const float lmax = uni(wmax(c32 < rr ? lam : 0.f));
  const bool live = c32 < rr && lam > lmax * kEigFloor;
  const int rl = __builtin_popcountll(__ballot(live && h == 0));

  // ---- eigenvectors of the tridiagonal: twisted factorisation per eigenvalue ------------------
  // Both lanes of a pair compute vector c32; lane half h keeps entries 2 s + h in Y[s]. One
  // register array serves both sweeps: slot i holds e_i / D-_{i+1} (bottom-up pivots) for
  // i >= kb and e_i / D+_i (top-down pivots, recomputed once the twist kb is known) for i < kb;
  // each z then overwrites the slot its own step consumed.
  float Y[N / 2];
  {
    float rt[N];
    float dm = S.dg[N - 1] - lam;
#pragma unroll
    for (int i = N - 2; i >= 0; --i) {
      const float ei = S.e[i];
      const float q = ei * __builtin_amdgcn_rcpf(nz(dm));
      rt[i] = q;
      dm = (S.dg[i] - lam) - ei * q;
    }
    rt[N - 1] = 0.f;
    float dp = S.dg[0] - lam, best = FLT_MAX;
    int kb = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) {        // twist: argmin |gamma_i|, gamma_i = D+_i - e_i^2 / D-_{i+1}
      const float ei = S.e[i];
      const float gm = (i < N - 1) ? dp - ei * rt[i] : dp;
      if (fabsf(gm) < best) { best = fabsf(gm); kb = i; }
      if (i < N - 1) dp = (S.dg[i + 1] - lam) - ei * (ei * __builtin_amdgcn_rcpf(nz(dp)));
    }
    dp = S.dg[0] - lam;
    const int kb0 = opaque(kb);
#pragma unroll
    for (int i = 0; i < N - 1; ++i) {    // e_i / D+_i into the slots above the twist
      const float ei = S.e[i];
      const float q = ei * __builtin_amdgcn_rcpf(nz(dp));
      if (i < kb0) rt[i] = q;
      dp = (S.dg[i + 1] - lam) - ei * q;
    }
    // below the twist z_{i+1} = -rt[i] z_i (into rt[i]); above it z_i = -rt[i] z_{i+1} (into rt[i])
    // (zc is 1 until the sweep passes the twist, so one comparison per slot selects)
    float zc = 1.f;
    const int kb1 = opaque(kb);
#pragma unroll
    for (int i = 0; i < N - 1; ++i) {
      const bool on = i >= kb1;
      const float z = -rt[i] * zc;
      if (on) rt[i] = z;
      zc = on ? z : 1.f;
    }
    zc = 1.f;
    const int kb2 = opaque(kb);
#pragma unroll
    for (int i = N - 2; i >= 0; --i) {
      const bool on = i < kb2;
      const float z = -rt[i] * zc;
      if (on) rt[i] = z;
      zc = on ? z : 1.f;
    }
    // z_j = rt[j] (j < kb), 1 (j = kb), rt[j - 1] (j > kb)
    float nn0 = 0.f, nn1 = 0.f;
    const int kb3 = opaque(kb);
#pragma unroll
    for (int s = 0; s < N / 2; ++s) {
      const int je = 2 * s, jo = 2 * s + 1;
      const float ze = je < kb3 ? rt[je] : (je == kb3 ? 1.f : rt[je > 0 ? je - 1 : 0]);
      const float zo = jo < kb3 ? rt[jo] : (jo == kb3 ? 1.f : rt[jo - 1]);
      Y[s] = h ? zo : ze;
      if (s & 1) nn1 += Y[s] * Y[s]; else nn0 += Y[s] * Y[s];
    }
    float nn = nn0 + nn1;
    nn += partner(nn);
    const bool ok = nn > 0.f && nn < FLT_MAX;
    const float inv = ok ? 1.f / sqrtf(nn) : 0.f;
#pragma unroll
    for (int s = 0; s < N / 2; ++s) Y[s] = !live ? 0.f : (ok ? Y[s] * inv : ((2 * s + h) == kb ? 1.f : 0.f));
  }

  // ---- modified Gram-Schmidt across the rr vectors, two at a time (norms applied at the end) ---
  // For the pair (y_c, y_c+1) with a = |y_c|^2, b = y_c . y_c+1, d = |y_c+1|^2, mu = b / a and
  // nu^2 = d - mu b: y_c+1 <- y_c+1 - mu y_c (scaled by 1 / nu at the end), y_c scaled by
  // 1 / sqrt(a); a later z with h1 = z . y_c, h2 = z . y_c+1 loses a2 = (h2 - mu h1) / nu^2
  // times y_c+1 and h1 / a - mu a2 times y_c.
  float ys = 1.f;
  // A vector that keeps less than kDep of its squared norm (1 after the twisted factorisation)
  // once the earlier ones are taken out is a copy of them (two shifts inside one unresolved
  // cluster give nearly the same vector): it is dropped, as dividing by its tiny residual would
  // blow rounding noise up into every direction.
  constexpr float kDep = 1e-4f;
  // The twisted factorisation leaves two vectors orthogonal up to about the core's rounding over
  // the gap between their eigenvalues, which for a gap above kClus times the largest is far
  // below the factor formats' resolution. So Gram-Schmidt runs only within clusters: runs of
  // consecutive eigenvalues (lane c32 holds the c32-th largest) whose gaps are at most kClus
  // times the largest. Bit c of sb is set when eigenvalue c starts a cluster.
  constexpr float kClus = 1e-3f;
  uint64_t sb;
  {
    const float lp = __shfl(lam, lane - 1);
    const bool start = c32 == 0 || !(lp - lam <= kClus * lmax);
    sb = __ballot(start && h == 0);
  }
  for (int c = 0; c < rl; c += 2) {
    const bool pair = c + 1 < rl;  // uniform
    float n4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < N / 2; ++s) n4[s & 3] += Y[s] * Y[s];
    float nn = (n4[0] + n4[1]) + (n4[2] + n4[3]);
    nn += partner(nn);
    // nothing to orthogonalise: c + 1 starts a cluster (or there is none), and so does c + 2
    if ((!pair || ((sb >> (c + 1)) & 1ull)) && (c + 2 >= rl || ((sb >> (c + 2)) & 1ull))) {  // uniform
      if (c32 == c || (pair && c32 == c + 1)) ys = nn > kDep ? 1.f / sqrtf(nn) : 0.f;
      continue;
    }
    if (c32 == c || c32 == c + 1) {
      float* buf = (c32 == c ? S.y2 : S.bvw) + N * h;
#pragma unroll
      for (int s4 = 0; s4 < N / 8; ++s4)
        reinterpret_cast<float4*>(buf)[s4] = make_float4(Y[4 * s4], Y[4 * s4 + 1], Y[4 * s4 + 2], Y[4 * s4 + 3]);
    }
    wave_lds_sync();
    float ya[N / 2], yb[N / 2];
#pragma unroll
    for (int s4 = 0; s4 < N / 8; ++s4) {
      const float4 a4 = reinterpret_cast<const float4*>(S.y2 + N * h)[s4];
      const float4 b4 = reinterpret_cast<const float4*>(S.bvw + N * h)[s4];
      ya[4 * s4] = a4.x; ya[4 * s4 + 1] = a4.y; ya[4 * s4 + 2] = a4.z; ya[4 * s4 + 3] = a4.w;
      yb[4 * s4] = b4.x; yb[4 * s4 + 1] = b4.y; yb[4 * s4 + 2] = b4.z; yb[4 * s4 + 3] = b4.w;
    }
    __builtin_amdgcn_sched_barrier(0);
    float p4[4] = {0.f, 0.f, 0.f, 0.f}, q4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < N / 2; ++s) {
      p4[s & 3] += Y[s] * ya[s];
      q4[s & 3] += Y[s] * yb[s];
    }
    float h1 = (p4[0] + p4[1]) + (p4[2] + p4[3]);
    float h2 = (q4[0] + q4[1]) + (q4[2] + q4[3]);
    h1 += partner(h1);
    h2 += partner(h2);
    const float a = bcast(nn, c);
    const float d = pair ? bcast(nn, c + 1) : 0.f;
    const float b = pair ? bcast(h1, c + 1) : 0.f;
    const float ia = a > kDep ? 1.f / a : 0.f;
    const float mu = b * ia;
    const float nu2 = d - mu * b;
    const float inu2 = pair && nu2 > kDep ? 1.f / nu2 : 0.f;
    float f1 = 0.f, f2 = 0.f;
    if (c32 > c + 1 || (!pair && c32 > c)) {
      f2 = pair ? (h2 - mu * h1) * inu2 : 0.f;
      f1 = h1 * ia - mu * f2;
    } else if (pair && c32 == c + 1) {
      f1 = mu;
    }
#pragma unroll
    for (int s = 0; s < N / 2; ++s) Y[s] = fmaf(-f2, yb[s], fmaf(-f1, ya[s], Y[s]));
    if (c32 == c) ys = a > kDep ? 1.f / sqrtf(a) : 0.f;
    if (pair && c32 == c + 1) ys = nu2 > kDep ? 1.f / sqrtf(nu2) : 0.f;
    wave_lds_sync();
  }
#pragma unroll
  for (int s = 0; s < N / 2; ++s) Y[s] = c32 < rl ? Y[s] * ys : 0.f;

  // ---- back-transformation Y <- H_0 H_1 ... H_{N-3} Y, two reflectors at a time --------------
  // H_{j-1} H_j Y = Y - t_j v_j g1 - t_{j-1} v_{j-1} (g0 - t_j kappa g1) with g1 = v_j^T Y,
  // g0 = v_{j-1}^T Y and kappa = v_{j-1}^T v_j. Vectors go through LDS with entry i at
  // (i % 2) 32 + i / 2, so that each lane half reads its parity as 8 float4. The loop is
  // software-pipelined over two buffers: once a pair's reads are issued, the next pair's
  // reflectors go to the other buffer and their kappa is reduced, so that neither the LDS round
  // trip nor the reduction waits in front of the pair's products. A pair whose two taus are zero
  // (columns that needed no reflection) is applied as it stands: f0 = f1 = 0 leave Y unchanged.
  {
    const int pos = (row & 1) * (N / 2) + (row >> 1);
    float nt1, nt0, nkap;
#define CW_PREP(J, B)                                                                              \
  do {                                                                                             \
    nt1 = S.tau[J];                                                                                \
    nt0 = S.tau[(J) - 1];                                                                          \
    const float pv1 = MGET(Bm, J), pv0 = MGET(Bm, (J) - 1);                                        \
    nkap = uni(rsum<N>(pv0 * pv1));                                                                \
    (S.y2 + (B) * N)[pos] = pv1;                                                                   \
    (S.bvw + (B) * N)[pos] = pv0;                                                                  \
  } while (0)
    CW_PREP(N - 3, 0);
    int buf = 0;
    // the pairs (j - 1, j) with j in [16 qb, 16 qb + 16) touch rows 16 qb.. only: slots 8 qb..
#pragma unroll
    for (int qb = N / 16 - 1; qb >= 0; --qb) {
      const int s40 = 2 * qb;   // first float4 of the slots touched
      for (int j = (qb == N / 16 - 1 ? N - 3 : 16 * qb + 15); j >= 16 * qb; j -= 2) {
        const float t1 = nt1, t0 = nt0, kap = nkap;
        wave_lds_sync();   // this pair's vectors, written one iteration ahead, are visible
        const float* __restrict__ y1p = S.y2 + buf * N + (N / 2) * h;
        const float* __restrict__ y0p = S.bvw + buf * N + (N / 2) * h;
        float a1[N / 2], a0[N / 2];
#pragma unroll
        for (int s4 = s40; s4 < N / 8; ++s4) {
          const float4 x4 = reinterpret_cast<const float4*>(y1p)[s4];
          const float4 z4 = reinterpret_cast<const float4*>(y0p)[s4];
          a1[4 * s4] = x4.x; a1[4 * s4 + 1] = x4.y; a1[4 * s4 + 2] = x4.z; a1[4 * s4 + 3] = x4.w;
          a0[4 * s4] = z4.x; a0[4 * s4 + 1] = z4.y; a0[4 * s4 + 2] = z4.z; a0[4 * s4 + 3] = z4.w;
        }
        __builtin_amdgcn_sched_barrier(0);
        if (j >= 3) CW_PREP(j - 2, buf ^ 1);  // uniform: the next pair, possibly the next block's
        buf ^= 1;
        float p4[4] = {0.f, 0.f, 0.f, 0.f}, q4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 4 * s40; s < N / 2; ++s) {
          p4[s & 3] += a1[s] * Y[s];
          q4[s & 3] += a0[s] * Y[s];
        }
        float g1 = (p4[0] + p4[1]) + (p4[2] + p4[3]);
        float g0 = (q4[0] + q4[1]) + (q4[2] + q4[3]);
        g1 += partner(g1);
        g0 += partner(g0);
        const float f1 = t1 * g1;
        const float f0 = t0 * (g0 - kap * f1);
#pragma unroll
        for (int s = 4 * s40; s < N / 2; ++s) Y[s] = fmaf(-f0, a0[s], fmaf(-f1, a1[s], Y[s]));
      }
    }
#undef CW_PREP
    wave_lds_sync();
  }

  const float q4 = live ? sqrtf(sqrtf(lam * bs)) : 1.f;   // of the unscaled eigenvalue
  const float qv = live ? 1.f / q4 : 0.f;          // lambda^(-1/4)
  const float ql = live ? 1.f / (q4 * q4) : 0.f;   // lambda^(-1/2)

  // ---- X_V = diag(ibal) L Y lambda^(-1/4) (m x r) ----------------------------------------------
  constexpr int NTI = N / 32;  // 32-row tiles of an m x r operand
  float xop[N / 2];
  {
    f32x16 xv[NTI];
#pragma unroll
    for (int I = 0; I < NTI; ++I) xv[I] = zero16();
#pragma unroll
    for (int s = 0; s < N / 2; ++s) {
#pragma unroll
      for (int I = 0; I < NTI; ++I)
        xv[I] = __builtin_amdgcn_mfma_f32_32x32x2f32(S.Lp[(32 * I + c32) * LDL + 2 * s + h], Y[s], xv[I], 0, 0, 0);
    }
#pragma unroll
    for (int I = 0; I < NTI; ++I) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 i4 = reinterpret_cast<const float4*>(S.ibal)[8 * I + 2 * q + h];
        xv[I][4 * q + 0] *= i4.x * qv;
        xv[I][4 * q + 1] *= i4.y * qv;
        xv[I][4 * q + 2] *= i4.z * qv;
        xv[I][4 * q + 3] *= i4.w * qv;
      }
      tile_to_kops(xv[I], I, xop);
    }
  }

  // ---- V' = V_s X_V (d_v x r), rounded to bf16; W = V_s^T V' -------------------------------------
  // V' of lane (c, h) is kept as bf16 pairs: word j NT/2 + e holds d = NT i_j + 2 e, + 1 with
  // i_j = 8 (j / 4) + 4 h + j % 4. Words 4 s .. 4 s + 3 are then the MFMA 32x32x16 B operand of
  // K-step s for d = 8 NT q + 4 NT h + 8 u + (0..7), q = s / (NT / 2), u = s % (NT / 2).
  constexpr int NV = DV / 32, NU = DK / 32;
  uint32_t vw[16 * NV / 2];
  {
    f32x16 vt[NV];
    FactorLoads<DV, N> fv;
    factor_load<DV, N>(Vb, m, fv);
    factor_times<DV, N, FDT>(fv, m, xop, vt);
    // elements d = NV i + (0 .. NV - 1) of column c32, i = 8 (j / 4) + 4 h + j % 4: the 8 / NV
    // values of j from a multiple of 8 / NV share one group of 8 (one draw call)
    uint4 dr = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int d0 = NV * (8 * (j >> 2) + 4 * h + (j & 3));
      if constexpr (SR) {
        if (j % (8 / NV) == 0) dr = sr_group_call(A.rng_key, kSiteCompressV, c32, unit, window, d0);
      }
#pragma unroll
      for (int e = 0; e < NV / 2; ++e) {
        const float x0 = vt[2 * e][j], x1 = vt[2 * e + 1][j];
        vw[j * NV / 2 + e] = sr ? (static_cast<uint32_t>(round_sr<FDT>(x0, draw16(dr, (d0 + 2 * e) & 7))) |
                                   (static_cast<uint32_t>(round_sr<FDT>(x1, draw16(dr, (d0 + 2 * e + 1) & 7))) << 16))
                                : pack2<FDT>(x0, x1);
      }
    }
  }
  // U' = M V' q with q = 1 / sigma, estimated twice: lambda^(-1/2) from the core, and
  // 1 / |V'|^2 from the stored (rounded) V' column, since |V'_c|^2 = lambda_c^(1/2) in exact
  // arithmetic. The two agree on every direction the fp32 core resolves. Below its resolution
  // either can be far off: a rounded lambda far below the column's true Rayleigh quotient makes
  // lambda^(-1/2) inflate the product, while a column tilted towards a strong direction makes
  // 1 / |V'|^2 count that direction twice. The smaller of the two keeps every column's term
  // M V' V'^T q within both a projection of M and the eigenvalue-scaled term.
  float vss = 0.f;
#pragma unroll
  for (int t = 0; t < 16 * NV / 2; ++t) {
    const float x0 = lo16<FDT>(vw[t]), x1 = hi16<FDT>(vw[t]);
    vss = fmaf(x0, x0, fmaf(x1, x1, vss));
  }
  vss += partner(vss);
  const float qu = (live && vss > 0.f) ? fminf(ql, 1.f / vss) : 0.f;
  FactorLoads<DK, N> fu;   // U_s's reads for U', issued once W's products are
  {
    f32x16 w[2] = {zero16(), zero16()};
    const bool ok0 = c32 < m, ok1 = N == 64 && c32 + 32 < m;
    const uint16_t* p0 = Vb + (ok0 ? c32 : 0) * DV + 4 * NV * h;
    const uint16_t* p1 = Vb + (ok1 ? c32 + 32 : 0) * DV + 4 * NV * h;
    // every read of V_s first (masked at its use), as in factor_times
    uint4 r0[DV / 16], r1[N == 64 ? DV / 16 : 1];
#pragma unroll
    for (int s = 0; s < DV / 16; ++s) {
      const int q = s / (NV / 2), u = s % (NV / 2);
      const int off = 8 * NV * q + 8 * u;
      r0[s] = *reinterpret_cast<const uint4*>(p0 + off);
      if constexpr (N == 64) r1[s] = *reinterpret_cast<const uint4*>(p1 + off);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < DV / 16; ++s) {
      uint4 u0 = r0[s];
      uint4 u1 = make_uint4(0u, 0u, 0u, 0u);
      if constexpr (N == 64) u1 = r1[s];
      if (!ok0) u0 = make_uint4(0u, 0u, 0u, 0u);
      if (!ok1) u1 = make_uint4(0u, 0u, 0u, 0u);
      const uint4 bw4 = make_uint4(vw[4 * s], vw[4 * s + 1], vw[4 * s + 2], vw[4 * s + 3]);
      using MF = Mf16<FDT>;
      using V8 = typename MF::V8;
      const V8 bop = __builtin_bit_cast(V8, bw4);
      w[0] = MF::mfma(__builtin_bit_cast(V8, u0), bop, w[0]);
      if constexpr (N == 64) w[1] = MF::mfma(__builtin_bit_cast(V8, u1), bop, w[1]);
    }
    factor_load<DK, N>(Ub, m, fu);
    // X_U = diag(colsc) W / |V'|^2 (U' = U_s D_c V_s^T V' / sigma), as B operands
#pragma unroll
    for (int I = 0; I < NTI; ++I) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 c4 = reinterpret_cast<const float4*>(S.colsc)[8 * I + 2 * q + h];
        w[I][4 * q + 0] *= c4.x * qu;
        w[I][4 * q + 1] *= c4.y * qu;
        w[I][4 * q + 2] *= c4.z * qu;
        w[I][4 * q + 3] *= c4.w * qu;
      }
      tile_to_kops(w[I], I, xop);
    }
  }

  // ---- write the r kept columns of V' (V_s is not read again: its last reads fed W, whose
  // MFMAs waited for them); its registers are then free for U' ------------------------------------
  __builtin_amdgcn_sched_barrier(0);
  if (c32 < r) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int i = 8 * (j >> 2) + 4 * h + (j & 3);
      if constexpr (NV == 4)
        *reinterpret_cast<uint2*>(Vb + c32 * DV + NV * i) = make_uint2(vw[2 * j], vw[2 * j + 1]);
      else
        *reinterpret_cast<uint32_t*>(Vb + c32 * DV + NV * i) = vw[j];
    }
  }

  // ---- U' = U_s X_U (d_k x r) (KDA: rows times Gamma) ---------------------------------------------
  uint32_t uw[16 * NU / 2];
  {
    f32x16 ut[NU];
    float* __restrict__ ap = A.a + unit * DK + NU * c32;
    float a0[NU], fold[NU];
    if (h == 0) {
      if constexpr (NU == 4) {
        const float4 v = *reinterpret_cast<const float4*>(ap);
        a0[0] = v.x; a0[1] = v.y; a0[2] = v.z; a0[3] = v.w;
      } else {
        const float2 v = *reinterpret_cast<const float2*>(ap);
        a0[0] = v.x; a0[1] = v.y;
      }
    }
    const float s0 = sc[0];
    factor_times<DK, N, FDT, true>(fu, m, xop, ut, S.cf, fold);
#pragma unroll
    for (int I = 0; I < NU; ++I) fold[I] += partner(fold[I]);
    if (h == 0) {
      float an[NU];
#pragma unroll
      for (int I = 0; I < NU; ++I)
        an[I] = DIAG ? S.gam[NU * c32 + I] * (a0[I] + fold[I]) : fmaf(s0, a0[I], fold[I]);
      if constexpr (NU == 4) *reinterpret_cast<float4*>(ap) = make_float4(an[0], an[1], an[2], an[3]);
      else *reinterpret_cast<float2*>(ap) = make_float2(an[0], an[1]);
    }
    uint4 dr = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int i = 8 * (j >> 2) + 4 * h + (j & 3);
      const int d0 = NU * i;
      if constexpr (SR) {
        if (j % (8 / NU) == 0) dr = sr_group_call(A.rng_key, kSiteCompressU, c32, unit, window, d0);
      }
      float g[NU];
#pragma unroll
      for (int I = 0; I < NU; ++I) g[I] = 1.f;
      if constexpr (DIAG) {
#pragma unroll
        for (int I = 0; I < NU; ++I) g[I] = S.gam[NU * i + I];
      }
#pragma unroll
      for (int e = 0; e < NU / 2; ++e) {
        const float x0 = ut[2 * e][j] * g[2 * e], x1 = ut[2 * e + 1][j] * g[2 * e + 1];
        uw[j * NU / 2 + e] = sr ? (static_cast<uint32_t>(round_sr<FDT>(x0, draw16(dr, (d0 + 2 * e) & 7))) |
                                   (static_cast<uint32_t>(round_sr<FDT>(x1, draw16(dr, (d0 + 2 * e + 1) & 7))) << 16))
                                : pack2<FDT>(x0, x1);
      }
    }
  }

  // ---- write the r kept columns of U' (every read of U_s is above) -------------------------------
  __builtin_amdgcn_sched_barrier(0);
  if (c32 < r) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int i = 8 * (j >> 2) + 4 * h + (j & 3);
      if constexpr (NU == 4)
        *reinterpret_cast<uint2*>(Ub + c32 * DK + NU * i) = make_uint2(uw[2 * j], uw[2 * j + 1]);
      else
        *reinterpret_cast<uint32_t*>(Ub + c32 * DK + NU * i) = uw[j];
    }
  }
  // decay scales restart at 1, sink coefficients at 0, the window count goes one up, m is r
  for (int i = lane; i < A.scale_len; i += 64)
    sc[i] = i < A.coef_off ? 1.f
            : (i < A.win_off ? 0.f
                             : __uint_as_float(i == A.win_off ? window + 1u : static_cast<uint32_t>(r)));
}

// ---- state energy (the diagnostic of seed_state_energy) for 16-bit factors ---------------------
// One wavefront per unit: the Grams of the stored columns by the MFMA routine above (KDA's
// Gamma^2 on the U side), the content energy sum_{i,j} G_U[i][j] G_V[i][j] (with the lazy column
// scales c_i c_j for GDN and Mamba-2) from the row-per-lane tiles; the sink a_true and the cross
// term (U^T a) . (V^T vbar) by lanes over d and over columns. Reads the factors once.
template <int DK, int DV, bool DIAG, int N, int FDT>
__global__ __launch_bounds__(64) void k_energy_wave(const EnergyArgs A) {
  using namespace cw;
  __shared__ float gam[DK];
  __shared__ float at[DK];
  __shared__ float colsc[N];
  const int lane = threadIdx.x;
  const int col = N == 64 ? lane : (lane & 31);
  const int64_t unit = blockIdx.x;
  const int r = A.rank, C = A.slots;
  const float* __restrict__ sc = A.scale + unit * A.scale_len;
  const uint32_t mu = __float_as_uint(sc[A.m_off]);   // unsigned; beyond the slots: all of them
  const int m = mu > static_cast<uint32_t>(C) ? C : static_cast<int>(mu);
  const uint16_t* __restrict__ Ub = reinterpret_cast<const uint16_t*>(A.U) + unit * static_cast<int64_t>(C) * DK;
  const uint16_t* __restrict__ Vb = reinterpret_cast<const uint16_t*>(A.V) + unit * static_cast<int64_t>(C) * DV;
  const float* __restrict__ vb = A.vbar + static_cast<int64_t>(unit % A.heads) * DV;

  if constexpr (DIAG) {
    for (int d = lane; d < DK; d += 64) gam[d] = sc[d];
  }
  const float cs = col < m ? (DIAG ? 1.f : sc[col < r ? 0 : 1 + col - r]) : 0.f;
  colsc[col] = cs;
  wave_lds_sync();

  // content: the Grams (zero beyond m), then sum over rho of c_rho G_U[rho][col] G_V[rho][col]
  float content;
  {
    GramLoads<DK, N> lu;
    GramLoads<DV, N> lv;
    gram_load<DK, N>(Ub, m, lu);
    gram_load<DV, N>(Vb, m, lv);
    __builtin_amdgcn_sched_barrier(0);
    const M64 gu = gram<DK, DIAG, N, FDT>(lu, m, gam);
    const M64 gv = gram<DV, false, N, FDT>(lv, m, nullptr);
    const f32x32 GU_lo = gu.lo, GU_hi = gu.hi, GV_lo = gv.lo, GV_hi = gv.hi;
    float p = 0.f;
#pragma unroll
    for (int rho = 0; rho < N; ++rho) p = fmaf(colsc[rho] * MGET(GU, rho), MGET(GV, rho), p);
    content = rsum<N>(p * cs);
  }

  // a_true = (slot-0 decay, or Gamma) a_0 + sum_{j >= r} c_j U_true[j], lanes over d
  for (int d = lane; d < DK; d += 64) {
    float acc = (DIAG ? gam[d] : sc[0]) * A.a[unit * DK + d];
    for (int j = r; j < m; ++j)
      acc = fmaf(sc[A.coef_off + j - r] * (DIAG ? gam[d] : colsc[j]), to_f32<FDT>(Ub[static_cast<int64_t>(j) * DK + d]), acc);
    at[d] = acc;
  }
  wave_lds_sync();
  float pa = 0.f, pv = 0.f;
  for (int d = lane; d < DK; d += 64) pa = fmaf(at[d], at[d], pa);
  for (int d = lane; d < DV; d += 64) pv = fmaf(vb[d], vb[d], pv);
  const float sink = wave_sum(pa) * wave_sum(pv);
  // cross: x_col = U_true[col] . a_true, y_col = V[col] . vbar (one lane per column)
  float xy = 0.f;
  if (col < m && (N == 64 || lane < 32)) {
    float x = 0.f, y = 0.f;
    const uint16_t* pu = Ub + static_cast<int64_t>(col) * DK;
    const uint16_t* pv2 = Vb + static_cast<int64_t>(col) * DV;
#pragma unroll 4
    for (int d = 0; d < DK; d += 8) {
      const uint4 w4 = *reinterpret_cast<const uint4*>(pu + d);
      const uint32_t ww[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d0 = d + 2 * e;
        x = fmaf((DIAG ? gam[d0] : 1.f) * lo16<FDT>(ww[e]), at[d0], x);
        x = fmaf((DIAG ? gam[d0 + 1] : 1.f) * hi16<FDT>(ww[e]), at[d0 + 1], x);
      }
    }
#pragma unroll 4
    for (int d = 0; d < DV; d += 8) {
      const uint4 w4 = *reinterpret_cast<const uint4*>(pv2 + d);
      const uint32_t ww[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y = fmaf(lo16<FDT>(ww[e]), vb[d + 2 * e], y);
        y = fmaf(hi16<FDT>(ww[e]), vb[d + 2 * e + 1], y);
      }
    }
    xy = (DIAG ? 1.f : cs) * x * y;
  }
  const float cross = wave_sum(xy);
  if (lane == 0) {
    A.out[unit * 3 + 0] = sink + 2.f * cross + content;
    A.out[unit * 3 + 1] = sink;
    A.out[unit * 3 + 2] = content;
  }
}

namespace {
using EnergyWaveFn = void (*)(const EnergyArgs);

template <int N, int FDT>
EnergyWaveFn pick_energy_width(const seed_shape& sh) {
  const bool diag = sh.kind == SEED_KDA;
  if (sh.d_k == 128 && sh.d_v == 128)
    return diag ? k_energy_wave<128, 128, true, N, FDT> : k_energy_wave<128, 128, false, N, FDT>;
  if (sh.d_k == 128 && sh.d_v == 64)
    return diag ? k_energy_wave<128, 64, true, N, FDT> : k_energy_wave<128, 64, false, N, FDT>;
  if (sh.d_k == 64 && sh.d_v == 128)
    return diag ? k_energy_wave<64, 128, true, N, FDT> : k_energy_wave<64, 128, false, N, FDT>;
  if (sh.d_k == 64 && sh.d_v == 64)
    return diag ? k_energy_wave<64, 64, true, N, FDT> : k_energy_wave<64, 64, false, N, FDT>;
  return nullptr;
}

EnergyWaveFn pick_energy_wave(const seed_shape& sh) {
  if (sh.rank + sh.period > 64) return nullptr;
  const bool narrow = sh.rank + sh.period <= 32;
  if (sh.factor_dtype == SEED_BF16) return narrow ? pick_energy_width<32, 1>(sh) : pick_energy_width<64, 1>(sh);
  if (sh.factor_dtype == SEED_F16) return narrow ? pick_energy_width<32, 2>(sh) : pick_energy_width<64, 2>(sh);
  return nullptr;
}
}  // namespace

hipError_t launch_energy_wave(const seed_shape& sh, const EnergyArgs& a, hipStream_t s, bool* used) {
  EnergyWaveFn fn = pick_energy_wave(sh);
  *used = fn != nullptr;
  if (!fn) return hipSuccess;
  hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(a.units)), dim3(64), 0, s, a);
  return hipGetLastError();
}

namespace {
using WaveFn = void (*)(const CompressArgs);

template <int N, int FDT, bool SR>
WaveFn pick_width(const seed_shape& sh) {
  const bool diag = sh.kind == SEED_KDA;
  if (sh.d_k == 128 && sh.d_v == 128)
    return diag ? k_compress_wave<128, 128, true, N, FDT, SR> : k_compress_wave<128, 128, false, N, FDT, SR>;
  if (sh.d_k == 128 && sh.d_v == 64)
    return diag ? k_compress_wave<128, 64, true, N, FDT, SR> : k_compress_wave<128, 64, false, N, FDT, SR>;
  if (sh.d_k == 64 && sh.d_v == 128)
    return diag ? k_compress_wave<64, 128, true, N, FDT, SR> : k_compress_wave<64, 128, false, N, FDT, SR>;
  if (sh.d_k == 64 && sh.d_v == 64)
    return diag ? k_compress_wave<64, 64, true, N, FDT, SR> : k_compress_wave<64, 64, false, N, FDT, SR>;
  return nullptr;
}

template <int N, int FDT>
WaveFn pick_rounding(const seed_shape& sh) {
  return sh.rounding == SEED_ROUND_STOCHASTIC ? pick_width<N, FDT, true>(sh) : pick_width<N, FDT, false>(sh);
}

template <int FDT>
WaveFn pick_format(const seed_shape& sh) {
  return sh.rank + sh.period <= 32 ? pick_rounding<32, FDT>(sh) : pick_rounding<64, FDT>(sh);
}

// 16-bit factors (bf16, fp16) with r <= 32
WaveFn pick_compress_wave(const seed_shape& sh) {
  if (sh.rank > cw::RX || sh.rank + sh.period > 64) return nullptr;
  if (sh.factor_dtype == SEED_BF16) return pick_format<1>(sh);
  if (sh.factor_dtype == SEED_F16) return pick_format<2>(sh);
  return nullptr;
}
}  // namespace

hipError_t launch_spectrum(const seed_shape& sh, const CompressArgs& a, hipStream_t s) {
  seed_shape nr = sh;
  nr.rounding = SEED_ROUND_NEAREST;  // no store is made: the nearest-rounding instance serves
  WaveFn fn = pick_compress_wave(nr);
  if (!fn) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(a.units)), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_compress_wave(const seed_shape& sh, const CompressArgs& a, hipStream_t s, bool* used) {
  WaveFn fn = pick_compress_wave(sh);
  *used = fn != nullptr;
  if (!fn) return hipSuccess;
  hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(compress_blocks(a))), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace seed
