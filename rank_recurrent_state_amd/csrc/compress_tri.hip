// Compression back to rank r with a tridiagonal eigensolver for the core (bf16 factors, r <= 32).
//
// Same contract and the same factored-core reduction as compress.hip: Grams of the stored
// columns; the decay scale folded into a balancing of each column pair; pivoted Cholesky
// G_U ~ L L^T; core B = L^T G_V L with eigenvalues sigma_i^2; U' = U_P L_P^{-T} Y_r
// lambda^(1/4) and V' = V L Y_r lambda^(-1/4). The eigensolver and the data movement differ:
//
//   Grams                 MFMA 32x32x16 bf16 straight from the stored factors (fp32 sums);
//   pivoted Cholesky      one wavefront, row per lane, with physical row/column swaps so that
//                         every trailing update is a contiguous block (G_V is permuted along);
//   B = L^T G_V L         MFMA 32x32x2 fp32, one 32 x 32 tile per wavefront;
//   eigenpairs of B       Householder reduction to tridiagonal T (one wavefront, row per lane,
//                         the vectors broadcast with readlane), the r largest eigenvalues by
//                         Sturm-count multisection (8 probes per step, 8 lanes per eigenvalue),
//                         one eigenvector of T per eigenvalue from a twisted factorisation of
//                         T - lambda I (twist at the smallest |gamma_k|), modified Gram-Schmidt
//                         across them, back-transformation by the stored reflectors;
//   X_V, reconstruction   MFMA 32x32x2 fp32; X_U by back substitution on L_P^T.
//
// Everything is fp32 in one 256-thread workgroup per unit with about 45 KB of LDS, so three
// units share a CU.
#include <float.h>

#include "common.hpp"
#include "kernels.hpp"

namespace seed {

namespace tri {

constexpr int MX = 64;          // maximum columns (r + T <= 64)
constexpr int LD = MX + 1;      // padded leading dimension of the m x m matrices
constexpr int RX = 32;          // maximum rank on this path
constexpr int EVLD = 66;        // leading dimension of the eigenvector block (RX rows)
constexpr int NB = 9;           // multisection steps (the bracket shrinks 9x per step)
constexpr float kPivTol = 1e-7f;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct Smem {
  float GA[MX * LD];            // G_U -> pivoted Cholesky in place (L in the lower part)
  float GB[MX * LD];            // G_V (permuted) -> T1 -> B -> reflectors -> X_V (m x r)
  float EV[RX * EVLD];          // eigenvectors [c][i] -> X_U [c][a]
  float bal[MX], ibal[MX], colsc[MX];
  float dg[MX], eo[MX], tv[MX], lam[RX];
  float gam[128];
  int perm[MX];
  int kk;
};

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(v, off, 64);
    const int oi = __shfl_xor(i, off, 64);
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// min / max over aligned groups of 8 lanes (every lane gets the result)
__device__ __forceinline__ float g8_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  return v;
}
__device__ __forceinline__ float g8_min(float v) {
  v = fminf(v, dpp<0xB1>(v));
  v = fminf(v, dpp<0x4E>(v));
  v = fminf(v, dpp<0x141>(v));
  return v;
}

__device__ __forceinline__ float bcast(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

__device__ __forceinline__ float nz(float x) {
  // a pivot that is exactly zero is replaced by a tiny one of negative sign
  return x == 0.f ? -FLT_MIN : x;
}

// 32 x 32 tile (rows a0.., columns b0..) of X X^T for m <= 64 rows of length D held as bf16
// rows of `base`; rows >= m count as zero. With ROWSCALE, the A operand carries gam^2 along the
// row (KDA's per-channel lazy decay: G_U = U_s Diag(Gamma^2) U_s^T).
template <int D, bool ROWSCALE>
__device__ __forceinline__ f32x16 gram_tile(const uint16_t* __restrict__ base, const int m, const int a0,
                                            const int b0, const float* __restrict__ gam) {
  const int lane = threadIdx.x & 63;
  const int i = lane & 31, kh = lane >> 5;
  const int ra = a0 + i, rb = b0 + i;
  f32x16 acc;
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = 0.f;
#pragma unroll
  for (int k0 = 0; k0 < D; k0 += 16) {
    uint4 ua = make_uint4(0u, 0u, 0u, 0u), ub = ua;
    if (ra < m) ua = *reinterpret_cast<const uint4*>(base + static_cast<int64_t>(ra) * D + k0 + 8 * kh);
    if (rb < m) ub = *reinterpret_cast<const uint4*>(base + static_cast<int64_t>(rb) * D + k0 + 8 * kh);
    bf16x8 va = __builtin_bit_cast(bf16x8, ua);
    const bf16x8 vb = __builtin_bit_cast(bf16x8, ub);
    if constexpr (ROWSCALE) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float gj = gam[k0 + 8 * kh + j];
        va[j] = static_cast<__bf16>(static_cast<float>(va[j]) * gj * gj);
      }
    }
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, vb, acc, 0, 0, 0);
  }
  return acc;
}

// Write a 32 x 32 MFMA accumulator tile to LDS rows r0.., columns c0.. (entries beyond nr x nc
// are skipped).
__device__ __forceinline__ void store_tile(float* __restrict__ M, const f32x16& acc, const int r0, const int c0,
                                           const int nr, const int nc) {
  const int lane = threadIdx.x & 63;
  const int col = c0 + (lane & 31);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int row = r0 + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
    if (row < nr && col < nc) M[row * LD + col] = acc[j];
  }
}

// Sturm count: number of eigenvalues of T (diagonal dg, off-diagonal eo) below x.
__device__ __forceinline__ int sturm(const float* __restrict__ dg, const float* __restrict__ eo,
                                     const int n, const float x) {
  float q = dg[0] - x;
  int c = q < 0.f;
  for (int i = 1; i < n; ++i) {
    const float e = eo[i - 1];
    q = dg[i] - x - e * e * __builtin_amdgcn_rcpf(nz(q));
    c += q < 0.f;
  }
  return c;
}

}  // namespace tri

template <int DK, int DV, bool DIAG>
__global__ __launch_bounds__(256) void k_compress_tri(const CompressArgs A) {
  using namespace tri;
  __shared__ Smem S;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wv = t >> 6;
  const int64_t unit = blockIdx.x;
  const int m = A.m, r = A.rank, C = A.slots;
  uint16_t* __restrict__ Ub = reinterpret_cast<uint16_t*>(A.U) + unit * static_cast<int64_t>(C) * DK;
  uint16_t* __restrict__ Vb = reinterpret_cast<uint16_t*>(A.V) + unit * static_cast<int64_t>(C) * DV;
  float* __restrict__ sc = A.scale + unit * A.scale_len;

  if constexpr (DIAG) {
    for (int i = t; i < DK; i += 256) S.gam[i] = sc[i];
    if (t < MX) S.colsc[t] = 1.f;
  } else {
    if (t < MX) S.colsc[t] = (t < m) ? sc[t < r ? 0 : 1 + t - r] : 0.f;
  }
  // the single-wavefront phases sweep whole 8-column blocks, so the matrices start at zero
  for (int idx = t; idx < MX * LD; idx += 256) { S.GA[idx] = 0.f; S.GB[idx] = 0.f; }
  __syncthreads();

  // ---- Grams of the stored columns (MFMA, one tile of each per wavefront) ---------------------
  {
    const int a0 = 32 * (wv >> 1), b0 = 32 * (wv & 1);
    if (a0 < m && b0 < m) {
      const f32x16 gu = gram_tile<DK, DIAG>(Ub, m, a0, b0, S.gam);
      const f32x16 gv = gram_tile<DV, false>(Vb, m, a0, b0, nullptr);
      store_tile(S.GA, gu, a0, b0, m, m);
      store_tile(S.GB, gv, a0, b0, m, m);
    }
  }
  __syncthreads();

  // ---- decay scales folded into a balancing of each column pair -------------------------------
  if (t < m) {
    const float gu = S.GA[t * LD + t], gv = S.GB[t * LD + t], c = S.colsc[t];
    if (gu > 0.f && gv > 0.f && c > 0.f) {
      const float qu = sqrtf(sqrtf(gu)), qv = sqrtf(sqrtf(gv)), s = sqrtf(c);
      S.bal[t] = s * qv / qu;
      S.ibal[t] = s * qu / qv;
    } else {
      S.bal[t] = 0.f;
      S.ibal[t] = 0.f;
    }
  }
  __syncthreads();
  for (int idx = t; idx < MX * MX; idx += 256) {
    const int a = idx >> 6, b = idx & 63;
    if (a < m && b < m) {
      S.GA[a * LD + b] *= S.bal[a] * S.bal[b];
      S.GB[a * LD + b] *= S.ibal[a] * S.ibal[b];
    }
  }
  __syncthreads();

  // ---- pivoted Cholesky of G_U, one wavefront, lane i owns row i ------------------------------
  // Pivot rows/columns are swapped into place (in GA and, alongside, in GB), so that position a
  // holds original column perm[a] and L is GA's lower triangle over the first k columns.
  if (wv == 0) {
    float d = (lane < m) ? S.GA[lane * LD + lane] : -1.f;
    int pm = lane;
    const float tau = kPivTol * wave_max(d);
    int k = m;
    for (int l = 0; l < m; ++l) {
      float v = (lane >= l && lane < m) ? d : -1.f;
      int p = lane;
      wave_argmax(v, p);
      if (!(v > tau) || !(tau > 0.f)) { k = l; break; }  // uniform
      if (p != l) {
        if (lane < m) {
          float x = S.GA[l * LD + lane];
          S.GA[l * LD + lane] = S.GA[p * LD + lane];
          S.GA[p * LD + lane] = x;
          x = S.GB[l * LD + lane];
          S.GB[l * LD + lane] = S.GB[p * LD + lane];
          S.GB[p * LD + lane] = x;
        }
        wave_lds_sync();
        if (lane < m) {
          float x = S.GA[lane * LD + l];
          S.GA[lane * LD + l] = S.GA[lane * LD + p];
          S.GA[lane * LD + p] = x;
          x = S.GB[lane * LD + l];
          S.GB[lane * LD + l] = S.GB[lane * LD + p];
          S.GB[lane * LD + p] = x;
        }
        const float dl = __shfl(d, l, 64), dq = __shfl(d, p, 64);
        const int pl = __shfl(pm, l, 64), pq = __shfl(pm, p, 64);
        if (lane == l) { d = dq; pm = pq; }
        else if (lane == p) { d = dl; pm = pl; }
        wave_lds_sync();
      }
      const float lll = sqrtf(v);
      // the L column, computed by every lane (zero outside (l, m)) so that readlane may take it
      // from any lane: values of lanes left out of a branch are undefined
      const bool below = lane > l && lane < m;
      const float gl = S.GA[lane * LD + l];
      const float li = below ? gl / lll : 0.f;
      if (lane == l) S.GA[l * LD + l] = lll;
      if (below) S.GA[lane * LD + l] = li;
      wave_lds_sync();
      // trailing update in blocks of 8 columns, all lanes active: L_j is zero outside (l, m), so
      // rows and columns outside the trailing block are rewritten unchanged
      for (int j0 = (l + 1) & ~7; j0 < m; j0 += 8) {
        float a[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = S.GA[lane * LD + j0 + e];
#pragma unroll
        for (int e = 0; e < 8; ++e) S.GA[lane * LD + j0 + e] = a[e] - li * bcast(li, j0 + e);
      }
      d -= li * li;
      wave_lds_sync();
    }
    if (lane < MX) S.perm[lane] = (lane < m) ? pm : 0;
    if (lane == 0) S.kk = k;
  }
  __syncthreads();
  const int k = S.kk;

  // L operand: L[i][b] = GA[i][b] for i >= b, b < k, else 0
  auto Lat = [&](int i, int b) -> float { return (i >= b && b < k && i < m) ? S.GA[i * LD + b] : 0.f; };

  // ---- core B = L^T G_V L (k x k) via MFMA 32x32x2 fp32 ---------------------------------------
  {
    const int a0 = 32 * (wv >> 1), b0 = 32 * (wv & 1);
    const int i = lane & 31, kh = lane >> 5;
    f32x16 acc;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.f;
    if (a0 < m && b0 < k) {                               // T1 = G_V L (m x k)
      for (int s = 0; s < m; s += 2) {
        const int kk = s + kh;
        const float av = (a0 + i < m && kk < m) ? S.GB[(a0 + i) * LD + kk] : 0.f;
        const float bv = Lat(kk, b0 + i);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
      }
    }
    __syncthreads();
    if (a0 < m && b0 < k) store_tile(S.GB, acc, a0, b0, m, k);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.f;
    if (a0 < k && b0 < k) {                               // B = L^T T1 (k x k)
      for (int s = 0; s < m; s += 2) {
        const int kk = s + kh;
        const float av = Lat(kk, a0 + i);
        const float bv = (kk < m && b0 + i < k) ? S.GB[kk * LD + b0 + i] : 0.f;
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
      }
    }
    __syncthreads();
    if (a0 < k && b0 < k) store_tile(S.GB, acc, a0, b0, k, k);
    __syncthreads();
    for (int idx = t; idx < MX * MX; idx += 256) {       // symmetrise the rounding
      const int a = idx >> 6, b = idx & 63;
      if (a < b && b < k) {
        const float sv = 0.5f * (S.GB[a * LD + b] + S.GB[b * LD + a]);
        S.GB[a * LD + b] = sv;
        S.GB[b * LD + a] = sv;
      }
    }
    __syncthreads();
  }
  const int n = k;

  // ---- Householder tridiagonalisation of B, one wavefront, lane i owns row i ------------------
  if (wv == 0) {
    for (int j = 0; j + 2 < n; ++j) {
      const bool tr = lane > j && lane < n;             // lane is in the trailing block
      const float xr = S.GB[lane * LD + j];
      const float x = tr ? xr : 0.f;
      const float sig = group_sum<64>(x * x);
      const float x0 = bcast(x, j + 1);
      float tau_j = 0.f, e_j = x0, v = x;
      if (sig - x0 * x0 > 1e-30f * sig && sig > 0.f) {
        const float al = (x0 >= 0.f) ? -sqrtf(sig) : sqrtf(sig);
        const float v0 = x0 - al;
        tau_j = 2.f / (sig - x0 * x0 + v0 * v0);
        e_j = al;
        v = (lane == j + 1) ? v0 : x;
      }
      if (tr) S.GB[lane * LD + j] = v;                   // the reflector, kept below the diagonal
      if (lane == j) { S.dg[j] = S.GB[j * LD + j]; S.eo[j] = e_j; S.tv[j] = tau_j; }
      if (tau_j == 0.f) continue;                         // uniform: column already reduced
      // all lanes active from here: v and w are zero outside the trailing block (every lane
      // computes them), so whole 8-column blocks need no test and readlane sees defined values
      float p = 0.f;                                      // p = tau B v
      for (int l0 = (j + 1) & ~7; l0 < n; l0 += 8) {
        float b[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) b[e] = S.GB[lane * LD + l0 + e];
#pragma unroll
        for (int e = 0; e < 8; ++e) p += b[e] * bcast(v, l0 + e);
      }
      p = tr ? p * tau_j : 0.f;
      const float K = 0.5f * tau_j * group_sum<64>(p * v);
      const float w = tr ? p - K * v : 0.f;              // B <- B - v w^T - w v^T
      for (int l0 = (j + 1) & ~7; l0 < n; l0 += 8) {
        float b[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) b[e] = S.GB[lane * LD + l0 + e];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          S.GB[lane * LD + l0 + e] = b[e] - (v * bcast(w, l0 + e) + w * bcast(v, l0 + e));
      }
    }
    if (n >= 2 && lane == n - 2) {
      S.dg[n - 2] = S.GB[(n - 2) * LD + n - 2];
      S.eo[n - 2] = S.GB[(n - 2) * LD + n - 1];        // own row (B stays symmetric)
      S.tv[n - 2] = 0.f;
    }
    if (n >= 1 && lane == n - 1) { S.dg[n - 1] = S.GB[(n - 1) * LD + n - 1]; S.eo[n - 1] = 0.f; S.tv[n - 1] = 0.f; }
  }
  __syncthreads();

  // ---- the rr largest eigenvalues by Sturm-count multisection -----------------------------------
  const int rr = r < n ? r : n;
  {
    const int g = t >> 3, s = t & 7;
    float lo = 0.f, hi = 0.f;
    for (int i = 0; i < n; ++i) {
      const float rad = (i > 0 ? fabsf(S.eo[i - 1]) : 0.f) + (i + 1 < n ? fabsf(S.eo[i]) : 0.f);
      lo = (i == 0) ? S.dg[i] - rad : fminf(lo, S.dg[i] - rad);
      hi = (i == 0) ? S.dg[i] + rad : fmaxf(hi, S.dg[i] + rad);
    }
    const float pad = 1e-6f * fmaxf(fabsf(lo), fabsf(hi)) + FLT_MIN;
    lo -= pad;
    hi += pad;
    const int target = n - 1 - g;  // c-th largest = (n-1-c)-th smallest
    if (g < rr) {                   // whole 8-lane groups take this branch together
      for (int it = 0; it < NB; ++it) {
        const float x = lo + static_cast<float>(s + 1) * (hi - lo) * (1.f / 9.f);
        const int cnt = tri::sturm(S.dg, S.eo, n, x);
        const float clo = (cnt <= target) ? x : -FLT_MAX;
        const float chi = (cnt > target) ? x : FLT_MAX;
        lo = fmaxf(lo, g8_max(clo));
        hi = fminf(hi, g8_min(chi));
      }
      if (s == 0) S.lam[g] = 0.5f * (lo + hi);
    }
  }
  __syncthreads();

  // ---- eigenvectors of T: twisted factorisation per eigenvalue ---------------------------------
  // Bottom-up pivots D-_i of T - lambda I = U- D- U-^T (registers), top-down pivots D+_i of
  // L+ D+ L+^T (parked in this thread's EV row), twist index kb = argmin |gamma_k| with
  // gamma_k = D+_k - e_k^2 / D-_{k+1}; then z_kb = 1, z_i = -(e_i / D+_i) z_{i+1} above kb and
  // z_{i+1} = -(e_i / D-_{i+1}) z_i below.
  if (t < rr) {
    const float lm = S.lam[t];
    float* zr = S.EV + t * EVLD;
    float Dm[MX];
#pragma unroll
    for (int i = MX - 1; i >= 0; --i) {
      if (i == n - 1) Dm[i] = S.dg[i] - lm;
      else if (i < n - 1) {
        const float e = S.eo[i];
        Dm[i] = S.dg[i] - lm - e * e * __builtin_amdgcn_rcpf(nz(Dm[i + 1]));
      } else Dm[i] = 1.f;
    }
    float best = FLT_MAX, dprev = 1.f;
    int kb = 0;
#pragma unroll
    for (int i = 0; i < MX; ++i) {
      if (i < n) {
        float dpi;
        if (i == 0) dpi = S.dg[0] - lm;
        else {
          const float e = S.eo[i - 1];
          dpi = S.dg[i] - lm - e * e * __builtin_amdgcn_rcpf(nz(dprev));
        }
        zr[i] = dpi;
        float gm = dpi;
        if (i < n - 1) {
          const float e = S.eo[i];
          gm = dpi - e * e * __builtin_amdgcn_rcpf(nz(Dm[i + 1]));
        }
        if (fabsf(gm) < best) { best = fabsf(gm); kb = i; }
        dprev = dpi;
      }
    }
    float nn = 1.f, zc = 1.f;
    for (int i = kb - 1; i >= 0; --i) {  // above the twist, from the parked D+_i
      zc = -S.eo[i] * __builtin_amdgcn_rcpf(nz(zr[i])) * zc;
      zr[i] = zc;
      nn += zc * zc;
    }
    zr[kb] = 1.f;
    zc = 1.f;
#pragma unroll
    for (int i = 0; i < MX - 1; ++i) {   // below the twist
      if (i >= kb && i + 1 < n) {
        zc = -S.eo[i] * __builtin_amdgcn_rcpf(nz(Dm[i + 1])) * zc;
        zr[i + 1] = zc;
        nn += zc * zc;
      }
    }
    const bool ok = nn > 0.f && nn < FLT_MAX;
    const float inv = ok ? 1.f / sqrtf(nn) : 0.f;
    for (int i = 0; i < n; ++i) zr[i] = ok ? zr[i] * inv : (i == kb ? 1.f : 0.f);
  }
  __syncthreads();

  // ---- modified Gram-Schmidt across the rr eigenvectors (8 lanes per vector) ------------------
  const int g = t >> 3, s8 = t & 7;
  float y[8];
  if (g < rr) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = s8 + 8 * e;
      y[e] = (i < n) ? S.EV[g * EVLD + i] : 0.f;
    }
  }
  for (int c = 0; c < rr; ++c) {
    if (g == c) {
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) p += y[e] * y[e];
      p = group_sum<8>(p);
      const float f = p > 0.f ? 1.f / sqrtf(p) : 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y[e] *= f;
        const int i = s8 + 8 * e;
        if (i < n) S.EV[g * EVLD + i] = y[e];
      }
    }
    __syncthreads();
    if (g > c && g < rr) {
      float h = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = s8 + 8 * e;
        if (i < n) h += y[e] * S.EV[c * EVLD + i];
      }
      h = group_sum<8>(h);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = s8 + 8 * e;
        if (i < n) y[e] -= h * S.EV[c * EVLD + i];
      }
    }
  }

  // ---- back-transformation Y = H_0 H_1 ... Z (reflectors in GB's lower part) ------------------
  if (g < rr) {
    for (int j = n - 3; j >= 0; --j) {
      const float tj = S.tv[j];
      if (tj == 0.f) continue;  // uniform
      float h = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = s8 + 8 * e;
        if (i > j && i < n) h += S.GB[i * LD + j] * y[e];
      }
      h = tj * group_sum<8>(h);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = s8 + 8 * e;
        if (i > j && i < n) y[e] -= h * S.GB[i * LD + j];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = s8 + 8 * e;
      if (i < n) S.EV[g * EVLD + i] = y[e];
    }
  }
  __syncthreads();

  // eigenvalue floor: tiny or negative eigenvalues give zero columns
  float lmax = 0.f;
  for (int c = 0; c < rr; ++c) lmax = fmaxf(lmax, S.lam[c]);
  const float lfl = lmax * 1e-14f;

  // ---- X_V = L Y_r lambda^(-1/4) (m x r, permuted rows) via MFMA, into GB ---------------------
  {
    const int a0 = 32 * wv;
    const int i = lane & 31, kh = lane >> 5;
    f32x16 acc;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.f;
    if (wv < 2 && a0 < m) {
      for (int s = 0; s < k; s += 2) {
        const int kk = s + kh;
        const float av = Lat(a0 + i, kk);
        const float bv = (i < rr && kk < k) ? S.EV[i * EVLD + kk] : 0.f;
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
      }
    }
    __syncthreads();  // GB's reflectors are dead from here on
    if (wv < 2 && a0 < m) {
      const int c = i;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int row = a0 + 8 * (j >> 2) + 4 * kh + (j & 3);
        if (row < m && c < r) {
          const float lm = (c < rr) ? S.lam[c] : 0.f;
          const bool live = c < rr && lm > lfl;
          S.GB[row * LD + c] = live ? acc[j] * S.ibal[S.perm[row]] / sqrtf(sqrtf(lm)) : 0.f;
        }
      }
    }
    __syncthreads();
  }

  // ---- X_U: L_P^T X = Y_r lambda^(1/4) by back substitution, 8 lanes per column ---------------
  if (g < r) {
    const float lm = (g < rr) ? S.lam[g] : 0.f;
    const bool live = g < rr && lm > lfl;
    const float q4 = live ? sqrtf(sqrtf(lm)) : 0.f;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int a = s8 + 8 * e;
      x[e] = (live && a < k) ? S.EV[g * EVLD + a] * q4 : 0.f;
    }
    if (live) {
      for (int a = k - 1; a >= 0; --a) {
        const int owner = a & 7, slot = a >> 3;
        float xa = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) if (e == slot) xa = x[e];
        xa = __shfl(xa, (lane & ~7) | owner, 64) / S.GA[a * LD + a];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int b = s8 + 8 * e;
          if (b == a) x[e] = xa;
          else if (b < a) x[e] -= S.GA[a * LD + b] * xa;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int a = s8 + 8 * e;
      S.EV[g * EVLD + a] = (a < k) ? x[e] * S.bal[S.perm[a]] : 0.f;
    }
  }
  __syncthreads();

  // ---- reconstruction via MFMA: U'^T tile = X_U^T U_s[perm], V'^T tile = X_V^T V[perm] --------
  // Each wavefront owns 32 output columns (d indices); its operands are read in full before the
  // barrier that precedes the in-place writes.
  {
    const int i = lane & 31, kh = lane >> 5;
    constexpr int NU = DK / 32;
    f32x16 acc;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.f;
    float bu[MX / 2];
    const int cu = 32 * wv + i;  // output column (d_k index) of this lane
#pragma unroll
    for (int s = 0; s < MX / 2; ++s) {
      const int a = 2 * s + kh;
      bu[s] = (wv < NU && a < k) ? bf16_to_f32(Ub[static_cast<int64_t>(S.perm[a]) * DK + cu]) : 0.f;
    }
    __syncthreads();  // all reads of U precede the writes below
    if (wv < NU) {
#pragma unroll
      for (int s = 0; s < MX / 2; ++s) {
        const int a = 2 * s + kh;
        const float av = (i < r && a < k) ? S.EV[i * EVLD + a] : 0.f;
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bu[s], acc, 0, 0, 0);
      }
      const float post = DIAG ? S.gam[cu] : 1.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int c = 8 * (j >> 2) + 4 * kh + (j & 3);
        if (c < r) Ub[static_cast<int64_t>(c) * DK + cu] = f32_to_bf16(acc[j] * post);
      }
    }
  }
  {
    const int i = lane & 31, kh = lane >> 5;
    constexpr int NV = DV / 32;
    f32x16 acc;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.f;
    float bv[MX / 2];
    const int cv = 32 * wv + i;
#pragma unroll
    for (int s = 0; s < MX / 2; ++s) {
      const int a = 2 * s + kh;
      bv[s] = (wv < NV && a < m) ? bf16_to_f32(Vb[static_cast<int64_t>(S.perm[a]) * DV + cv]) : 0.f;
    }
    __syncthreads();
    if (wv < NV) {
#pragma unroll
      for (int s = 0; s < MX / 2; ++s) {
        const int a = 2 * s + kh;
        const float av = (i < r && a < m) ? S.GB[a * LD + i] : 0.f;
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv[s], acc, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int c = 8 * (j >> 2) + 4 * kh + (j & 3);
        if (c < r) Vb[static_cast<int64_t>(c) * DV + cv] = f32_to_bf16(acc[j]);
      }
    }
  }
  for (int i = t; i < A.scale_len; i += 256) sc[i] = 1.f;
}

namespace {
using TriFn = void (*)(const CompressArgs);
}  // namespace

// The tridiagonal path serves bf16 factors with r <= 32 (fp32 factors keep the fp64 core).
TriFn pick_compress_tri(const seed_shape& sh) {
  if (sh.factor_dtype != SEED_BF16 || sh.rank > tri::RX || sh.rank + sh.period > tri::MX) return nullptr;
  const bool diag = sh.kind == SEED_KDA;
  if (sh.d_k == 128 && sh.d_v == 128) return diag ? k_compress_tri<128, 128, true> : k_compress_tri<128, 128, false>;
  if (sh.d_k == 128 && sh.d_v == 64) return diag ? k_compress_tri<128, 64, true> : k_compress_tri<128, 64, false>;
  if (sh.d_k == 64 && sh.d_v == 128) return diag ? k_compress_tri<64, 128, true> : k_compress_tri<64, 128, false>;
  if (sh.d_k == 64 && sh.d_v == 64) return diag ? k_compress_tri<64, 64, true> : k_compress_tri<64, 64, false>;
  return nullptr;
}

hipError_t launch_compress_tri(const seed_shape& sh, const CompressArgs& a, hipStream_t s, bool* used) {
  TriFn fn = pick_compress_tri(sh);
  *used = fn != nullptr;
  if (!fn) return hipSuccess;
  hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(a.units)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace seed
