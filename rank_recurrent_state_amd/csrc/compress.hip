// Compression of the factored content back to rank r, and the prefill-end compression of a
// dense state into the sink + rank-r form.
//
// Method (pages titled "Shallow Encoding Emits Deep Memories"): the factors are compressed
// back to rank r every T steps (picx.dev summary, "Open-Loop Error Bound (Corollary 4)";
// thelatestinai.com figures & tables, overview table), and a state leaving the prefill is
// split along vbar (picx.dev summary, Lemma 1) and brought to rank r once. The pages print no
// compression algorithm; the one implemented is the exact best rank-r approximation of the
// content, computed through a small core:
//
//   1. Grams of the stored columns, G_U = U_s^T U_s (KDA: with the per-channel Gamma of the
//      lazy decay applied) and G_V = V^T V;
//   2. the per-column decay scale c_j (GDN, Mamba-2) is folded in together with a balancing
//      of each column pair: u_j <- sqrt(c_j) (|v_j| / |u_s,j|)^(1/2) u_s,j and
//      v_j <- sqrt(c_j) (|u_s,j| / |v_j|)^(1/2) v_j, an exact rescaling of the rank-one term
//      c_j u_s,j v_j^T that never squares c_j (decay products underflow in Mamba-2); pairs
//      with a zero side are dropped exactly;
//   3. pivoted Cholesky G_U ~ L L^T (L is m x k): U = O L^T with O orthonormal, so
//      U V^T = O (V L)^T and the core B = L^T G_V L (k x k) has eigenvalues sigma_i^2;
//   4. cyclic Jacobi on B (round-robin pairing, up to 32 rotations per round in parallel);
//   5. top r eigenpairs (Y_r, lambda_r): U' = U_P L_P^{-T} Y_r lambda_r^(1/4) and
//      V' = V L Y_r lambda_r^(-1/4), i.e. sqrt(sigma) on both factors.
//
// Precision. With bf16 factors the core runs in fp32. With fp32 factors the Grams, the core
// and the reconstruction sums run in fp64 (MI355X's fp64 vector rate equals its non-packed
// fp32 rate): an fp32 Schur complement cannot resolve column residuals below ~3e-4 of the
// largest column, which a fast-decaying (numerically low-rank) state needs.
//
// Design (gfx950): one 256-thread workgroup per unit; all small matrices (m <= 64) live in
// LDS with a padded leading dimension; the reconstruction's inputs are staged in LDS before
// any output is written (the output overwrites the first r column slots in place).
#include <float.h>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace seed {

constexpr int MX = 64;       // maximum columns handled by the core (r + T <= 64)
constexpr int LD = MX + 1;   // padded leading dimension of the m x m matrices
constexpr int kMaxSweeps = 16;
constexpr int kJacobiMaxSweeps = 30;  // one-sided Jacobi sweeps for 128 x 128 dense states, at most
constexpr double kJacobiTol = 1e-8;   // a pair is rotated while |w_p . w_q| > kJacobiTol |w_p| |w_q|

template <typename CT> struct Tol;
template <> struct Tol<float> {
  static constexpr float piv = 1e-7f;      // pivot stops at Schur diagonal <= piv * max diagonal
  static constexpr float jac = 1e-7f;      // Jacobi skips |b_pq| <= jac * sqrt(b_pp b_qq)
  static constexpr float tiny = FLT_MIN;
  static constexpr float lfloor = 1e-14f;  // eigenvalues <= lfloor * max give zero columns
};
template <> struct Tol<double> {
  static constexpr double piv = 1e-13;
  static constexpr double jac = 1e-14;
  static constexpr double tiny = DBL_MIN;
  static constexpr double lfloor = 1e-28;
};

template <typename CT>
struct Core {
  CT GA[MX * LD];   // G_U -> Schur complement -> T1 = G_V L -> X_V (m x r)
  CT GB[MX * LD];   // G_V -> B -> X_U (k x r)
  CT LM[MX * LD];   // L (m x k); staging area before and after
  CT YM[MX * LD];   // Jacobi eigenvectors; staging area before and after (contiguous with LM)
  CT bal[MX];    // balanced U column = bal * stored column
  CT ibal[MX];   // balanced V column = ibal * V column
  CT colsc[MX];  // per-column decay scale c_j (1 when already applied)
  CT lam[MX];
  CT dsh[MX];
  CT rc[MX / 2], rs[MX / 2];
  CT pivval, tau;
  int perm[MX], sel[MX], chosen[MX], pp[MX / 2], qq[MX / 2];
  int kk, piv, flag[3];
};

template <typename T>
__device__ __forceinline__ void wave_argmax(T& v, int& i) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const T ov = __shfl_xor(v, off, 64);
    const int oi = __shfl_xor(i, off, 64);
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
  }
}

template <typename CT> __device__ __forceinline__ CT csqrt(CT x);
template <> __device__ __forceinline__ float csqrt<float>(float x) { return sqrtf(x); }
template <> __device__ __forceinline__ double csqrt<double>(double x) { return sqrt(x); }

// ---- the core: from the stored-column Gram G_Us (in GA), G_V (in GB) and the column scales
// (colsc), m x m, to X_U (GB, k x r, rows in pivot order, applied to the stored U columns) and
// X_V (GA, m x r, applied to the V columns) -------------------------------------------------
template <typename CT>
__device__ void core_truncate(Core<CT>& S, const int m, const int r) {
  using TL = Tol<CT>;
  const int t = threadIdx.x;

  // 2. fold the decay scales and balance the column pairs
  if (t < m) {
    const CT gu = S.GA[t * LD + t], gv = S.GB[t * LD + t], c = S.colsc[t];
    if (gu > CT(0) && gv > CT(0) && c > CT(0)) {
      const CT qu = csqrt(csqrt(gu)), qv = csqrt(csqrt(gv)), sc = csqrt(c);
      S.bal[t] = sc * qv / qu;
      S.ibal[t] = sc * qu / qv;
    } else {
      S.bal[t] = CT(0);
      S.ibal[t] = CT(0);
    }
  }
  __syncthreads();
  for (int idx = t; idx < m * m; idx += 256) {
    const int a = idx / m, b = idx - a * m;
    S.GA[a * LD + b] *= S.bal[a] * S.bal[b];
    S.GB[a * LD + b] *= S.ibal[a] * S.ibal[b];
  }
  __syncthreads();

  // 3. pivoted Cholesky of G_U (right-looking, Schur complement kept in GA)
  if (t < m) { S.dsh[t] = S.GA[t * LD + t]; S.chosen[t] = 0; }
  __syncthreads();
  if (t < kWave) {
    CT v = (t < m) ? S.dsh[t] : CT(0);
    int i = t;
    wave_argmax(v, i);
    if (t == 0) S.tau = TL::piv * v;
  }
  __syncthreads();
  const CT tau = S.tau;
  int k = 0;
  for (int l = 0; l < m; ++l) {
    if (t < kWave) {
      CT v = (t < m && !S.chosen[t]) ? S.dsh[t] : CT(-1);
      int i = t;
      wave_argmax(v, i);
      if (t == 0) { S.piv = i; S.pivval = v; }
    }
    __syncthreads();
    const int p = S.piv;
    const CT dp = S.pivval;
    if (!(dp > tau) || !(tau > CT(0))) break;  // uniform across the workgroup
    const CT sq = csqrt(dp);
    if (t < m) {
      CT Lv;
      if (t == p) Lv = sq;
      else if (S.chosen[t]) Lv = CT(0);
      else Lv = S.GA[t * LD + p] / sq;
      S.LM[t * LD + l] = Lv;
    }
    __syncthreads();
    if (t == 0) { S.chosen[p] = 1; S.perm[l] = p; }
    for (int idx = t; idx < m * m; idx += 256) {
      const int a = idx / m, b = idx - a * m;
      S.GA[a * LD + b] -= S.LM[a * LD + l] * S.LM[b * LD + l];
    }
    __syncthreads();
    if (t < m) S.dsh[t] = S.GA[t * LD + t];
    k = l + 1;
    __syncthreads();
  }

  // core B = L^T G_V L: T1 = G_V L into GA, then B into GB (symmetric by construction)
  for (int idx = t; idx < m * k; idx += 256) {
    const int i = idx / k, b = idx - i * k;
    CT acc = CT(0);
    for (int j = 0; j < m; ++j) acc += S.GB[i * LD + j] * S.LM[j * LD + b];
    S.GA[i * LD + b] = acc;
  }
  __syncthreads();
  for (int idx = t; idx < k * k; idx += 256) {
    const int a = idx / k, b = idx - a * k;
    if (a > b) continue;
    CT acc = CT(0);
    for (int i = 0; i < m; ++i) acc += S.LM[i * LD + a] * S.GA[i * LD + b];
    S.GB[a * LD + b] = acc;
    S.GB[b * LD + a] = acc;
  }
  const int n = (k + 1) & ~1;  // Jacobi size, padded to even
  __syncthreads();
  if (k < n) {
    for (int idx = t; idx < n; idx += 256) { S.GB[k * LD + idx] = CT(0); S.GB[idx * LD + k] = CT(0); }
  }
  for (int idx = t; idx < n * n; idx += 256) {
    const int i = idx / n, j = idx - i * n;
    S.YM[i * LD + j] = (i == j) ? CT(1) : CT(0);
  }
  if (t < 3) S.flag[t] = 0;
  __syncthreads();

  // 4. cyclic Jacobi, round-robin pairs: round rho pairs (n-1, rho) and
  //    ((rho + i) mod (n-1), (rho - i) mod (n-1)) for i = 1 .. n/2 - 1
  const int np = n / 2;
  for (int sw = 0; sw < kMaxSweeps && n > 1; ++sw) {
    if (t == 0) S.flag[(sw + 1) % 3] = 0;
    for (int rho = 0; rho < n - 1; ++rho) {
      if (t < np) {
        int p, q;
        if (t == 0) { p = n - 1; q = rho; }
        else { p = (rho + t) % (n - 1); q = (rho - t + (n - 1)) % (n - 1); }
        const CT app = S.GB[p * LD + p], aqq = S.GB[q * LD + q], apq = S.GB[p * LD + q];
        CT c = CT(1), s = CT(0);
        if (fabs(apq) > TL::jac * csqrt(fabs(app * aqq)) && fabs(apq) > TL::tiny) {
          const CT th = (aqq - app) / (CT(2) * apq);
          const CT ath = fabs(th);
          CT tt = (ath > CT(1e18)) ? CT(0.5) / ath : CT(1) / (ath + csqrt(CT(1) + th * th));
          if (th < CT(0)) tt = -tt;
          c = CT(1) / csqrt(CT(1) + tt * tt);
          s = tt * c;
          S.flag[sw % 3] = 1;
        }
        S.pp[t] = p; S.qq[t] = q; S.rc[t] = c; S.rs[t] = s;
      }
      __syncthreads();
      // B <- R^T B R on the 2x2 blocks (upper triangle of the pair grid, mirrored)
      for (int blk = t; blk < np * np; blk += 256) {
        const int bi = blk / np, bj = blk - bi * np;
        if (bi > bj) continue;
        const CT si = S.rs[bi], sj = S.rs[bj];
        if (si == CT(0) && sj == CT(0)) continue;
        const int pi = S.pp[bi], qi = S.qq[bi], pj = S.pp[bj], qj = S.qq[bj];
        const CT ci = S.rc[bi], cj = S.rc[bj];
        const CT x00 = S.GB[pi * LD + pj], x01 = S.GB[pi * LD + qj];
        const CT x10 = S.GB[qi * LD + pj], x11 = S.GB[qi * LD + qj];
        const CT y00 = x00 * cj - x01 * sj, y01 = x00 * sj + x01 * cj;
        const CT y10 = x10 * cj - x11 * sj, y11 = x10 * sj + x11 * cj;
        const CT z00 = ci * y00 - si * y10, z01 = ci * y01 - si * y11;
        const CT z10 = si * y00 + ci * y10, z11 = si * y01 + ci * y11;
        if (bi == bj) {
          // the rotation annihilates b_pq
          S.GB[pi * LD + pi] = z00; S.GB[qi * LD + qi] = z11;
          S.GB[pi * LD + qi] = CT(0); S.GB[qi * LD + pi] = CT(0);
        } else {
          S.GB[pi * LD + pj] = z00; S.GB[pi * LD + qj] = z01;
          S.GB[qi * LD + pj] = z10; S.GB[qi * LD + qj] = z11;
          S.GB[pj * LD + pi] = z00; S.GB[qj * LD + pi] = z01;
          S.GB[pj * LD + qi] = z10; S.GB[qj * LD + qi] = z11;
        }
      }
      // Y <- Y R
      for (int idx = t; idx < n * np; idx += 256) {
        const int row = idx / np, pr = idx - row * np;
        const CT s = S.rs[pr];
        if (s == CT(0)) continue;
        const int p = S.pp[pr], q = S.qq[pr];
        const CT c = S.rc[pr];
        const CT yp = S.YM[row * LD + p], yq = S.YM[row * LD + q];
        S.YM[row * LD + p] = c * yp - s * yq;
        S.YM[row * LD + q] = s * yp + c * yq;
      }
      __syncthreads();
    }
    if (S.flag[sw % 3] == 0) break;  // no rotation in this sweep: converged
  }

  // 5. eigenvalues, descending order, top r
  if (t < k) S.lam[t] = S.GB[t * LD + t];
  __syncthreads();
  CT lmax = CT(0);
  for (int j = 0; j < k; ++j) lmax = S.lam[j] > lmax ? S.lam[j] : lmax;
  const CT lfl = lmax * TL::lfloor;
  if (t < k) {
    const CT li = S.lam[t];
    int rank = 0;
    for (int j = 0; j < k; ++j) {
      const CT lj = S.lam[j];
      rank += (lj > li) || (lj == li && j < t);
    }
    if (rank < r) S.sel[rank] = (li > lfl) ? t : -1;
  }
  if (t >= k && t < r) S.sel[t] = -1;
  __syncthreads();

  // X_V = L Y_r lambda^(-1/4) (m x r) into GA, balancing folded in
  for (int idx = t; idx < m * r; idx += 256) {
    const int j = idx / r, c = idx - j * r;
    const int e = S.sel[c];
    CT acc = CT(0);
    if (e >= 0) {
      for (int b = 0; b < k; ++b) acc += S.LM[j * LD + b] * S.YM[b * LD + e];
      acc *= S.ibal[j] / csqrt(csqrt(S.lam[e]));
    }
    S.GA[j * LD + c] = acc;
  }
  // right-hand side Y_r lambda^(1/4) into GB (k x r)
  for (int idx = t; idx < k * r; idx += 256) {
    const int a = idx / r, c = idx - a * r;
    const int e = S.sel[c];
    S.GB[a * LD + c] = (e >= 0) ? S.YM[a * LD + e] * csqrt(csqrt(S.lam[e])) : CT(0);
  }
  __syncthreads();
  // X_U: solve L_P^T X = rhs by back substitution (L_P[a][b] = L[perm[a]][b], lower
  // triangular), one column per thread; then fold the balancing (with the decay scale)
  if (t < r) {
    const int c = t;
    for (int a = k - 1; a >= 0; --a) {
      CT acc = S.GB[a * LD + c];
      for (int b = a + 1; b < k; ++b) acc -= S.LM[S.perm[b] * LD + a] * S.GB[b * LD + c];
      S.GB[a * LD + c] = acc / S.LM[S.perm[a] * LD + a];
    }
    for (int a = 0; a < k; ++a) {
      const int pa = S.perm[a];
      S.GB[a * LD + c] *= S.bal[pa];
    }
  }
  if (t == 0) S.kk = k;
  __syncthreads();
}

// Gram of m <= 64 columns of length D held as rows of `base` (column j at base + j * D),
// each value scaled by gam[i] (MODE 1, per row of the column) or not at all (MODE 0). The
// m x m result goes to out (leading dimension LD). Staging uses S.LM; accumulation is AccT
// on 4 x 4 tiles per thread.
template <typename CT, typename AccT, int D, int FDT, int MODE>
__device__ void gram_rows(Core<CT>& S, const stor_t<FDT>* __restrict__ base, const int m,
                          const float* __restrict__ gam, CT* __restrict__ out) {
  const int t = threadIdx.x;
  const int ta = t >> 4, tb = t & 15;
  AccT acc[4][4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[e][f] = AccT(0);
  CT* st = S.LM;
  for (int i0 = 0; i0 < D; i0 += 64) {
    for (int idx = t; idx < 64 * 64; idx += 256) {
      const int j = idx >> 6, ii = idx & 63;
      CT v = CT(0);
      if (j < m) {
        v = CT(to_f32<FDT>(base[static_cast<int64_t>(j) * D + i0 + ii]));
        if constexpr (MODE == 1) v *= CT(gam[i0 + ii]);
      }
      st[j * LD + ii] = v;
    }
    __syncthreads();
    if (4 * ta < m && 4 * tb < m) {
      for (int ii = 0; ii < 64; ++ii) {
        AccT av[4], bv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) { av[e] = AccT(st[(4 * ta + e) * LD + ii]); bv[e] = AccT(st[(4 * tb + e) * LD + ii]); }
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int f = 0; f < 4; ++f) acc[e][f] += av[e] * bv[f];
      }
    }
    __syncthreads();
  }
  if (4 * ta < m && 4 * tb < m) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int f = 0; f < 4; ++f)
        if (4 * ta + e < m && 4 * tb + f < m) out[(4 * ta + e) * LD + 4 * tb + f] = CT(acc[e][f]);
  }
  __syncthreads();
}

// How the factor stores of one call round: nearest-even, or stochastic with draws for the
// store site (element e of column c of the unit takes its draw from the group e / 8).
struct Rounding {
  bool sr;
  uint32_t key;
  uint32_t site;
  int64_t unit;
  uint32_t window;
};

template <int FDT>
__device__ __forceinline__ stor_t<FDT> round_store(float x, const Rounding& R, int col, int elem) {
  if constexpr (FDT != 0) {
    if (R.sr) return round_sr<FDT>(x, draw16(sr_group(R.key, R.site, 0u, col, R.unit, R.window, elem), elem & 7));
  }
  return from_f32<FDT>(x);
}

// Reconstruction: out[c][i] = post_i * sum_{a<n} st[a][i] * X[a][c] for c < r, with the n
// source rows of length D staged in S.LM..S.YM (n * D <= 2 * MX * LD values).
template <typename CT, int D, int FDT, bool ROWSCALE>
__device__ void reconstruct_rows(Core<CT>& S, const CT* __restrict__ X, const int n, const int r,
                                 const float* __restrict__ post, stor_t<FDT>* __restrict__ out,
                                 const Rounding& R) {
  const int t = threadIdx.x;
  constexpr int NCS = 256 / D;
  const int i = t % D, cset = t / D;
  const CT* st = S.LM;
  for (int c = cset; c < r; c += NCS) {
    CT acc = CT(0);
    for (int a = 0; a < n; ++a) acc += st[a * D + i] * X[a * LD + c];
    if constexpr (ROWSCALE) acc *= CT(post[i]);
    out[static_cast<int64_t>(c) * D + i] = round_store<FDT>(static_cast<float>(acc), R, c, i);
  }
}

template <int FDT> using core_t = typename std::conditional<FDT == 0, double, float>::type;

template <int DK, int DV, int FDT, bool DIAG>
__global__ __launch_bounds__(256) void k_compress(const CompressArgs A) {
  using FT = stor_t<FDT>;
  using CT = core_t<FDT>;
  static_assert(2 * MX * LD >= MX * DK && 2 * MX * LD >= MX * DV, "staging fits LM + YM");
  extern __shared__ float4 lds4[];
  Core<CT>& S = *reinterpret_cast<Core<CT>*>(lds4);
  float* gam = reinterpret_cast<float*>(reinterpret_cast<char*>(lds4) + sizeof(Core<CT>));
  const int t = threadIdx.x;
  int64_t unit = blockIdx.x;
  if (A.list != nullptr) {   // list mode: the unit this block compresses (an index out of range: none)
    unit = A.list[blockIdx.x];
    if (unit < 0 || unit >= A.units) return;
  }
  const int r = A.rank, C = A.slots;
  float* __restrict__ sc = A.scale + unit * A.scale_len;
  int m = A.m;
  if (A.ragged) {
    // only the units whose own column count reached A.m (and holds columns beyond r); the
    // count is the same for every thread, so the whole block leaves together
    const int mu = static_cast<int>(__float_as_uint(sc[A.m_off]));
    if (mu < A.m || mu <= r || mu > C) return;
    m = mu;
  }
  FT* __restrict__ Ub = reinterpret_cast<FT*>(A.U) + unit * static_cast<int64_t>(C) * DK;
  FT* __restrict__ Vb = reinterpret_cast<FT*>(A.V) + unit * static_cast<int64_t>(C) * DV;
  // the unit's compression-window count (stochastic rounding's counter; one more at the end)
  const uint32_t window = __float_as_uint(sc[A.win_off]);
  const Rounding RU{A.rounding != 0, A.rng_key, kSiteCompressU, unit, window};
  const Rounding RV{A.rounding != 0, A.rng_key, kSiteCompressV, unit, window};

  // lazy decay: per-column scales (GDN, Mamba-2) or per-channel Gamma (KDA)
  if constexpr (DIAG) {
    for (int i = t; i < DK; i += 256) gam[i] = sc[i];
    if (t < MX) S.colsc[t] = CT(1);
  } else {
    if (t < MX) S.colsc[t] = (t < m) ? CT(sc[t < r ? 0 : 1 + t - r]) : CT(0);
  }
  __syncthreads();

  // the lazy sink folded into a: a = (slot-0 decay) a_0 + sum_{j >= r} c_j (true column j)
  // (KDA: Gamma . (a_0 + sum_j c_j U_j)); the window columns are not rewritten below. The
  // column reads go out 8 at a time, independent of one another.
  for (int d = t; d < DK; d += 256) {
    float acc = 0.f;
    for (int j0 = r; j0 < m; j0 += 8) {
      float u[8], cj[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = j0 + i < m ? j0 + i : m - 1;
        cj[i] = j0 + i < m ? sc[A.coef_off + j - r] * (DIAG ? 1.f : sc[1 + j - r]) : 0.f;
        u[i] = to_f32<FDT>(Ub[static_cast<int64_t>(j) * DK + d]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = fmaf(cj[i], u[i], acc);
    }
    A.a[unit * DK + d] = DIAG ? gam[d] * (A.a[unit * DK + d] + acc) : sc[0] * A.a[unit * DK + d] + acc;
  }

  // 1. Grams of the stored columns
  gram_rows<CT, CT, DK, FDT, DIAG ? 1 : 0>(S, Ub, m, gam, S.GA);
  gram_rows<CT, CT, DV, FDT, 0>(S, Vb, m, gam, S.GB);

  core_truncate(S, m, r);
  const int k = S.kk;

  // U' = Gamma . (U_s[:, perm] X_U): stage the k pivot columns, then write r columns
  for (int idx = t; idx < k * DK; idx += 256) {
    const int a = idx / DK, i = idx - a * DK;
    S.LM[a * DK + i] = CT(to_f32<FDT>(Ub[static_cast<int64_t>(S.perm[a]) * DK + i]));
  }
  __syncthreads();
  reconstruct_rows<CT, DK, FDT, DIAG>(S, S.GB, k, r, gam, Ub, RU);
  __syncthreads();
  // V' = V X_V
  for (int idx = t; idx < m * DV; idx += 256) {
    const int j = idx / DV, i = idx - j * DV;
    S.LM[j * DV + i] = CT(to_f32<FDT>(Vb[static_cast<int64_t>(j) * DV + i]));
  }
  __syncthreads();
  reconstruct_rows<CT, DV, FDT, false>(S, S.GA, m, r, nullptr, Vb, RV);
  // decay scales back to 1, sink coefficients to 0, the window count one up, m to r
  for (int i = t; i < A.scale_len; i += 256)
    sc[i] = i < A.coef_off ? 1.f
            : (i < A.win_off ? 0.f
                             : __uint_as_float(i == A.win_off ? window + 1u : static_cast<uint32_t>(r)));
}

template <int DK, int FDT>
constexpr size_t compress_lds_bytes() {
  return sizeof(Core<core_t<FDT>>) + DK * sizeof(float);
}

// ---- prefill-end compression ------------------------------------------------------------------
// Dense S (DK x DV, row i = key channel i). a = S vbar / |vbar|^2, C = S - a vbar^T. The
// content is put in factored form with m <= 64 columns, then the core truncates it exactly:
//   DV <= 64:       U = C, V = I_DV          (m = DV, exact)
//   DK <= 64 < DV:  U = I_DK, V = C^T        (m = DK, exact)
// Both read C back from the dense state for the reconstruction. 128 x 128 states go to
// k_from_dense_jacobi below.
template <int DK, int DV, int FDT>
struct FD {
  static constexpr bool UC = (DV <= 64);               // U = C, V = I
  static constexpr bool VC = (!UC && DK <= 64);        // U = I, V = C^T
  static_assert(UC || VC, "one side of at most 64");
  static constexpr int M = UC ? DV : DK;
  using CT = core_t<FDT>;
  static constexpr int LDC = DV + 1;                   // staged C rows
  static constexpr size_t CORE = sizeof(Core<CT>);
  static constexpr size_t CST = sizeof(float) * DK * LDC;
  static constexpr size_t BIG = ((CORE > CST ? CORE : CST) + 15) / 16 * 16;
  static constexpr size_t LDS = BIG + sizeof(float) * (DK + DV + 4);
};

template <int DK, int DV, int FDT>
__global__ __launch_bounds__(256) void k_from_dense(const CompressArgs A) {
  using FT = stor_t<FDT>;
  using L = FD<DK, DV, FDT>;
  using CT = typename L::CT;
  constexpr int M = L::M;
  extern __shared__ float4 lds4[];
  char* base = reinterpret_cast<char*>(lds4);
  Core<CT>& S = *reinterpret_cast<Core<CT>*>(base);
  float* Cst = reinterpret_cast<float*>(base);           // staged C rows (before the core)
  float* sa = reinterpret_cast<float*>(base + L::BIG);
  float* svb = sa + DK;
  float* misc = svb + DV;
  static_assert(DK <= 256 && DV <= 256, "one thread per row");

  const int t = threadIdx.x;
  const int64_t unit = blockIdx.x;
  const int head = static_cast<int>(unit % A.heads);
  const int r = A.rank, Cs = A.slots;
  const float* __restrict__ Sd = A.S + unit * DK * DV;
  FT* __restrict__ Ub = reinterpret_cast<FT*>(A.U) + unit * static_cast<int64_t>(Cs) * DK;
  FT* __restrict__ Vb = reinterpret_cast<FT*>(A.V) + unit * static_cast<int64_t>(Cs) * DV;

  // sink split: a = S vbar / |vbar|^2, C = S - a vbar^T staged in LDS
  for (int j = t; j < DV; j += 256) svb[j] = A.vbar[static_cast<int64_t>(head) * DV + j];
  __syncthreads();
  if (t < kWave) {
    float p = 0.f;
    for (int j = t; j < DV; j += kWave) p += svb[j] * svb[j];
    p = group_sum<64>(p);
    if (t == 0) misc[0] = p;
  }
  for (int idx = t; idx < DK * DV; idx += 256) {
    const int i = idx / DV, j = idx - i * DV;
    Cst[i * L::LDC + j] = Sd[idx];
  }
  __syncthreads();
  const float nn = misc[0];
  const float inv = nn > 0.f ? 1.f / nn : 0.f;
  if (t < DK) {
    float p = 0.f;
    for (int j = 0; j < DV; ++j) p += Cst[t * L::LDC + j] * svb[j];
    const float ai = p * inv;
    sa[t] = ai;
    A.a[unit * DK + t] = ai;
  }
  __syncthreads();
  for (int idx = t; idx < DK * DV; idx += 256) {
    const int i = idx / DV, j = idx - i * DV;
    Cst[i * L::LDC + j] -= sa[i] * svb[j];
  }
  __syncthreads();

  // Grams of the factored content, accumulated in registers, then written to the core
  // region once every thread is done with the staged C
  {
    using AccT = typename std::conditional<std::is_same<CT, double>::value, double, float>::type;
    const int ta = t >> 4, tb = t & 15;
    AccT au[4][4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int f = 0; f < 4; ++f) au[e][f] = AccT(0);
    // the non-identity Gram: U^T U (UC: C^T C over rows i) or V^T V (VC: C C^T)
    if (4 * ta < M && 4 * tb < M) {
      if constexpr (L::UC) {
        for (int i = 0; i < DK; ++i) {
          AccT x[4], y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[e] = (4 * ta + e < M) ? AccT(Cst[i * L::LDC + 4 * ta + e]) : AccT(0);
            y[e] = (4 * tb + e < M) ? AccT(Cst[i * L::LDC + 4 * tb + e]) : AccT(0);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int f = 0; f < 4; ++f) au[e][f] += x[e] * y[f];
        }
      } else if constexpr (L::VC) {
        for (int j = 0; j < DV; ++j) {
          AccT x[4], y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[e] = (4 * ta + e < M) ? AccT(Cst[(4 * ta + e) * L::LDC + j]) : AccT(0);
            y[e] = (4 * tb + e < M) ? AccT(Cst[(4 * tb + e) * L::LDC + j]) : AccT(0);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int f = 0; f < 4; ++f) au[e][f] += x[e] * y[f];
        }
      }
    }
    __syncthreads();  // the staged C is dead from here on: the core overwrites it
    if (4 * ta < M && 4 * tb < M) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int a = 4 * ta + e, b = 4 * tb + f;
          if (a < M && b < M) {
            const CT g = CT(au[e][f]);
            const CT id = (a == b) ? CT(1) : CT(0);
            if constexpr (L::VC) { S.GA[a * LD + b] = id; S.GB[a * LD + b] = g; }
            else { S.GA[a * LD + b] = g; S.GB[a * LD + b] = id; }
          }
        }
    }
    if (t < MX) S.colsc[t] = CT(1);
    __syncthreads();
  }

  core_truncate(S, M, r);
  const int k = S.kk;
  // the first window (count 0)
  const Rounding RU{A.rounding != 0, A.rng_key, kSiteFromDenseU, unit, 0u};
  const Rounding RV{A.rounding != 0, A.rng_key, kSiteFromDenseV, unit, 0u};

  if constexpr (L::UC) {
    // U'[c][i] = sum_a C[i][perm[a]] X_U[a][c]; V'[c][j] = X_V[j][c]
    for (int c = t / DK; c < r; c += 256 / DK) {
      const int i = t % DK;
      const float ai = sa[i];
      CT acc = CT(0);
      for (int a = 0; a < k; ++a) {
        const int j = S.perm[a];
        acc += CT(Sd[i * DV + j] - ai * svb[j]) * S.GB[a * LD + c];
      }
      Ub[static_cast<int64_t>(c) * DK + i] = round_store<FDT>(static_cast<float>(acc), RU, c, i);
    }
    for (int c = t / DV; c < r; c += 256 / DV) {
      const int j = t % DV;
      Vb[static_cast<int64_t>(c) * DV + j] = round_store<FDT>(static_cast<float>(S.GA[j * LD + c]), RV, c, j);
    }
  } else if constexpr (L::VC) {
    // U'[c][perm[a]] = X_U[a][c] (zero on non-pivot rows); V'[c][j] = sum_i C[i][j] X_V[i][c]
    for (int c = t / DK; c < r; c += 256 / DK) {
      const int i = t % DK;
      CT val = CT(0);
      for (int a = 0; a < k; ++a)
        if (S.perm[a] == i) val = S.GB[a * LD + c];
      Ub[static_cast<int64_t>(c) * DK + i] = round_store<FDT>(static_cast<float>(val), RU, c, i);
    }
    for (int c = t / DV; c < r; c += 256 / DV) {
      const int j = t % DV;
      CT acc = CT(0);
      for (int i = 0; i < DK; ++i) acc += CT(Sd[i * DV + j] - sa[i] * svb[j]) * S.GA[i * LD + c];
      Vb[static_cast<int64_t>(c) * DV + j] = round_store<FDT>(static_cast<float>(acc), RV, c, j);
    }
  }
  // decay scales 1, sink coefficients 0, window count 0, m = r
  float* __restrict__ sc = A.scale + unit * A.scale_len;
  for (int i = t; i < A.scale_len; i += 256)
    sc[i] = i < A.coef_off ? 1.f : (i == A.m_off ? __uint_as_float(static_cast<uint32_t>(r)) : 0.f);
}


// ---- prefill-end compression of 128 x 128 states: one-sided Jacobi SVD of the content ----------
// The content C = S - a vbar^T (a as stored) is held in LDS in fp64 as its 128 columns w_j, one
// per value channel. Sweeps of plane rotations over all column pairs orthogonalise them: with the
// accumulated rotation J, C J = W, so C = sum_c w_c j_c^T with orthogonal w_c, and sigma_c =
// |w_c| are the singular values. A sweep is 127 rounds of 64 disjoint pairs (the circle method:
// position 127 stays, the others turn). A pair with a = |w_p|^2, b = |w_q|^2, g = w_p . w_q is
// rotated while |g| > kJacobiTol sqrt(a b), by the angle that makes the two columns orthogonal;
// columns below the noise floor (1e-28 of the content's energy) are left alone. The iteration stops
// at the first sweep that rotates no pair, or after kJacobiMaxSweeps. The r longest columns give
// U'_k = w_c / sqrt(sigma_c), and V'_k = j_c sqrt(sigma_c) = C^T w_c / sigma_c^(3/2) is formed from
// the dense state itself, so J is never stored. There is no Gram (whose condition number is the
// square of C's), no iteration count to guess, and the truncation is exact up to the stopping
// tolerance and fp64 rounding.
template <int FDT>
struct FDJ {
  static constexpr int D = 128;
  static constexpr int LDW = D + 1;
  static constexpr size_t LDS = sizeof(double) * (D * LDW + D + 8) + sizeof(float) * (2 * D + 4) +
                                sizeof(int) * 64;
};

__device__ __forceinline__ double quad_sum_d(double v) {
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  return v;
}

template <int FDT>
__global__ __launch_bounds__(256) void k_from_dense_jacobi(const CompressArgs A) {
  using FT = stor_t<FDT>;
  constexpr int D = FDJ<FDT>::D;
  constexpr int LDW = FDJ<FDT>::LDW;
  extern __shared__ float4 lds4[];
  double* W = reinterpret_cast<double*>(lds4);   // column c at W + c * LDW
  double* sig = W + D * LDW;                      // [D] column lengths
  double* red = sig + D;                          // [8] reduction scratch
  float* sa = reinterpret_cast<float*>(red + 8);  // [D] the sink a
  float* svb = sa + D;                            // [D] vbar
  float* misc = svb + D;                          // [4]
  int* sel = reinterpret_cast<int*>(misc + 4);    // [64] the kept columns, longest first

  const int t = threadIdx.x;
  const int64_t unit = blockIdx.x;
  const int head = static_cast<int>(unit % A.heads);
  const int r = A.rank, Cs = A.slots;
  const float* __restrict__ Sd = A.S + unit * D * D;
  FT* __restrict__ Ub = reinterpret_cast<FT*>(A.U) + unit * static_cast<int64_t>(Cs) * D;
  FT* __restrict__ Vb = reinterpret_cast<FT*>(A.V) + unit * static_cast<int64_t>(Cs) * D;

  // sink split: a = S vbar / |vbar|^2 (stored in fp32), C = S - a vbar^T
  for (int j = t; j < D; j += 256) svb[j] = A.vbar[static_cast<int64_t>(head) * D + j];
  __syncthreads();
  if (t < kWave) {
    float p = 0.f;
    for (int j = t; j < D; j += kWave) p += svb[j] * svb[j];
    p = group_sum<64>(p);
    if (t == 0) misc[0] = p;
  }
  __syncthreads();
  const float inv = misc[0] > 0.f ? 1.f / misc[0] : 0.f;
  if (t < D) {
    float p = 0.f;
    for (int j = 0; j < D; ++j) p += Sd[t * D + j] * svb[j];
    const float ai = p * inv;
    sa[t] = ai;
    A.a[unit * D + t] = ai;
  }
  __syncthreads();
  double e = 0.0;
  for (int idx = t; idx < D * D; idx += 256) {
    const int i = idx / D, j = idx - i * D;
    const double c = static_cast<double>(Sd[idx]) - static_cast<double>(sa[i]) * static_cast<double>(svb[j]);
    W[j * LDW + i] = c;
    e += c * c;
  }
  for (int off = 32; off > 0; off >>= 1) e += __shfl_xor(e, off);
  if ((t & (kWave - 1)) == 0) red[t >> 6] = e;
  __syncthreads();
  const double floor = 1e-28 * (red[0] + red[1] + red[2] + red[3]);

  // sweeps; the 4 lanes of a pair hold rows part + 4 k of its two columns
  const int pr = t >> 2, part = t & 3;
  for (int sweep = 0; sweep < kJacobiMaxSweeps; ++sweep) {
    int rot = 0;
    for (int k = 0; k < D - 1; ++k) {
      const int p = pr == 0 ? D - 1 : (k + pr) % (D - 1);
      const int q = pr == 0 ? k : (k - pr + (D - 1)) % (D - 1);
      double* wp = W + p * LDW + part;
      double* wq = W + q * LDW + part;
      double x[D / 4], y[D / 4];
      double a = 0.0, b = 0.0, g = 0.0;
#pragma unroll
      for (int i = 0; i < D / 4; ++i) {
        x[i] = wp[4 * i];
        y[i] = wq[4 * i];
        a = fma(x[i], x[i], a);
        b = fma(y[i], y[i], b);
        g = fma(x[i], y[i], g);
      }
      a = quad_sum_d(a);
      b = quad_sum_d(b);
      g = quad_sum_d(g);
      // the four lanes of a pair hold the same sums, so they take the same branch
      if (a > floor && b > floor && fabs(g) > kJacobiTol * sqrt(a) * sqrt(b)) {
        const double zeta = (b - a) / (2.0 * g);
        const double tn = (zeta >= 0.0 ? 1.0 : -1.0) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
        const double c = 1.0 / sqrt(1.0 + tn * tn), s = c * tn;
#pragma unroll
        for (int i = 0; i < D / 4; ++i) {
          wp[4 * i] = c * x[i] - s * y[i];
          wq[4 * i] = s * x[i] + c * y[i];
        }
        rot = 1;
      }
      __syncthreads();
    }
    if (!__syncthreads_or(rot)) break;
  }

  // singular values and the r longest columns
  if (t < D) {
    double n2 = 0.0;
    for (int i = 0; i < D; ++i) n2 = fma(W[t * LDW + i], W[t * LDW + i], n2);
    sig[t] = sqrt(n2);
  }
  __syncthreads();
  if (t < D) {
    const double st = sig[t];
    int rank = 0;
    for (int c = 0; c < D; ++c) rank += (sig[c] > st) || (sig[c] == st && c < t);
    if (rank < r) sel[rank] = t;
  }
  __syncthreads();
  const double smax = sig[sel[0]];
  const double sfloor = 1e-13 * smax;
  const Rounding RU{A.rounding != 0, A.rng_key, kSiteFromDenseU, unit, 0u};
  const Rounding RV{A.rounding != 0, A.rng_key, kSiteFromDenseV, unit, 0u};
  // U'_k = w_c / sqrt(sigma_c) (zero past the content's rank)
  for (int idx = t; idx < r * D; idx += 256) {
    const int kk = idx / D, i = idx - kk * D;
    const int c = sel[kk];
    const double sc = sig[c];
    const double v = sc > sfloor ? W[c * LDW + i] / sqrt(sc) : 0.0;
    Ub[static_cast<int64_t>(kk) * D + i] = round_store<FDT>(static_cast<float>(v), RU, kk, i);
  }
  // V'_k = C^T w_c / sigma_c^(3/2): thread j (value channel) of half h takes k = h, h + 2, ...
  {
    const int j = t & (D - 1), h = t >> 7;
    double acc[32];
#pragma unroll
    for (int q = 0; q < 32; ++q) acc[q] = 0.0;
    const double vj = static_cast<double>(svb[j]);
    for (int i = 0; i < D; ++i) {
      const double cij = static_cast<double>(Sd[i * D + j]) - static_cast<double>(sa[i]) * vj;
#pragma unroll
      for (int q = 0; q < 32; ++q) {
        const int kk = h + 2 * q;
        if (kk < r) acc[q] = fma(cij, W[sel[kk] * LDW + i], acc[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      const int kk = h + 2 * q;
      if (kk < r) {
        const double sc = sig[sel[kk]];
        const double v = sc > sfloor ? acc[q] / (sc * sqrt(sc)) : 0.0;
        Vb[static_cast<int64_t>(kk) * D + j] = round_store<FDT>(static_cast<float>(v), RV, kk, j);
      }
    }
  }
  // decay scales 1, sink coefficients 0, window count 0, m = r
  float* __restrict__ sc = A.scale + unit * A.scale_len;
  for (int i = t; i < A.scale_len; i += 256)
    sc[i] = i < A.coef_off ? 1.f : (i == A.m_off ? __uint_as_float(static_cast<uint32_t>(r)) : 0.f);
}

// ---- host dispatch ---------------------------------------------------------------------------
namespace {
using KFn = void (*)(const CompressArgs);

template <int DK, int DV>
KFn pick_c(int dt, bool diag, size_t* lds) {
  if (dt == SEED_BF16) {
    *lds = compress_lds_bytes<DK, 1>();
    return diag ? k_compress<DK, DV, 1, true> : k_compress<DK, DV, 1, false>;
  }
  if (dt == SEED_F16) {
    *lds = compress_lds_bytes<DK, 2>();
    return diag ? k_compress<DK, DV, 2, true> : k_compress<DK, DV, 2, false>;
  }
  *lds = compress_lds_bytes<DK, 0>();
  return diag ? k_compress<DK, DV, 0, true> : k_compress<DK, DV, 0, false>;
}
KFn pick_compress(const seed_shape& sh, size_t* lds) {
  const bool diag = sh.kind == SEED_KDA;
  if (sh.rank + sh.period > MX) return nullptr;
  if (sh.d_k == 128 && sh.d_v == 128) return pick_c<128, 128>(sh.factor_dtype, diag, lds);
  if (sh.d_k == 128 && sh.d_v == 64) return pick_c<128, 64>(sh.factor_dtype, diag, lds);
  if (sh.d_k == 64 && sh.d_v == 128) return pick_c<64, 128>(sh.factor_dtype, diag, lds);
  if (sh.d_k == 64 && sh.d_v == 64) return pick_c<64, 64>(sh.factor_dtype, diag, lds);
  return nullptr;
}

template <int DK, int DV>
KFn pick_f(int dt, size_t* lds) {
  if (dt == SEED_BF16) { *lds = FD<DK, DV, 1>::LDS; return k_from_dense<DK, DV, 1>; }
  if (dt == SEED_F16) { *lds = FD<DK, DV, 2>::LDS; return k_from_dense<DK, DV, 2>; }
  *lds = FD<DK, DV, 0>::LDS;
  return k_from_dense<DK, DV, 0>;
}
KFn pick_from_dense(const seed_shape& sh, size_t* lds) {
  if (sh.d_k == 128 && sh.d_v == 128) {
    if (sh.factor_dtype == SEED_BF16) { *lds = FDJ<1>::LDS; return k_from_dense_jacobi<1>; }
    if (sh.factor_dtype == SEED_F16) { *lds = FDJ<2>::LDS; return k_from_dense_jacobi<2>; }
    *lds = FDJ<0>::LDS;
    return k_from_dense_jacobi<0>;
  }
  if (sh.d_k == 128 && sh.d_v == 64) return pick_f<128, 64>(sh.factor_dtype, lds);
  if (sh.d_k == 64 && sh.d_v == 128) return pick_f<64, 128>(sh.factor_dtype, lds);
  if (sh.d_k == 64 && sh.d_v == 64) return pick_f<64, 64>(sh.factor_dtype, lds);
  return nullptr;
}

// The dynamic-LDS limit of a kernel that takes more than 64 KB is set before each of its
// launches (a host-side attribute of the kernel on the current device: no stream work, and no
// state kept by the library).
hipError_t raise_lds_limit(KFn fn, size_t lds) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(lds));
}

hipError_t launch_big_lds(KFn fn, size_t lds, int64_t units, const CompressArgs& a, hipStream_t s) {
  hipError_t e = raise_lds_limit(fn, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(units)), dim3(256), lds, s, a);
  return hipGetLastError();
}
}  // namespace

static_assert(FD<128, 64, 0>::LDS <= 160 * 1024 && FD<64, 128, 0>::LDS <= 160 * 1024 &&
              FD<64, 64, 0>::LDS <= 160 * 1024 && FDJ<0>::LDS <= 160 * 1024, "from_dense LDS budget");
static_assert(compress_lds_bytes<128, 0>() <= 160 * 1024, "compress LDS budget");

bool compress_supported(const seed_shape& sh) {
  size_t lds = 0;
  return pick_compress(sh, &lds) != nullptr;
}

hipError_t launch_compress(const seed_shape& sh, const CompressArgs& a, hipStream_t s) {
  bool used = false;
  hipError_t te = launch_compress_wave(sh, a, s, &used);  // bf16 factors, r <= 32
  if (used) return te;
  size_t lds = 0;
  KFn fn = pick_compress(sh, &lds);
  if (!fn) return hipErrorInvalidValue;
  return launch_big_lds(fn, lds, compress_blocks(a), a, s);
}

hipError_t launch_from_dense(const seed_shape& sh, const CompressArgs& a, hipStream_t s) {
  size_t lds = 0;
  KFn fn = pick_from_dense(sh, &lds);
  if (!fn) return hipErrorInvalidValue;
  return launch_big_lds(fn, lds, a.units, a, s);
}

int32_t from_dense_iterations() { return kJacobiMaxSweeps; }

}  // namespace seed
