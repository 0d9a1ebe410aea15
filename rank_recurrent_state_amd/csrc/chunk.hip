// Chunked factored update: L consecutive tokens of every unit in one call. It gives each
// token's read-out and leaves the state that L decode steps would leave (equal in exact
// arithmetic; the rounding order differs).
//
// Method: pages titled "Shallow Encoding Emits Deep Memories", picx.dev summary, "Exact Update
// (Lemma 2)" (one token: a+ = g a + beta (omega - g kappa^T a) kappa, U+ = [g U, kappa],
// V+ = [V, beta (eps - g V U^T kappa)]) and "Theoretical and Practical Implications", Lemma 1
// (the sink coefficient and the content each follow the head's own recurrence). The pages give
// the one-token form; unrolled over a chunk of L tokens t = 0 .. L-1 it reads
//   Gamma(t, s) = prod_{s < u <= t} g_u (Gamma(t, t) = 1), gamma_t = Gamma(t, -1);
//   S_t = gamma_t S_0 + sum_{s <= t} Gamma(t, s) kappa_s delta_s^T, delta_s = c_s vbar + w_s;
//   (I + A) c = beta (omega - gamma a~ . kappa),  (I + A) W = beta (eps - gamma V (U~^T kappa)),
//   A[t][s] = beta_t Gamma(t, s) kappa_t . kappa_s for s < t (Mamba-2: A = 0 and no state term);
//   o_t = vbar (gamma_t a~ . q_t + sum_{s <= t} Gamma(t, s) (q_t . kappa_s) c_s)
//         + gamma_t V (U~^T q_t) + sum_{s <= t} Gamma(t, s) (q_t . kappa_s) w_s,
// with a~ and U~ the true (decayed) sink and columns at the start of the chunk. c_s and w_s are
// the sink coefficient and V column that decode step s produces, so the chunk appends exactly
// the columns of L steps: kappa_s to U with lazy decay scale Gamma(L-1, s), w_s to V, and c_s
// to the sink coefficients; the decay scales held before the chunk take gamma_{L-1}.
//
// Design (gfx950): one 256-thread workgroup per unit; the scalar-decay kinds (GDN, Mamba-2).
// The token count is padded to LM = 16 or 32 (a compiled width): the padding tokens have zero
// inputs, so every loop runs to LM without a test, and only the stores look at L.
//   staging      keys and queries of the chunk in LDS (bf16 as given for bf16 inputs, else
//                fp32; rows padded by 16 bytes, so that the pair products below read rows t and
//                s without bank conflicts); they share their LDS with the residuals W, which
//                are written only after their last read;
//   U pass       U~^T kappa and U~^T q by MFMA 32x32x2 (fp32): one 32-column, 32-token tile
//                per wave; each lane's row of U is loaded at the start of the kernel (its
//                latency overlaps the staging), the key and query rows come from LDS;
//   pair terms   kappa_t . kappa_s and q_t . kappa_s over the lower triangle, and the decay
//                products Gamma(t, s) by running products;
//   V pass       thread d of the first half owns value channel d: V (U~^T kappa) in registers,
//                then the forward substitution for W (every thread its own channel, no
//                exchange) and, alongside, for the scalar c (the same matrix); thread d of the
//                second half forms V (U~^T q);
//   read-out     the second half combines its V (U~^T q) with the residuals w_s + c_s vbar
//                from LDS.
// U and V are each read once; the chunk's keys become the new U columns unchanged (rounded to
// the factor format), its W the new V columns.
#include "common.hpp"
#include "kernels.hpp"

namespace seed {

namespace {

constexpr int kChunkMax = 32;      // tokens per call
constexpr int kChunkMaxDiag = 16;  // tokens per call, KDA
constexpr int kColsMax = 64;   // column slots per unit

// The chunk's keys and queries in LDS: as given (bf16) when the inputs are bf16, so that a
// 32-token chunk leaves room for three workgroups per CU; fp32 for fp32 inputs and for KDA,
// whose decayed copies are formed from them. Rows are padded by 16 bytes.
template <int IDT, bool DIAG> struct KqStore { using T = float; static constexpr int PAD = 4; };
template <> struct KqStore<1, false> { using T = uint16_t; static constexpr int PAD = 8; };

__device__ __forceinline__ float kqf(float x) { return x; }
__device__ __forceinline__ float kqf(uint16_t x) { return bf16_to_f32(x); }

// four consecutive elements of a key or query row as fp32
__device__ __forceinline__ float4 kq4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 kq4(const uint16_t* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
                     __uint_as_float(w.y & 0xffff0000u));
}

template <int DK, int DV, int LM, bool DIAG, int IDT>
struct ChunkSmem {
  using KQ = typename KqStore<IDT, DIAG>::T;
  static constexpr int KP = KqStore<IDT, DIAG>::PAD;
  union {
    struct {
      alignas(16) KQ K[LM][DK + KP];  // the chunk's keys and queries (until the pair terms are done)
      alignas(16) KQ Q[LM][DK + KP];
    } kq;
    alignas(16) float W[LM][DV];      // then the chunk's residuals delta_t = w_t + c_t vbar
  };
  alignas(16) float PK[kColsMax][LM];  // U~^T kappa_t (row j: column j of U)
  alignas(16) float PQ[kColsMax][LM];  // U~^T q_t
  float Gm[DIAG ? 1 : LM][LM + 1];     // Gm[t][s + 1] = Gamma(t, s), s = -1 .. t (scalar decay)
  float Akk[LM][LM + 1];               // A[t][s] = beta_t Gamma(t, s) kappa_t . kappa_s, s < t
  float Aqk[LM][LM + 1];               // Gamma(t, s) q_t . kappa_s, s <= t
  float vb[DV];
  float a0[DK];
  float g[LM], beta[LM], omega[LM], aK[LM], aQ[LM], c[LM];
  // KDA only: the gates, and each token's decay from the state held before the chunk through
  // the state's own channel scales, Gamma P_t (the decayed keys and queries are this times the
  // keys and queries)
  float Al[DIAG ? LM : 1][DIAG ? DK : 1];
  float Pg[DIAG ? LM : 1][DIAG ? DK + 1 : 1];
};

// KDA: a channel whose scale would fall below this is folded into the stored columns (as in the
// decode step), so that a new column k / scale stays finite in the factor format
template <int FDT> constexpr float kChunkFoldFloor = 0x1p-40f;
template <> constexpr float kChunkFoldFloor<2> = 0x1p-12f;

}  // namespace

template <int DK, int DV, bool DELTA, bool DIAG, int FDT, int IDT, int LM>
__global__ __launch_bounds__(256) void k_decode_chunk(const StepArgs A) {
  static_assert(DV <= 128 && DK <= 128 && LM % 4 == 0 && LM <= kChunkMax, "shapes");
  static_assert(!DIAG || DELTA, "the diagonal gate comes with the delta rule (KDA)");
  using FT = stor_t<FDT>;
  using IT = stor_t<IDT>;
  __shared__ ChunkSmem<DK, DV, LM, DIAG, IDT> S;
  using KQ = typename ChunkSmem<DK, DV, LM, DIAG, IDT>::KQ;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int64_t unit = blockIdx.x;
  const int H = A.heads;
  const int64_t bq = unit / H;
  const int hd = static_cast<int>(unit - bq * H);
  const int L = A.len, r = A.rank, C = A.slots;
  float* __restrict__ sc = A.scale + unit * A.scale_len;
  int m = A.m;
  if (A.ragged) {
    // every unit from its own column count; units masked out, or without room for the chunk,
    // are left untouched (their rows of o are not written)
    m = static_cast<int>(__float_as_uint(sc[A.m_off]));
    if ((A.active != nullptr && A.active[unit] == 0) || m < r || m + L > C) return;
  }
  FT* __restrict__ Ub = reinterpret_cast<FT*>(A.U) + unit * static_cast<int64_t>(C) * DK;
  FT* __restrict__ Vb = reinterpret_cast<FT*>(A.V) + unit * static_cast<int64_t>(C) * DV;
  // row of token t in the [batch][L][heads] layout of the chunk's inputs and outputs
  auto tok = [&](int t) { return (bq * L + t) * H + hd; };
  // factor stores: nearest, or stochastic with the draws the decode steps would take for the
  // same columns (site, slot, unit, compression window, element)
  const bool sr = FDT != 0 && A.rounding != 0;
  const uint32_t window = sr ? __float_as_uint(sc[A.win_off]) : 0u;
  auto put = [&](FT* dst, float x, uint32_t site, uint32_t aux, int slot, int elem) {
    if constexpr (FDT != 0) {
      if (sr) {
        const uint4 dr = sr_group(A.rng_key, site, aux, slot, unit, window, elem);
        *dst = round_sr<FDT>(x, draw16(dr, elem & 7));
        return;
      }
    }
    *dst = from_f32<FDT>(x);
  };

  // ---- the U pass's column loads go out first: their latency overlaps the staging -------------
  // Wave wv takes column block jt = wv % 2; lane (c, h) loads row 32 jt + c of U: the whole row
  // for 16-bit factors, its first half for fp32 factors (the second half follows later).
  const int ujt = wv & 1;
  const int uj = 32 * ujt + (lane & 31);
  const bool ujok = uj < m;
  const uint4* __restrict__ urow = reinterpret_cast<const uint4*>(Ub + static_cast<int64_t>(ujok ? uj : 0) * DK);
  constexpr int UW = DK / 8;   // 16-byte words held: DK 16-bit elements, or DK / 2 fp32 ones
  uint4 uraw[UW];
  if (32 * ujt < m) {  // uniform
#pragma unroll
    for (int i = 0; i < UW; ++i) uraw[i] = urow[i];
  }

  // ---- staging (padding tokens: zero inputs, zero pair terms) ---------------------------------
  for (int i = tid; i < LM * (DK / 4); i += 256) {
    const int t = i / (DK / 4), d = 4 * (i - t * (DK / 4));
    if constexpr (sizeof(KQ) == 2) {
      // the inputs' bf16 bits as they are
      uint2 x = make_uint2(0u, 0u), y = make_uint2(0u, 0u);
      if (t < L) {
        x = *reinterpret_cast<const uint2*>(reinterpret_cast<const IT*>(A.k) + tok(t) * DK + d);
        y = *reinterpret_cast<const uint2*>(reinterpret_cast<const IT*>(A.q) + tok(t) * DK + d);
      }
      *reinterpret_cast<uint2*>(&S.kq.K[t][d]) = x;
      *reinterpret_cast<uint2*>(&S.kq.Q[t][d]) = y;
    } else {
      float x[4] = {0.f, 0.f, 0.f, 0.f}, y[4] = {0.f, 0.f, 0.f, 0.f};
      if (t < L) {
        load_f32<IDT, 4>(reinterpret_cast<const IT*>(A.k) + tok(t) * DK + d, x);
        load_f32<IDT, 4>(reinterpret_cast<const IT*>(A.q) + tok(t) * DK + d, y);
      }
      *reinterpret_cast<float4*>(&S.kq.K[t][d]) = make_float4(x[0], x[1], x[2], x[3]);
      *reinterpret_cast<float4*>(&S.kq.Q[t][d]) = make_float4(y[0], y[1], y[2], y[3]);
    }
  }
  for (int i = tid; i < kColsMax * LM; i += 256) {
    (&S.PK[0][0])[i] = 0.f;
    (&S.PQ[0][0])[i] = 0.f;
  }
  for (int i = tid; i < LM * (LM + 1); i += 256) {
    (&S.Akk[0][0])[i] = 0.f;
    (&S.Aqk[0][0])[i] = 0.f;
    if constexpr (!DIAG) (&S.Gm[0][0])[i] = 0.f;
  }
  for (int i = tid; i < DV; i += 256) S.vb[i] = A.vbar[static_cast<int64_t>(hd) * DV + i];
  for (int i = tid; i < DK; i += 256) S.a0[i] = A.a[unit * DK + i];
  if constexpr (DIAG) {
    // the gates, one per key channel ([batch][L][heads][d_k]); padding tokens keep 1
    for (int i = tid; i < LM * DK; i += 256) {
      const int t = i / DK, dd = i - t * DK;
      S.Al[t][dd] = t < L ? A.g[tok(t) * DK + dd] : 1.f;
    }
  }
  if (tid < LM) {
    S.g[tid] = (!DIAG && tid < L) ? A.g[tok(tid)] : 0.f;
    S.beta[tid] = tid < L ? A.beta[tok(tid)] : 0.f;
    S.omega[tid] = 0.f;
    S.aK[tid] = 0.f;
    S.aQ[tid] = 0.f;
  }
  __syncthreads();

  // ---- decay products, the new U columns, U~^T kappa and U~^T q, the value split ----------------
  if constexpr (DIAG) {
    // channel d: Gamma P_t with P_t = prod_{u <= t} alpha_u (running), the decay of the
    // terms of the state held before the chunk
    for (int dd = tid; dd < DK; dd += 256) {
      float p = sc[dd];
      for (int t = 0; t < LM; ++t) {
        p *= S.Al[t][dd];
        S.Pg[t][dd] = p;
      }
    }
    __syncthreads();
  } else {
    if (tid < L) {
      const int t = tid;
      float p = 1.f;
      S.Gm[t][t + 1] = 1.f;
      for (int s = t - 1; s >= -1; --s) {
        p *= S.g[s + 1];
        S.Gm[t][s + 1] = p;
      }
    }
    for (int i = tid; i < L * (DK / 4); i += 256) {
      const int t = i / (DK / 4), d = 4 * (i - t * (DK / 4));
      const float4 x4 = kq4(&S.kq.K[t][d]);
      const float x[4] = {x4.x, x4.y, x4.z, x4.w};
      if (sr) {
#pragma unroll
        for (int e = 0; e < 4; ++e) put(Ub + static_cast<int64_t>(m + t) * DK + d + e, x[e], kSiteDecodeU, 0u, m + t, d + e);
      } else {
        store_f32<FDT, 4>(Ub + static_cast<int64_t>(m + t) * DK + d, x);
      }
    }
  }
  // the keys and queries the U pass uses: as given (the slot scales apply per column), or KDA's
  // decayed ones, Gamma P_t kappa_t and Gamma P_t q_t
  auto kval = [&](int t, int d) {
    if constexpr (DIAG) return S.Pg[t][d] * kqf(S.kq.K[t][d]);
    else return kqf(S.kq.K[t][d]);
  };
  auto qval = [&](int t, int d) {
    if constexpr (DIAG) return S.Pg[t][d] * kqf(S.kq.Q[t][d]);
    else return kqf(S.kq.Q[t][d]);
  };
  {
    // U pass by MFMA 32x32x2 (fp32): wave wv forms the 32 x 32 tile of column block jt = wv % 2
    // and keys (wv < 2) or queries of (U^T K)[j][t] = sum_d U[j][d] K[t][d]. Lane (c, h) feeds
    // A = U[32 jt + c][d] and B = K[c][d] for d = 2 s + h: its column's elements from the
    // words loaded above, its key row's from LDS; tokens past L and columns past m are zero.
    typedef float f32x16 __attribute__((ext_vector_type(16)));
    const bool isq = wv >= 2;
    if (32 * ujt < m) {  // uniform
      const int c = lane & 31, h = lane >> 5;
      const bool cok = c < LM;
      uint4 uraw2[FDT == 0 ? UW : 1];   // fp32 factors: the row's second half
      if constexpr (FDT == 0) {
#pragma unroll
        for (int i = 0; i < UW; ++i) uraw2[i] = urow[UW + i];
      }
      auto word = [](const uint4& q, int k) { return k == 0 ? q.x : (k == 1 ? q.y : (k == 2 ? q.z : q.w)); };
      f32x16 acc;
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
      for (int d8 = 0; d8 < DK; d8 += 8) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float av;
          if constexpr (FDT == 0) {
            const int i = d8 + 2 * e;                          // even: i and i + 1 share a word
            const uint4& q = i < DK / 2 ? uraw[i / 4] : uraw2[(i - DK / 2) / 4];
            av = __uint_as_float(h ? word(q, i % 4 + 1) : word(q, i % 4));
          } else {
            const uint32_t w = word(uraw[d8 / 8], e);
            av = h ? hi16<FDT>(w) : lo16<FDT>(w);
          }
          av = ujok ? av : 0.f;
          const float bv = cok ? (isq ? qval(c, d8 + 2 * e + h) : kval(c, d8 + 2 * e + h)) : 0.f;
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
        }
      }
      // acc[v] is the tile's entry (row 8 (v / 4) + 4 h + v % 4, column c): column j of U,
      // token c
      if (c < LM) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int jj = 32 * ujt + 8 * (v >> 2) + 4 * h + (v & 3);
          if (jj < m) {
            // true columns: slot 0 scales the r columns kept by the last compression, slot 1 + i
            // window column r + i (KDA: the channel scales are in the keys)
            const float sj = DIAG ? 1.f : sc[jj < r ? 0 : 1 + jj - r];
            if (isq) S.PQ[jj][c] = sj * acc[v];
            else S.PK[jj][c] = sj * acc[v];
          }
        }
      }
    }
  }
  {
    // omega_t = v_t . vbar / |vbar|^2 (wave wv: tokens wv, wv + 4, ...)
    constexpr int NB = DV / 64;
    float nn = 0.f;
#pragma unroll
    for (int e = 0; e < NB; ++e) nn += S.vb[NB * lane + e] * S.vb[NB * lane + e];
    nn = wave_sum(nn);
    // every token's values first (the loads in flight together), then the sums
    float vv[LM / 4][NB];
#pragma unroll
    for (int i = 0; i < LM / 4; ++i) {
      const int t = wv + 4 * i;
      load_f32<IDT, NB>(reinterpret_cast<const IT*>(A.v) + tok(t < L ? t : L - 1) * DV + NB * lane, vv[i]);
    }
#pragma unroll
    for (int i = 0; i < LM / 4; ++i) {
      const int t = wv + 4 * i;
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < NB; ++e) p += vv[i][e] * S.vb[NB * lane + e];
      p = wave_sum(p);
      if (lane == 0 && t < L) S.omega[t] = nn > 0.f ? p / nn : 0.f;
    }
  }
  __syncthreads();

  // ---- pair terms; the sink's share a~ . kappa_t and a~ . q_t ----------------------------------
  if constexpr (DIAG) {
    // Gamma(t, s) is a vector here: wave wv takes s = wv, wv + 4, ..., runs t up from s with
    // the running product of the gates per channel (lanes over channels) and sums over them
    constexpr int NA = DK / 64;
    for (int s = wv; s < L; s += 4) {
      float G[NA], ks[NA];
#pragma unroll
      for (int e = 0; e < NA; ++e) {
        G[e] = 1.f;
        ks[e] = kqf(S.kq.K[s][NA * lane + e]);
      }
      for (int t = s; t < L; ++t) {
        float kk = 0.f, qk = 0.f;
#pragma unroll
        for (int e = 0; e < NA; ++e) {
          if (t > s) G[e] *= S.Al[t][NA * lane + e];
          const float gk = G[e] * ks[e];
          kk = fmaf(kqf(S.kq.K[t][NA * lane + e]), gk, kk);
          qk = fmaf(kqf(S.kq.Q[t][NA * lane + e]), gk, qk);
        }
        kk = wave_sum(kk);
        qk = wave_sum(qk);
        if (lane == 0) {
          S.Akk[t][s] = s < t ? S.beta[t] * kk : 0.f;
          S.Aqk[t][s] = qk;
        }
      }
    }
  }
  const int npairs = DIAG ? 0 : L * (L + 1) / 2;
  for (int p = tid; p < npairs; p += 256) {
    int t = static_cast<int>((sqrtf(8.f * p + 1.f) - 1.f) * 0.5f);
    while (t * (t + 1) / 2 > p) --t;
    while ((t + 1) * (t + 2) / 2 <= p) ++t;
    const int s = p - t * (t + 1) / 2;
    float kk = 0.f, qk = 0.f;
#pragma unroll 4
    for (int d = 0; d < DK; d += 4) {
      const float4 ks = kq4(&S.kq.K[s][d]);
      const float4 kt = kq4(&S.kq.K[t][d]);
      const float4 qt = kq4(&S.kq.Q[t][d]);
      kk += kt.x * ks.x + kt.y * ks.y + kt.z * ks.z + kt.w * ks.w;
      qk += qt.x * ks.x + qt.y * ks.y + qt.z * ks.z + qt.w * ks.w;
    }
    const float G = S.Gm[t][s + 1];
    S.Akk[t][s] = (DELTA && s < t) ? S.beta[t] * G * kk : 0.f;
    S.Aqk[t][s] = G * qk;
  }
  {
    // a~ = (slot-0 decay) a_0 + sum_{j >= r} c_j U~_j: lanes over channels for a_0, over
    // columns for the window's coefficients
    constexpr int NA = DK / 64;
    const float s0 = DIAG ? 1.f : sc[0];
    const float cj = (lane >= r && lane < m) ? sc[A.coef_off + lane - r] : 0.f;
    for (int t = wv; t < L; t += 4) {
      float xk = 0.f, xq = 0.f;
#pragma unroll
      for (int e = 0; e < NA; ++e) {
        xk += S.a0[NA * lane + e] * kval(t, NA * lane + e);
        xq += S.a0[NA * lane + e] * qval(t, NA * lane + e);
      }
      xk = s0 * xk + cj * S.PK[lane][t];
      xq = s0 * xq + cj * S.PQ[lane][t];
      xk = wave_sum(xk);
      xq = wave_sum(xq);
      if (lane == 0) {
        S.aK[t] = xk;
        S.aQ[t] = xq;
      }
    }
  }
  __syncthreads();

  // ---- V pass: W and c by forward substitution (first half), V (U~^T q) (second half) ---------
  // Each half reads its channel of the m stored V columns, sixteen loads ahead of their use.
  const int d = tid < DV ? tid : tid - DV;
  auto v_times = [&](const float (*P)[LM], float (&acc)[LM]) {
#pragma unroll
    for (int t = 0; t < LM; ++t) acc[t] = 0.f;
    // sixteen columns at a time, the next sixteen columns' loads in flight meanwhile (a column
    // past m reads column m - 1; its row of P is zero)
    auto vload = [&](int j0, float (&vj)[16]) {
#pragma unroll
      for (int e = 0; e < 16; ++e) vj[e] = to_f32<FDT>(Vb[static_cast<int64_t>(j0 + e < m ? j0 + e : m - 1) * DV + d]);
    };
    float vj[16], vn[16];
    vload(0, vj);
#pragma unroll 1
    for (int j0 = 0; j0 < m; j0 += 16) {
      vload(j0 + 16, vn);   // unconditional (clamped), so that no branch waits on it
#pragma unroll
      for (int e = 0; e < 16; ++e) {
#pragma unroll
        for (int t4 = 0; t4 < LM / 4; ++t4) {
          const float4 p = *reinterpret_cast<const float4*>(&P[j0 + e][4 * t4]);
          acc[4 * t4] = fmaf(vj[e], p.x, acc[4 * t4]);
          acc[4 * t4 + 1] = fmaf(vj[e], p.y, acc[4 * t4 + 1]);
          acc[4 * t4 + 2] = fmaf(vj[e], p.z, acc[4 * t4 + 2]);
          acc[4 * t4 + 3] = fmaf(vj[e], p.w, acc[4 * t4 + 3]);
        }
        // one row of P at a time (hoisted, the rows' reads would take 512 registers)
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) vj[e] = vn[e];
    }
  };
  float y[LM];
  if (tid < DV) {
    // the chunk's values in this channel (a padding token reads token L - 1's; its beta is 0)
    float vt[LM];
#pragma unroll
    for (int t = 0; t < LM; ++t)
      vt[t] = to_f32<IDT>(reinterpret_cast<const IT*>(A.v)[tok(t < L ? t : L - 1) * DV + d]);
    float x[LM];
    if constexpr (DELTA) {
      v_times(S.PK, x);
    } else {
#pragma unroll
      for (int t = 0; t < LM; ++t) x[t] = 0.f;
    }
    // the content residuals w (this thread's channel) and the sink coefficients c (the same
    // scalar system, solved by every thread of the half alongside its channel); padding tokens
    // have beta = 0 and zero rows of A, so they solve to zero
    const float vbd = S.vb[d];
    float cc[LM];
#pragma unroll
    for (int t = 0; t < LM; ++t) {
      const float bt = S.beta[t];
      // (KDA: the decay to token t is inside the decayed keys already)
      const float gt = DIAG ? 1.f : S.Gm[t][0];
      float w = bt * ((vt[t] - S.omega[t] * vbd) - (DELTA ? gt * x[t] : 0.f));
      float ct = bt * (S.omega[t] - (DELTA ? gt * S.aK[t] : 0.f));
      if constexpr (DELTA) {
#pragma unroll
        for (int s = 0; s < t; ++s) {
          const float a = S.Akk[t][s];
          w = fmaf(-a, x[s], w);
          ct = fmaf(-a, cc[s], ct);
        }
        // finish the row here: left to itself the compiler sinks the arithmetic of every row
        // to the stores below and holds all 528 entries of A in registers meanwhile
        asm volatile("" : "+v"(w), "+v"(ct));
      }
      x[t] = w;
      cc[t] = ct;
    }
    // K is dead (every reader of it is above the last barrier): the full residuals
    // delta_t = w_t + c_t vbar go to LDS for the read-outs
#pragma unroll
    for (int t = 0; t < LM; ++t) {
      S.W[t][d] = fmaf(cc[t], vbd, x[t]);
      if (t < L) put(Vb + static_cast<int64_t>(m + t) * DV + d, x[t], kSiteDecodeV, 0u, m + t, d);
    }
    if (tid == 0) {
#pragma unroll
      for (int t = 0; t < LM; ++t) S.c[t] = cc[t];
    }
  } else if (tid < 2 * DV) {
    v_times(S.PQ, y);
  }
  __syncthreads();

  // ---- read-outs: o_t = vbar gamma_t a~ . q_t + gamma_t V (U~^T q_t) + sum_{s <= t}
  // Gamma(t, s) (q_t . kappa_s) delta_s; then the decay scales, coefficients and column count --
  if (tid >= DV && tid < 2 * DV) {
    const float vbd = S.vb[d];
#pragma unroll
    for (int t = 0; t < LM; ++t) {
      float o = (DIAG ? 1.f : S.Gm[t][0]) * fmaf(vbd, S.aQ[t], y[t]);
#pragma unroll
      for (int s = 0; s <= t; ++s) o = fmaf(S.Aqk[t][s], S.W[s][d], o);
      if (t < L) reinterpret_cast<IT*>(A.o)[tok(t) * DV + d] = from_f32<IDT>(o);
    }
  }
  if constexpr (DIAG) {
    // channel d: the new columns stored against the channel scale after the chunk,
    // Gamma P_{L-1}; where that falls below the floor, the channel is folded first (its scale
    // into the stored columns and a_0, the scale back to 1) and the new columns are stored true
    for (int dd = tid; dd < DK; dd += 256) {
      const float g0 = sc[dd];
      float P[LM];
      float p = 1.f;
#pragma unroll
      for (int t = 0; t < LM; ++t) {
        p *= S.Al[t][dd];
        P[t] = p;
      }
      const float gfin = g0 * P[LM - 1];   // padding gates are 1
      const bool fold = gfin < kChunkFoldFloor<FDT>;
      float rest = 1.f;                    // Gamma(L-1, t): the gates after token t
#pragma unroll
      for (int t = LM - 1; t >= 0; --t) {
        if (t < L) {
          // the key from the input again: its LDS copy now holds the residuals
          const float kv = to_f32<IDT>(reinterpret_cast<const IT*>(A.k)[tok(t) * DK + dd]);
          const float x = fold ? kv * rest : kv / (g0 * P[t]);
          put(Ub + static_cast<int64_t>(m + t) * DK + dd, x, kSiteDecodeU, 0u, m + t, dd);
          rest *= S.Al[t][dd];
        }
      }
      if (fold) {
        for (int j = 0; j < m; ++j) {
          FT* e = Ub + static_cast<int64_t>(j) * DK + dd;
          put(e, to_f32<FDT>(*e) * gfin, kSiteFoldU, static_cast<uint32_t>(m), j, dd);
        }
        A.a[unit * DK + dd] = S.a0[dd] * gfin;
      }
      sc[dd] = fold ? 1.f : gfin;
    }
    if (tid < L) sc[A.coef_off + m + tid - r] = S.c[tid];
  } else {
    const float gL = S.Gm[L - 1][0];
    if (tid <= m - r) sc[tid] *= gL;  // slot 0 and the window columns held before the chunk
    if (tid < L) {
      sc[1 + m + tid - r] = S.Gm[L - 1][tid + 1];
      sc[A.coef_off + m + tid - r] = S.c[tid];
    }
  }
  if (tid == 0) sc[A.m_off] = __uint_as_float(static_cast<uint32_t>(m + L));
}

namespace {
using ChunkFn = void (*)(const StepArgs);

template <int DK, int DV, bool DELTA, bool DIAG, int LM>
ChunkFn pick_chunk_dt(int fdt, int idt) {
  if (idt == SEED_BF16) {
    switch (fdt) {
      case SEED_F32: return k_decode_chunk<DK, DV, DELTA, DIAG, 0, 1, LM>;
      case SEED_BF16: return k_decode_chunk<DK, DV, DELTA, DIAG, 1, 1, LM>;
      case SEED_F16: return k_decode_chunk<DK, DV, DELTA, DIAG, 2, 1, LM>;
      default: return nullptr;
    }
  }
  if (idt == SEED_F32) {
    switch (fdt) {
      case SEED_F32: return k_decode_chunk<DK, DV, DELTA, DIAG, 0, 0, LM>;
      case SEED_BF16: return k_decode_chunk<DK, DV, DELTA, DIAG, 1, 0, LM>;
      default: return nullptr;
    }
  }
  return nullptr;
}

template <bool DELTA, bool DIAG, int LM>
ChunkFn pick_chunk_dims(const seed_shape& sh) {
  const int f = sh.factor_dtype, i = sh.io_dtype;
  if (sh.d_k == 128 && sh.d_v == 128) return pick_chunk_dt<128, 128, DELTA, DIAG, LM>(f, i);
  if (sh.d_k == 128 && sh.d_v == 64) return pick_chunk_dt<128, 64, DELTA, DIAG, LM>(f, i);
  if (sh.d_k == 64 && sh.d_v == 128) return pick_chunk_dt<64, 128, DELTA, DIAG, LM>(f, i);
  if (sh.d_k == 64 && sh.d_v == 64) return pick_chunk_dt<64, 64, DELTA, DIAG, LM>(f, i);
  return nullptr;
}

template <int LM>
ChunkFn pick_chunk_kind(const seed_shape& sh) {
  if (sh.rank + sh.period > kColsMax) return nullptr;
  if (sh.kind == SEED_GDN) return pick_chunk_dims<true, false, LM>(sh);
  if (sh.kind == SEED_MAMBA2) return pick_chunk_dims<false, false, LM>(sh);
  return nullptr;
}

ChunkFn pick_chunk(const seed_shape& sh, int len) {
  // KDA stages its gates and decayed keys as well: 16 tokens per call fit the LDS
  if (sh.kind == SEED_KDA) {
    if (len > kChunkMaxDiag || sh.rank + sh.period > kColsMax) return nullptr;
    return pick_chunk_dims<true, true, 16>(sh);
  }
  return len <= 16 ? pick_chunk_kind<16>(sh) : pick_chunk_kind<32>(sh);
}
}  // namespace

int32_t chunk_max_tokens() { return kChunkMax; }

bool chunk_supported(const seed_shape& sh) { return pick_chunk(sh, 1) != nullptr; }

bool chunk_supported_len(const seed_shape& sh, int32_t len) { return pick_chunk(sh, len) != nullptr; }

hipError_t launch_decode_chunk(const seed_shape& sh, const StepArgs& a, hipStream_t s) {
  ChunkFn fn = pick_chunk(sh, a.len);
  if (!fn) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(a.units)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace seed
