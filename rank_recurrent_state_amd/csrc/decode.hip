// Factored decode step: read-out and exact rank-one update of the sink + rank-r state.
//
// Method: pages titled "Shallow Encoding Emits Deep Memories", picx.dev summary, "SEED
// Architecture" (S = a vbar^T + U V^T) and "Exact Update (Lemma 2)" (a+ = g a + beta (omega -
// g kappa^T a) kappa, U+ = [g U, kappa], V+ = [V, beta (eps - g V U^T kappa)]), with KDA's
// diagonal gate in place of g and Mamba-2 without the delta terms.
//
// Design (gfx950): one 64-lane wavefront per (request, head) unit, two units per 128-thread
// workgroup. The step is HBM-bound: its bytes are the m columns of U and of V, read once, with
// non-temporal loads (no reuse within a step). Each lane owns a 16-byte slice of a column; a
// wave-wide load covers 64 / (lanes per column) whole columns, so every load instruction
// streams a contiguous 1 KiB. The small per-unit vectors are loaded first, then U, and V
// either with U or, where both would not fit in 96 registers per lane, as soon as the U pass
// has consumed U (half the registers per wave: a 4096-unit launch is resident at once). With
// bf16 factors and inputs the U pass uses packed bf16 dot products (v_dot2_f32_bf16).
//   U pass: per column, x_j = (G U)_j . kappa and y_j = (G U)_j . q, summed over the lanes of
//           the column with transposed DPP exchanges (every lane ends with one column). The
//           decay is lazy: U is never rewritten, the per-column scales (GDN, Mamba-2) or
//           per-channel Gamma (KDA) absorb it.
//   V pass: V x and V y accumulated per lane, then summed across column groups with
//           transposed permlane swaps (every lane ends with a few elements of d_v).
//   Epilogue: w = beta (eps - V x) (delta kinds) or beta eps (Mamba-2) becomes column m of V,
//           the key becomes column m of U, and o = vbar (a+ . q) + V y + (kappa . q) w;
//           optionally o is normalised in place (per-head RMS norm with weight and gate, one
//           more wave sum: no further pass over the factors).
// The sink is lazy as well. Lemma 2 adds a multiple of kappa to a at every step, and kappa is
// the column the step appends to U, so the state keeps a_0 (the sink when the factors were last
// compressed) and one coefficient c_j per window column: a = (decay of slot 0) a_0 + sum_j c_j
// (decayed U)_j. The step reads a_0 and the coefficients and writes only its own c_m = beta
// (omega - kappa . a) (beta omega for Mamba-2). It never rewrites the d_k-vector a, whose
// read-modify-write made a third stream next to the factor reads and column writes. Compression
// folds a back to one vector and clears the coefficients.
#include "common.hpp"
#include "kernels.hpp"

namespace seed {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Third word of a raw buffer resource on gfx9-family chips (32-bit data, no swizzle).
constexpr int kRawBufferWord3 = 0x00020000;
// Cache-policy bits of a buffer load: non-temporal (gfx950's nt bit). A step reads each factor
// column once, and the next read of the same state comes only after the other layers' traffic.
constexpr int kNonTemporal = 2;

// NI wave-wide loads of 16 bytes per lane over consecutive KiB of a unit's factor columns, with
// the bytes past `bytes` (the columns at and after m) reading as zeros. Each resource covers
// four loads, so one lane offset and the immediate field serve them all and the range check sees
// the whole offset (the buffer range check covers the lane offset and the immediate only).
template <int NI>
__device__ __forceinline__ void load_columns(const void* base, int bytes, int lane_off, uint4 (&out)[NI]) {
#pragma unroll
  for (int g = 0; g < (NI + 3) / 4; ++g) {
    const int rest = bytes - g * 4096;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(static_cast<const char*>(base)) + g * 4096, 0, rest > 0 ? rest : 0, kRawBufferWord3);
#pragma unroll
    for (int k = 0; k < 4 && 4 * g + k < NI; ++k) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, lane_off + k * 1024, 0, kNonTemporal);
      out[4 * g + k] = make_uint4(x[0], x[1], x[2], x[3]);
    }
  }
}

template <int FDT, int VF>
__device__ __forceinline__ void unpack16(const uint4& r, float (&out)[VF]) {
  if constexpr (FDT == 0) {
    out[0] = __uint_as_float(r.x); out[1] = __uint_as_float(r.y);
    out[2] = __uint_as_float(r.z); out[3] = __uint_as_float(r.w);
  } else {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      out[2 * e] = lo16<FDT>(w[e]);
      out[2 * e + 1] = hi16<FDT>(w[e]);
    }
  }
}

template <int FDT, int VF>
__device__ __forceinline__ uint4 pack16(const float (&in)[VF]) {
  if constexpr (FDT == 0) {
    return make_uint4(__float_as_uint(in[0]), __float_as_uint(in[1]), __float_as_uint(in[2]), __float_as_uint(in[3]));
  } else {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = pack2<FDT>(in[2 * e], in[2 * e + 1]);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Store N consecutive elements (elem0 .. elem0 + N - 1, inside one group of 8) of a factor
// column: nearest-even, or, with sr, stochastic rounding drawn for that site, slot and unit.
template <int FDT, int N>
__device__ __forceinline__ void store_factor(stor_t<FDT>* __restrict__ p, const float (&x)[N], bool sr,
                                             uint32_t key, uint32_t site, uint32_t aux, int slot, int64_t unit,
                                             uint32_t window, int elem0) {
  if constexpr (FDT == 0) {
    store_f32<0, N>(p, x);
  } else {
    if (sr) {
      const uint4 w = sr_group(key, site, aux, slot, unit, window, elem0);
      uint32_t rr[N];
#pragma unroll
      for (int e = 0; e < N; ++e) rr[e] = draw16(w, (elem0 + e) & 7);
      store_sr<FDT, N>(p, x, rr);
    } else {
      store_f32<FDT, N>(p, x);
    }
  }
}

// One 16-byte slice (VF elements from elem0, inside one group of 8 for 16-bit formats) of a factor
// column, rounded as store_factor does.
template <int FDT, int VF>
__device__ __forceinline__ uint4 pack_factor(const float (&x)[VF], bool sr, uint32_t key, uint32_t site, uint32_t aux,
                                             int slot, int64_t unit, uint32_t window, int elem0) {
  if constexpr (FDT != 0) {
    if (sr) {
      const uint4 w = sr_group(key, site, aux, slot, unit, window, elem0);
      uint32_t h[VF];
#pragma unroll
      for (int e = 0; e < VF; ++e) h[e] = round_sr<FDT>(x[e], draw16(w, (elem0 + e) & 7));
      return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
    }
  }
  return pack16<FDT, VF>(x);
}

// KDA: a channel's cumulative gate below this is folded into the stored factors: 2^-40 for
// fp32 and bf16 storage, 2^-12 for fp16, whose range (65504) must hold kappa / Gamma.
template <int FDT>
constexpr float kFoldFloor = FDT == 2 ? 2.44140625e-4f : 9.094947e-13f;

// ---- transposed sums ---------------------------------------------------------------------------
// A lane holds N partial sums, each to be summed over a group of lanes. Rather than reducing
// every value over the whole group (N log2 W exchanges), pairs of values trade halves at each
// bit of the lane index: the lane whose bit is clear keeps the first of the pair plus its
// partner's copy, the other keeps the second, so the N sums take N - 1 exchanges and end up
// spread over the lanes.

// The partner at bit B of lane % 16 inside a 16-lane row: row_mirror (B = 8),
// row_half_mirror (4), lane ^ 2, lane ^ 1. Each partner differs in bit B and agrees on the bits
// above it, which is all the pairing needs.
template <int B>
__device__ __forceinline__ float row_partner(float v) {
  if constexpr (B == 8) return dpp<0x140>(v);
  else if constexpr (B == 4) return dpp<0x141>(v);
  else if constexpr (B == 2) return dpp<0x4E>(v);
  else return dpp<0xB1>(v);
}

// Sums over aligned groups of 2B lanes (B = W / 2 at the call; W <= 32): afterwards lane t of a
// group holds in v[0] the group's total of v[t * N / W] as it was on entry (N <= W; for N < W,
// W / N neighbouring lanes hold the same total).
template <int NMAX, int N, int B>
__device__ __forceinline__ void tsum_in_group(float (&v)[NMAX], int lane) {
  if constexpr (B >= 1) {
    constexpr int H = N / 2;
    if constexpr (N >= 2) {
      if constexpr (B == 16) {
#pragma unroll
        for (int k = 0; k < H; ++k) {
          lane_swap16(v[k], v[k + H]);
          v[k] += v[k + H];
        }
      } else {
        const bool hi = (lane & B) != 0;
#pragma unroll
        for (int k = 0; k < H; ++k) {
          const float keep = hi ? v[k + H] : v[k];
          const float send = hi ? v[k] : v[k + H];
          v[k] = keep + row_partner<B>(send);
        }
      }
      tsum_in_group<NMAX, H, B / 2>(v, lane);
    } else {
      if constexpr (B == 16) {
        float x = v[0], y = v[0];
        lane_swap16(x, y);
        v[0] = x + y;
      } else {
        v[0] += row_partner<B>(v[0]);
      }
      tsum_in_group<NMAX, 1, B / 2>(v, lane);
    }
  }
}

// Sums over the 64 / W lanes that share lane % W (bits B = 32 down to W of the lane index):
// afterwards the lanes of group g = lane / W hold the totals of v[g * N * W / 64 ...] in
// v[0 .. N * W / 64 - 1].
template <int NMAX, int N, int B, int W>
__device__ __forceinline__ void tsum_across_groups(float (&v)[NMAX], int lane) {
  if constexpr (B >= W) {
    static_assert(N >= 2, "fewer values than groups");
    constexpr int H = N / 2;
    if constexpr (B == 32 || B == 16) {
#pragma unroll
      for (int k = 0; k < H; ++k) {
        if constexpr (B == 32) lane_swap32(v[k], v[k + H]);
        else lane_swap16(v[k], v[k + H]);
        v[k] += v[k + H];
      }
    } else {
      static_assert(B == 8, "partner lane ^ 8 inside a row (row_ror 8)");
      const bool hi = (lane & B) != 0;
#pragma unroll
      for (int k = 0; k < H; ++k) {
        const float keep = hi ? v[k + H] : v[k];
        const float send = hi ? v[k] : v[k + H];
        v[k] = keep + dpp<0x128>(send);
      }
    }
    tsum_across_groups<NMAX, H, B / 2, W>(v, lane);
  }
}

// Lane geometry of one unit, and how its factors are staged. A lane owns a 16-byte slice of a
// column; NIU (NIV) wave-wide loads cover MAXC columns of U (V). When both sets together would
// hold more than 96 registers per lane, V is loaded only after the U pass has consumed U, so a
// wave needs half the registers and twice as many waves are resident.
template <int DK, int DV, int FDT, int MAXC>
struct DecodeGeom {
  static constexpr int VF = FDT == 0 ? 4 : 8;
  static constexpr int LPU = DK / VF, CPU_ = kWave / LPU, LPV = DV / VF, CPV = kWave / LPV;
  static constexpr int NIU = (MAXC + CPU_ - 1) / CPU_, NIV = (MAXC + CPV - 1) / CPV;
  static constexpr bool SPLIT = (NIU + NIV) * 4 > 96;
  static constexpr int DATA = 4 * (SPLIT ? (NIU > NIV ? NIU : NIV) : NIU + NIV);
  // waves per SIMD the register budget is cut for (512 registers per lane per SIMD)
  static constexpr int WAVES = DATA <= 64 ? 4 : (DATA <= 128 ? 2 : 1);
};

// Units (wavefronts) per workgroup. Two measured faster than four or eight on the layer-stack
// workload (22.0 against 22.4 and 22.7 us per 4096-unit launch): smaller workgroups are placed as
// soon as two wave slots free up.
constexpr int kUnitsPerBlock = 2;

template <int KIND, int DK, int DV, int FDT, int IDT, int MAXC>
__global__ __launch_bounds__(64 * kUnitsPerBlock) __attribute__((amdgpu_waves_per_eu(DecodeGeom<DK, DV, FDT, MAXC>::WAVES)))
void k_decode(const StepArgs A) {
  using FT = stor_t<FDT>;
  using IT = stor_t<IDT>;
  using Geo = DecodeGeom<DK, DV, FDT, MAXC>;
  constexpr int VF = Geo::VF;       // factor elements per 16-byte lane slice
  constexpr int LPU = Geo::LPU;     // lanes per U column
  constexpr int CPU_ = Geo::CPU_;   // U columns per wave-wide load
  constexpr int LPV = Geo::LPV;
  constexpr int CPV = Geo::CPV;
  constexpr int NIU = Geo::NIU;
  constexpr int NIV = Geo::NIV;
  constexpr bool SPLIT = Geo::SPLIT;
  constexpr int NB = VF * LPV / kWave;  // value elements per lane once the V pass is summed
  constexpr bool DELTA = (KIND != SEED_MAMBA2);
  constexpr bool DIAG = (KIND == SEED_KDA);
  static_assert(VF * sizeof(FT) == 16, "16-byte lane slices");
  static_assert(LPU <= 32 && LPV <= 32 && NIU <= LPU && NB >= 1, "lane geometry");
  static_assert(CPU_ * DK * sizeof(FT) == 1024 && CPV * DV * sizeof(FT) == 1024, "1 KiB per load");

  __shared__ float xs[kUnitsPerBlock][MAXC];
  __shared__ float ys[kUnitsPerBlock][MAXC];

  const int lane = threadIdx.x & (kWave - 1);
  // the wave index is uniform: keep it (and every per-unit address) in scalar registers
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * kUnitsPerBlock + wv;
  if (unit >= A.units) return;  // whole wave leaves together
  float* __restrict__ sc = A.scale + unit * A.scale_len;
  const int r = A.rank, C = A.slots;
  int m = A.m;
  if (A.ragged) {
    // the unit's own column count; inactive units, and counts outside [r, r + T) (a full unit
    // awaiting its compression), are left as they are (whole wave)
    m = static_cast<int>(__float_as_uint(sc[A.m_off]));
    if ((A.active != nullptr && A.active[unit] == 0) || m < r || m >= C) return;
  }
  const int head = static_cast<int>(unit % A.heads);

  const int ug = lane / LPU, uo = (lane % LPU) * VF;  // U column group and d_k offset
  const int vg = lane / LPV, vo = (lane % LPV) * VF;  // V column group and d_v offset
  // the column whose x and y this lane holds after the U pass's transposed sums
  const int jt = ((lane % LPU) * NIU / LPU) * CPU_ + ug;
  // the value elements this lane finishes: NB of them from d_v index ve
  const int ve = vo + vg * NB;

  FT* __restrict__ Ub = reinterpret_cast<FT*>(A.U) + unit * static_cast<int64_t>(C) * DK;
  FT* __restrict__ Vb = reinterpret_cast<FT*>(A.V) + unit * static_cast<int64_t>(C) * DV;

  // ---- 1. key-side vectors (U layout) and the lazy decay state -------------------------------
  // These small loads go ahead of the factors: loads complete in order, so the values that need
  // only them (the new U column, the column scales) do not wait for the factors.
  // bf16 factors with bf16 inputs (no channel gate): the U pass takes packed bf16 dot products
  constexpr bool DOT2 = (FDT == 1) && (IDT == 1) && !DIAG;
  const IT* __restrict__ qp = reinterpret_cast<const IT*>(A.q) + unit * DK + uo;
  const IT* __restrict__ kp = reinterpret_cast<const IT*>(A.k) + unit * DK + uo;
  uint4 qraw = make_uint4(0u, 0u, 0u, 0u), kraw = qraw;
  float kt[VF], qt[VF];  // the U pass's operands (KDA: Gamma . kappa, Gamma . q)
  if constexpr (DOT2) {
    qraw = *reinterpret_cast<const uint4*>(qp);
    kraw = *reinterpret_cast<const uint4*>(kp);
  } else {
    load_f32<IDT, VF>(qp, qt);
    load_f32<IDT, VF>(kp, kt);
  }
  const float beta = A.beta[unit];
  const float gs = DIAG ? 0.f : A.g[unit];
  float own_scale = 0.f, col_scale = 1.f, slot0 = 1.f, Gm[VF], alpha[VF], av[VF];
  if constexpr (DIAG) {
    load_f32<0, VF>(A.g + unit * DK + uo, alpha);
    load_f32<0, VF>(sc + uo, Gm);
  } else {
    // slot 0 scales the r columns kept by the last compression, slot 1 + i column r + i; a
    // column past the live ones gets a finite stand-in (its loads read zeros)
    own_scale = sc[min(lane, m - r)];
    col_scale = sc[jt < r ? 0 : min(1 + jt - r, m - r)];
    slot0 = sc[0];
  }
  // the lazy sink: a_0 (decayed like slot 0; KDA: by Gamma) plus c_j times each window column
  load_f32<0, VF>(A.a + unit * DK + uo, av);
  const float cw = (jt >= r && jt < m) ? sc[A.coef_off + jt - r] : 0.f;
  // stochastic rounding of the stores (16-bit factors): the unit's compression-window count
  const bool sr = FDT != 0 && A.rounding != 0;
  const uint32_t window = sr ? __float_as_uint(sc[A.win_off]) : 0u;

  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. stream the factors --------------------------------------------------------------------
  const int uoff = (ug * DK + uo) * static_cast<int>(sizeof(FT));
  const int voff = (vg * DV + vo) * static_cast<int>(sizeof(FT));
  uint4 ur[NIU];
  uint4 vr[NIV];
  auto load_v = [&]() { load_columns<NIV>(Vb, m * DV * static_cast<int>(sizeof(FT)), voff, vr); };
  load_columns<NIU>(Ub, m * DK * static_cast<int>(sizeof(FT)), uoff, ur);
  if constexpr (!SPLIT) load_v();
  // keep the factor loads ahead of the first wait (the scheduler would otherwise sink them
  // below the U pass to save registers, serialising the latencies)
  __builtin_amdgcn_sched_barrier(0);

  // kappa . q (the new column's share of the read-out) and the sink's a_0 part of kappa . a_d and
  // a_d . q, before the U pass
  float s, ka0, aq0;
  if constexpr (DIAG) {
    float Gn[VF];
    bool tiny = false;
#pragma unroll
    for (int e = 0; e < VF; ++e) {
      Gn[e] = alpha[e] * Gm[e];  // Gamma <- alpha . Gamma
      tiny |= !(Gn[e] >= kFoldFloor<FDT>);
    }
    if (__ballot(tiny) != 0) {
      // A channel whose Gamma fell below the floor (a zero gate included) is folded into the
      // stored columns now, U_s[d][:] *= Gamma_d, and restarts at Gamma_d = 1, so that the new
      // column kappa / Gamma stays finite. Rare (uniform branch); the fold is exact up to the
      // rounding of the rewritten factors.
      float f[VF];
#pragma unroll
      for (int e = 0; e < VF; ++e) {
        const bool fold = !(Gn[e] >= kFoldFloor<FDT>);
        f[e] = fold ? Gn[e] : 1.f;
        Gn[e] = fold ? 1.f : Gn[e];
      }
#pragma unroll
      for (int i = 0; i < NIU; ++i) {
        const int j = i * CPU_ + ug;
        float u[VF];
        unpack16<FDT, VF>(ur[i], u);
#pragma unroll
        for (int e = 0; e < VF; ++e) u[e] *= f[e];
        // the U pass below uses exactly the rewritten bits
        ur[i] = pack_factor<FDT, VF>(u, sr, A.rng_key, kSiteFoldU, static_cast<uint32_t>(m), j, unit, window, uo);
        if (j < m) *reinterpret_cast<uint4*>(Ub + static_cast<int64_t>(j) * DK + uo) = ur[i];
        __builtin_amdgcn_sched_barrier(0);  // one column at a time (keeps the draws' registers few)
      }
      // a_0 carries the same per-channel factor as the stored columns
#pragma unroll
      for (int e = 0; e < VF; ++e) av[e] *= f[e];
      if (ug == 0) store_f32<0, VF>(A.a + unit * DK + uo, av);
    }
    // the new U column kappa / Gamma and Gamma itself do not depend on the passes: written now
    // (the U pass reads only the columns before m), their registers are free for the U pass.
    // With stochastic rounding the column is written at the end instead, where the draws do not
    // compete with the factor loads for registers.
    if (ug == 0) {
      if (!sr) {
        float nu[VF];
#pragma unroll
        for (int e = 0; e < VF; ++e) nu[e] = kt[e] / Gn[e];
        store_f32<FDT, VF>(Ub + static_cast<int64_t>(m) * DK + uo, nu);
      }
      store_f32<0, VF>(sc + uo, Gn);
    }
    float pkq = 0.f, pka = 0.f, paq = 0.f;
#pragma unroll
    for (int e = 0; e < VF; ++e) {
      pkq += kt[e] * qt[e];
      kt[e] *= Gn[e];
      qt[e] *= Gn[e];
      pka += kt[e] * av[e];
      paq += qt[e] * av[e];
    }
    s = group_sum<LPU>(pkq);
    ka0 = group_sum<LPU>(pka);
    aq0 = group_sum<LPU>(paq);
  } else {
    col_scale *= gs;
    float kv[VF], qv[VF];
    if constexpr (DOT2) {
      unpack16<1, VF>(kraw, kv);
      unpack16<1, VF>(qraw, qv);
    } else {
#pragma unroll
      for (int e = 0; e < VF; ++e) { kv[e] = kt[e]; qv[e] = qt[e]; }
    }
    float pkq = 0.f, pka = 0.f, paq = 0.f;
#pragma unroll
    for (int e = 0; e < VF; ++e) {
      pkq += kv[e] * qv[e];
      pka += kv[e] * av[e];
      paq += qv[e] * av[e];
    }
    const float p0 = gs * slot0;  // a_0's decay to this step
    s = group_sum<LPU>(pkq);
    ka0 = p0 * group_sum<LPU>(pka);
    aq0 = p0 * group_sum<LPU>(paq);
  }

  // ---- 3. U pass: x = (G U)^T kappa, y = (G U)^T q ----------------------------------------------
  float px[NIU], py[NIU];
#pragma unroll
  for (int i = 0; i < NIU; ++i) {
    float pk = 0.f, pq = 0.f;
    if constexpr (DOT2) {
      const uint32_t uw[4] = {ur[i].x, ur[i].y, ur[i].z, ur[i].w};
      const uint32_t kw[4] = {kraw.x, kraw.y, kraw.z, kraw.w};
      const uint32_t qw[4] = {qraw.x, qraw.y, qraw.z, qraw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2 ue = __builtin_bit_cast(bf16x2, uw[e]);
        if constexpr (DELTA) pk = __builtin_amdgcn_fdot2_f32_bf16(ue, __builtin_bit_cast(bf16x2, kw[e]), pk, false);
        pq = __builtin_amdgcn_fdot2_f32_bf16(ue, __builtin_bit_cast(bf16x2, qw[e]), pq, false);
      }
    } else {
      float u[VF];
      unpack16<FDT, VF>(ur[i], u);
#pragma unroll
      for (int e = 0; e < VF; ++e) {
        if constexpr (DELTA) pk += u[e] * kt[e];
        pq += u[e] * qt[e];
      }
    }
    px[i] = pk;
    py[i] = pq;
  }
  // column sums over the LPU lanes of each column, transposed: this lane ends with column jt
  if constexpr (DELTA) tsum_in_group<NIU, NIU, LPU / 2>(px, lane);
  tsum_in_group<NIU, NIU, LPU / 2>(py, lane);
  // every column slot is written (zero past the live columns), so the V pass needs no mask;
  // lanes that share a column write the same value
  const float xj = col_scale * px[0], yj = col_scale * py[0];
  if constexpr (DELTA) xs[wv][jt] = xj;
  ys[wv][jt] = yj;

  // ---- 4. the value-side vectors, then V when it was not loaded up front -----------------------
  // The small loads go first: loads complete in order, so the value split waits only for them.
  if constexpr (SPLIT) __builtin_amdgcn_sched_barrier(0);
  float vv[NB], vb[NB];
  load_f32<IDT, NB>(reinterpret_cast<const IT*>(A.v) + unit * DV + ve, vv);
  load_f32<0, NB>(A.vbar + static_cast<int64_t>(head) * DV + ve, vb);
  // the head normalisation's weight and gate (when fused in), here so that their latency hides
  // behind the V pass
  const bool normed = A.norm_w != nullptr, gated = normed && A.norm_gate != nullptr;
  float nw[NB], gz[NB];
  if (normed) load_f32<0, NB>(A.norm_w + static_cast<int64_t>(head) * DV + ve, nw);
  if (gated) load_f32<IDT, NB>(reinterpret_cast<const IT*>(A.norm_gate) + unit * DV + ve, gz);
  if constexpr (SPLIT) {
    load_v();
    __builtin_amdgcn_sched_barrier(0);
  }
  wave_lds_sync();

  // the window's share of the sink: sum_j c_j x_j and sum_j c_j y_j (one copy of each column;
  // summed once the V loads are out)
  const bool first = ((lane % LPU) % (LPU / NIU)) == 0;
  const float cx = DELTA ? wave_sum(first ? cw * xj : 0.f) : 0.f;
  const float cy = wave_sum(first ? cw * yj : 0.f);

  // value split along vbar (omega, eps): every lane holds NB distinct elements of v
  float pvv = 0.f, pnn = 0.f;
#pragma unroll
  for (int e = 0; e < NB; ++e) { pvv += vv[e] * vb[e]; pnn += vb[e] * vb[e]; }
  pvv = wave_sum(pvv);
  pnn = wave_sum(pnn);
  const float omega = pnn > 0.f ? pvv / pnn : 0.f;

  // sink: a_d = G a, a+ = a_d + beta (omega - kappa . a_d) kappa (Mamba-2: no kappa . a_d). The
  // new column's coefficient is beta (omega - kappa . a_d) (Mamba-2: beta omega), and
  // a+ . q = a_d . q + coef (kappa . q).
  const float ka = ka0 + cx;
  const float coef = beta * (DELTA ? (omega - ka) : omega);
  const float aq = aq0 + cy + coef * s;

  // the coefficient and the decay state are final: write them now
  if (lane == 0) {
    sc[A.coef_off + m - r] = coef;
    sc[A.m_off] = __uint_as_float(static_cast<uint32_t>(m + 1));
  }
  if constexpr (!DIAG) {
    if (lane <= m - r) sc[lane] = gs * own_scale;
    else if (lane == m - r + 1) sc[lane] = 1.f;
  }

  // ---- 5. V pass: V x and V y -------------------------------------------------------------------
  float accx[VF], accy[VF];
#pragma unroll
  for (int e = 0; e < VF; ++e) { accx[e] = 0.f; accy[e] = 0.f; }
#pragma unroll
  for (int i = 0; i < NIV; ++i) {
    const int j = i * CPV + vg;
    const float xj = DELTA ? xs[wv][j] : 0.f;
    const float yj = ys[wv][j];
    float vc[VF];
    unpack16<FDT, VF>(vr[i], vc);
#pragma unroll
    for (int e = 0; e < VF; ++e) {
      if constexpr (DELTA) accx[e] += xj * vc[e];
      accy[e] += yj * vc[e];
    }
  }
  // sums over the column groups, transposed: this lane ends with elements ve .. ve + NB - 1
  if constexpr (DELTA) tsum_across_groups<VF, VF, 32, LPV>(accx, lane);
  tsum_across_groups<VF, VF, 32, LPV>(accy, lane);

  // ---- 6. epilogue: append the V column and write o (every lane: NB elements) -----------------
  float w[NB], o[NB];
#pragma unroll
  for (int e = 0; e < NB; ++e) {
    const float eps = vv[e] - omega * vb[e];
    w[e] = beta * (DELTA ? (eps - accx[e]) : eps);
    o[e] = vb[e] * aq + accy[e] + s * w[e];
  }
  store_factor<FDT, NB>(Vb + static_cast<int64_t>(m) * DV + ve, w, sr, A.rng_key, kSiteDecodeV, 0u, m, unit, window,
                        ve);
  if (normed) {  // uniform: the head normalisation of the read-out
    // The lanes hold distinct elements of o, so its mean square is one wave sum. The sink's
    // share vbar (a+ . q) is inside the norm: a bias along vbar, and part of the gain 1 / rms.
    if (gated) {
#pragma unroll
      for (int e = 0; e < NB; ++e) gz[e] *= __builtin_amdgcn_rcpf(1.f + __expf(-gz[e]));   // silu
    }
    const bool gfirst = gated && A.norm_gate_first != 0;
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < NB; ++e) {
      if (gfirst) o[e] *= gz[e];
      ss = fmaf(o[e], o[e], ss);
    }
    ss = wave_sum(ss);
    const float rinv = __builtin_amdgcn_rsqf(ss * (1.f / DV) + A.norm_eps);
#pragma unroll
    for (int e = 0; e < NB; ++e) {
      o[e] *= rinv * nw[e];
      if (gated && !gfirst) o[e] *= gz[e];
    }
  }
  store_f32<IDT, NB>(reinterpret_cast<IT*>(A.o) + unit * DV + ve, o);
  if constexpr (!DIAG) {
    // The new U column is the key itself. It is stored here, with the step's other writes: stored
    // ahead of the U pass, in the middle of the factor reads, it cost 0.4 us more per 4096-unit
    // launch.
    if (ug == 0) {
      float nu[VF];
      if constexpr (DOT2) {
        unpack16<1, VF>(kraw, nu);
      } else {
#pragma unroll
        for (int e = 0; e < VF; ++e) nu[e] = kt[e];
      }
      store_factor<FDT, VF>(Ub + static_cast<int64_t>(m) * DK + uo, nu, sr, A.rng_key, kSiteDecodeU, 0u, m, unit,
                            window, uo);
    }
  }
  if constexpr (DIAG && FDT != 0) {
    // KDA with stochastic rounding: the new U column kappa / Gamma, from the key read again and
    // the Gamma this lane stored above (the same quotients as the early store would take)
    if (sr && ug == 0) {
      float kk[VF], gg[VF], nu[VF];
      load_f32<IDT, VF>(kp, kk);
      load_f32<0, VF>(sc + uo, gg);
#pragma unroll
      for (int e = 0; e < VF; ++e) nu[e] = kk[e] / gg[e];
      store_factor<FDT, VF>(Ub + static_cast<int64_t>(m) * DK + uo, nu, true, A.rng_key, kSiteDecodeU, 0u, m, unit,
                            window, uo);
    }
  }
}

// ---- host-side dispatch ----------------------------------------------------------------------
namespace {

using DecodeFn = void (*)(const StepArgs);

template <int KIND, int DK, int DV, int FDT, int IDT>
DecodeFn pick_cols(int slots) {
  if (slots <= 32) return k_decode<KIND, DK, DV, FDT, IDT, 32>;
  return k_decode<KIND, DK, DV, FDT, IDT, 64>;
}

// factor / input dtypes: fp32 / fp32, bf16 / bf16, fp16 / bf16
template <int KIND, int DK, int DV>
DecodeFn pick_dt(int fdt, int idt, int slots) {
  if (fdt == SEED_F32 && idt == SEED_F32) return pick_cols<KIND, DK, DV, 0, 0>(slots);
  if (fdt == SEED_BF16 && idt == SEED_BF16) return pick_cols<KIND, DK, DV, 1, 1>(slots);
  if (fdt == SEED_F16 && idt == SEED_BF16) return pick_cols<KIND, DK, DV, 2, 1>(slots);
  return nullptr;
}

template <int KIND>
DecodeFn pick_dims(int dk, int dv, int fdt, int idt, int slots) {
  if (dk == 128 && dv == 128) return pick_dt<KIND, 128, 128>(fdt, idt, slots);
  if (dk == 128 && dv == 64) return pick_dt<KIND, 128, 64>(fdt, idt, slots);
  if (dk == 64 && dv == 128) return pick_dt<KIND, 64, 128>(fdt, idt, slots);
  if (dk == 64 && dv == 64) return pick_dt<KIND, 64, 64>(fdt, idt, slots);
  return nullptr;
}

DecodeFn pick_decode(const seed_shape& sh) {
  const int slots = sh.rank + sh.period;
  if (slots > 64) return nullptr;
  const int f = sh.factor_dtype, i = sh.io_dtype;
  switch (sh.kind) {
    case SEED_GDN: return pick_dims<SEED_GDN>(sh.d_k, sh.d_v, f, i, slots);
    case SEED_KDA: return pick_dims<SEED_KDA>(sh.d_k, sh.d_v, f, i, slots);
    case SEED_MAMBA2: return pick_dims<SEED_MAMBA2>(sh.d_k, sh.d_v, f, i, slots);
    default: return nullptr;
  }
}

}  // namespace

bool decode_supported(const seed_shape& sh) { return pick_decode(sh) != nullptr; }

hipError_t launch_decode(const seed_shape& sh, const StepArgs& a, hipStream_t s) {
  DecodeFn fn = pick_decode(sh);
  if (!fn) return hipErrorInvalidValue;
  const int64_t blocks = (a.units + kUnitsPerBlock - 1) / kUnitsPerBlock;
  hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(blocks)), dim3(64 * kUnitsPerBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace seed
