// Factored decode step: read-out and exact rank-one update of the sink + rank-r state.
//
// Method: pages titled "Shallow Encoding Emits Deep Memories", picx.dev summary, "SEED
// Architecture" (S = a vbar^T + U V^T) and "Exact Update (Lemma 2)" (a+ = g a + beta (omega -
// g kappa^T a) kappa, U+ = [g U, kappa], V+ = [V, beta (eps - g V U^T kappa)]), with KDA's
// diagonal gate in place of g and Mamba-2 without the delta terms.
//
// Design (gfx950): one 64-lane wavefront per (request, head) unit, four units per 256-thread
// workgroup. The step is HBM-bound: its bytes are the m columns of U and of V, read once.
// Each lane owns a 16-byte slice of a column; a wave-wide load covers 64 / (lanes per column)
// whole columns, so every load instruction streams a contiguous 1 KiB. All U and V loads of
// the unit are issued before any arithmetic, which keeps up to 32 KiB per wave in flight. With
// bf16 factors and inputs the U pass uses packed bf16 dot products (v_dot2_f32_bf16).
//   U pass: per column, x_j = (G U)_j . kappa and y_j = (G U)_j . q, reduced over the lanes of
//           the column with DPP row operations. The decay is lazy: U is never rewritten, the
//           per-column scales (GDN, Mamba-2) or per-channel Gamma (KDA) absorb it.
//   V pass: V x and V y accumulated per lane, then summed across column groups.
//   Epilogue: w = beta (eps - V x) (delta kinds) or beta eps (Mamba-2) becomes column m of V,
//           the key becomes column m of U, and o = vbar (a+ . q) + V y + (kappa . q) w.
#include "common.hpp"
#include "kernels.hpp"

namespace seed {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Third word of a raw buffer resource on gfx9-family chips (32-bit data, no swizzle).
constexpr int kRawBufferWord3 = 0x00020000;

template <int FDT, int VF>
__device__ __forceinline__ void unpack16(const uint4& r, float (&out)[VF]) {
  if constexpr (FDT == 0) {
    out[0] = __uint_as_float(r.x); out[1] = __uint_as_float(r.y);
    out[2] = __uint_as_float(r.z); out[3] = __uint_as_float(r.w);
  } else {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      out[2 * e] = __uint_as_float(w[e] << 16);
      out[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
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
      w[e] = static_cast<uint32_t>(f32_to_bf16(in[2 * e])) | (static_cast<uint32_t>(f32_to_bf16(in[2 * e + 1])) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// KDA: a channel's cumulative gate below this is folded into the stored factors (2^-40).
constexpr float kFoldFloor = 9.094947e-13f;

template <int KIND, int DK, int DV, int FDT, int IDT, int MAXC>
__global__ __launch_bounds__(256) void k_decode(const StepArgs A) {
  using FT = stor_t<FDT>;
  using IT = stor_t<IDT>;
  constexpr int VF = 16 / sizeof(FT);      // factor elements per 16-byte lane slice
  constexpr int LPU = DK / VF;             // lanes per U column
  constexpr int CPU_ = kWave / LPU;        // U columns per wave-wide load
  constexpr int LPV = DV / VF;
  constexpr int CPV = kWave / LPV;
  constexpr int NIU = (MAXC + CPU_ - 1) / CPU_;
  constexpr int NIV = (MAXC + CPV - 1) / CPV;
  constexpr bool DELTA = (KIND != SEED_MAMBA2);
  constexpr bool DIAG = (KIND == SEED_KDA);
  static_assert(LPU <= kWave && LPV <= kWave, "column wider than a wave");

  __shared__ float xs[4][MAXC];
  __shared__ float ys[4][MAXC];
  __shared__ float cscl[4][MAXC];  // per-column decay scale (GDN, Mamba-2)

  const int lane = threadIdx.x & (kWave - 1);
  // the wave index is uniform: keep it (and every per-unit address) in scalar registers
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * 4 + wv;
  if (unit >= A.units) return;  // whole wave leaves together
  const int m = A.m, r = A.rank, C = A.slots;
  const int head = static_cast<int>(unit % A.heads);

  const int ug = lane / LPU, uo = (lane % LPU) * VF;  // U column group and d_k offset
  const int vg = lane / LPV, vo = (lane % LPV) * VF;  // V column group and d_v offset

  FT* __restrict__ Ub = reinterpret_cast<FT*>(A.U) + unit * static_cast<int64_t>(C) * DK;
  FT* __restrict__ Vb = reinterpret_cast<FT*>(A.V) + unit * static_cast<int64_t>(C) * DV;

  // ---- 1. stream the factors: every U and V load of the unit is issued first -----------------
  // Buffer loads whose range ends at column m: a lane whose column is past the live ones reads
  // zeros (the range check covers the lane offset and the immediate, so the column offset is
  // kept there), and no load waits on another. Columns m..slots-1 may hold anything, even NaN.
  const __amdgpu_buffer_rsrc_t ru =
      __builtin_amdgcn_make_buffer_rsrc(Ub, 0, m * DK * static_cast<int>(sizeof(FT)), kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(Vb, 0, m * DV * static_cast<int>(sizeof(FT)), kRawBufferWord3);
  const int uoff = (ug * DK + uo) * static_cast<int>(sizeof(FT));
  const int voff = (vg * DV + vo) * static_cast<int>(sizeof(FT));
  uint4 ur[NIU];
  uint4 vr[NIV];
#pragma unroll
  for (int i = 0; i < NIU; ++i) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(ru, uoff + i * CPU_ * DK * static_cast<int>(sizeof(FT)), 0, 0);
    ur[i] = make_uint4(x[0], x[1], x[2], x[3]);
  }
#pragma unroll
  for (int i = 0; i < NIV; ++i) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(rv, voff + i * CPV * DV * static_cast<int>(sizeof(FT)), 0, 0);
    vr[i] = make_uint4(x[0], x[1], x[2], x[3]);
  }
  // keep every factor load ahead of the first wait (the scheduler would otherwise sink the V
  // loads below the U pass to save registers, serialising the two latencies)
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. per-unit vectors: key-side slices in U layout, value-side slices in V layout -------
  // bf16 factors with bf16 inputs (no channel gate): the U pass takes packed bf16 dot products
  constexpr bool DOT2 = (FDT == 1) && (IDT == 1) && !DIAG;
  float qv[VF], kv[VF], av[VF];
  uint4 qraw = make_uint4(0u, 0u, 0u, 0u), kraw = qraw;
  if constexpr (DOT2) {
    qraw = *reinterpret_cast<const uint4*>(reinterpret_cast<const IT*>(A.q) + unit * DK + uo);
    kraw = *reinterpret_cast<const uint4*>(reinterpret_cast<const IT*>(A.k) + unit * DK + uo);
    unpack16<1, VF>(qraw, qv);
    unpack16<1, VF>(kraw, kv);
  } else {
    load_f32<IDT, VF>(reinterpret_cast<const IT*>(A.q) + unit * DK + uo, qv);
    load_f32<IDT, VF>(reinterpret_cast<const IT*>(A.k) + unit * DK + uo, kv);
  }
  load_f32<0, VF>(A.a + unit * DK + uo, av);
  const float beta = A.beta[unit];
  float gv[VF];
  float gs = 0.f;
  if constexpr (DIAG) {
    load_f32<0, VF>(A.g + unit * DK + uo, gv);
  } else {
    gs = A.g[unit];
#pragma unroll
    for (int e = 0; e < VF; ++e) gv[e] = gs;
  }
  float vv[VF], vb[VF];
  load_f32<IDT, VF>(reinterpret_cast<const IT*>(A.v) + unit * DV + vo, vv);
  load_f32<0, VF>(A.vbar + static_cast<int64_t>(head) * DV + vo, vb);

  // lazy decay state
  float* __restrict__ sc = A.scale + unit * A.scale_len;
  float kt[VF], qt[VF], Gn[VF];
  float own_scale = 0.f;
  if constexpr (DIAG) {
    float Gm[VF];
    load_f32<0, VF>(sc + uo, Gm);
    bool tiny = false;
#pragma unroll
    for (int e = 0; e < VF; ++e) {
      Gn[e] = gv[e] * Gm[e];  // Gamma <- alpha . Gamma
      tiny |= !(Gn[e] >= kFoldFloor);
    }
    if (__ballot(tiny) != 0) {
      // A channel whose Gamma fell below the floor (a zero gate included) is folded into the
      // stored columns now, U_s[d][:] *= Gamma_d, and restarts at Gamma_d = 1, so that the new
      // column kappa / Gamma stays finite. Rare (uniform branch); the fold is exact up to the
      // rounding of the rewritten factors.
      float f[VF];
#pragma unroll
      for (int e = 0; e < VF; ++e) {
        const bool fold = !(Gn[e] >= kFoldFloor);
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
        if (j < m) store_f32<FDT, VF>(Ub + static_cast<int64_t>(j) * DK + uo, u);
        ur[i] = pack16<FDT, VF>(u);
      }
    }
#pragma unroll
    for (int e = 0; e < VF; ++e) {
      kt[e] = Gn[e] * kv[e];
      qt[e] = Gn[e] * qv[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < VF; ++e) { kt[e] = kv[e]; qt[e] = qv[e]; }
    // one load per lane: lane l holds slot min(l, m - r); column l's scale comes from its slot
    // (columns past the live ones get a finite stand-in: their loads read zeros)
    own_scale = sc[min(lane, m - r)];
    const float cl = gs * __shfl(own_scale, lane < r ? 0 : min(1 + lane - r, m - r));
    if (lane < MAXC) cscl[wv][lane] = cl;
    wave_lds_sync();
  }

  // ---- 3. value split along vbar (omega, eps) --------------------------------------------------
  float pvv = 0.f, pnn = 0.f;
#pragma unroll
  for (int e = 0; e < VF; ++e) { pvv += vv[e] * vb[e]; pnn += vb[e] * vb[e]; }
  pvv = group_sum<LPV>(pvv);
  pnn = group_sum<LPV>(pnn);
  const float omega = pnn > 0.f ? pvv / pnn : 0.f;
  float eps[VF];
#pragma unroll
  for (int e = 0; e < VF; ++e) eps[e] = vv[e] - omega * vb[e];

  // ---- 4. sink: a_d = G a, a+ = a_d + beta (omega - kappa . a_d) kappa (Mamba-2: no kappa . a_d)
  float ad[VF];
  float pka = 0.f, pkq = 0.f;
#pragma unroll
  for (int e = 0; e < VF; ++e) {
    ad[e] = gv[e] * av[e];
    pka += kv[e] * ad[e];
    pkq += kv[e] * qv[e];
  }
  const float ka = group_sum<LPU>(pka);
  const float s = group_sum<LPU>(pkq);  // kappa . q: the new column's share of the read-out
  const float coef = beta * (DELTA ? (omega - ka) : omega);
  float an[VF];
  float paq = 0.f;
#pragma unroll
  for (int e = 0; e < VF; ++e) {
    an[e] = ad[e] + coef * kv[e];
    paq += an[e] * qv[e];
  }
  const float aq = group_sum<LPU>(paq);

  // ---- 5. U pass: x = (G U)^T kappa, y = (G U)^T q ----------------------------------------------
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
    if constexpr (DELTA) pk = group_sum<LPU>(pk);
    pq = group_sum<LPU>(pq);
    const int j = i * CPU_ + ug;
    // every column slot is written (zero past the live columns), so the V pass needs no mask
    if ((lane % LPU) == 0) {
      const float c = DIAG ? 1.f : cscl[wv][j];
      xs[wv][j] = c * pk;
      ys[wv][j] = c * pq;
    }
  }
  wave_lds_sync();

  // ---- 6. V pass: V x and V y -------------------------------------------------------------------
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
#pragma unroll
  for (int e = 0; e < VF; ++e) {
    if constexpr (DELTA) accx[e] = across_groups_sum<LPV>(accx[e]);
    accy[e] = across_groups_sum<LPV>(accy[e]);
  }

  // ---- 7. epilogue: append the column pair, write a+, o and the decay state --------------------
  if (vg == 0) {
    float w[VF], o[VF];
#pragma unroll
    for (int e = 0; e < VF; ++e) {
      w[e] = beta * (DELTA ? (eps[e] - accx[e]) : eps[e]);
      o[e] = vb[e] * aq + accy[e] + s * w[e];
    }
    store_f32<FDT, VF>(Vb + static_cast<int64_t>(m) * DV + vo, w);
    store_f32<IDT, VF>(reinterpret_cast<IT*>(A.o) + unit * DV + vo, o);
  }
  if (ug == 0) {
    float nu[VF];
#pragma unroll
    for (int e = 0; e < VF; ++e) nu[e] = DIAG ? kv[e] / Gn[e] : kv[e];
    store_f32<FDT, VF>(Ub + static_cast<int64_t>(m) * DK + uo, nu);
    store_f32<0, VF>(A.a + unit * DK + uo, an);
    if constexpr (DIAG) store_f32<0, VF>(sc + uo, Gn);
  }
  if constexpr (!DIAG) {
    // slot 0: the r columns kept by the last compression; slot 1 + i: column r + i
    if (lane <= m - r) sc[lane] = gs * own_scale;
    else if (lane == m - r + 1) sc[lane] = 1.f;
  }
}

// ---- host-side dispatch ----------------------------------------------------------------------
namespace {

using DecodeFn = void (*)(const StepArgs);

template <int KIND, int DK, int DV, int DT>
DecodeFn pick_cols(int slots) {
  if (slots <= 32) return k_decode<KIND, DK, DV, DT, DT, 32>;
  return k_decode<KIND, DK, DV, DT, DT, 64>;
}

template <int KIND, int DK, int DV>
DecodeFn pick_dt(int dt, int slots) {
  return dt == SEED_BF16 ? pick_cols<KIND, DK, DV, 1>(slots) : pick_cols<KIND, DK, DV, 0>(slots);
}

template <int KIND>
DecodeFn pick_dims(int dk, int dv, int dt, int slots) {
  if (dk == 128 && dv == 128) return pick_dt<KIND, 128, 128>(dt, slots);
  if (dk == 128 && dv == 64) return pick_dt<KIND, 128, 64>(dt, slots);
  if (dk == 64 && dv == 128) return pick_dt<KIND, 64, 128>(dt, slots);
  if (dk == 64 && dv == 64) return pick_dt<KIND, 64, 64>(dt, slots);
  return nullptr;
}

DecodeFn pick_decode(const seed_shape& sh) {
  if (sh.factor_dtype != sh.io_dtype) return nullptr;
  const int slots = sh.rank + sh.period;
  if (slots > 64) return nullptr;
  switch (sh.kind) {
    case SEED_GDN: return pick_dims<SEED_GDN>(sh.d_k, sh.d_v, sh.factor_dtype, slots);
    case SEED_KDA: return pick_dims<SEED_KDA>(sh.d_k, sh.d_v, sh.factor_dtype, slots);
    case SEED_MAMBA2: return pick_dims<SEED_MAMBA2>(sh.d_k, sh.d_v, sh.factor_dtype, slots);
    default: return nullptr;
  }
}

}  // namespace

bool decode_supported(const seed_shape& sh) { return pick_decode(sh) != nullptr; }

hipError_t launch_decode(const seed_shape& sh, const StepArgs& a, hipStream_t s) {
  DecodeFn fn = pick_decode(sh);
  if (!fn) return hipErrorInvalidValue;
  const int64_t blocks = (a.units + 3) / 4;
  hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace seed
