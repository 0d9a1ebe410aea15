// Energy of the factored state per unit: the total |S~|_F^2, the sink's |a vbar^T|_F^2 and the
// content's |U V^T|_F^2, with S~ = a vbar^T + U V^T (true, decayed form).
//
// Method: pages titled "Shallow Encoding Emits Deep Memories", picx.dev summary, key finding 2
// and "Introduction and Theoretical Foundation" (the state sink: a rank-one term along the
// head's mean value direction holds most of the state's energy; the sink's share is the
// diagnostic the pages report, pooled over heads).
//
// Design (gfx950): a diagnostic, not on the decode path. 16-bit factors take a one-wavefront
// kernel with MFMA Grams (compress_wave.hip). This generic kernel (fp32 factors): one 256-thread
// workgroup per unit stages
// the m true columns of U in LDS as fp32 (33 KB for d_k = 128 and 64 columns), forms a_true from
// the lazy sink and U's Gram, then stages V in the same buffer, and reduces
//   |S~|^2 = |a|^2 |vbar|^2 + 2 (U^T a) . (V^T vbar) + sum_{i,j} (U_i . U_j)(V_i . V_j)
// over the column pairs i <= j (the Grams' elementwise product, symmetric). It reads the factors
// once; the per-unit column count comes from the state.
#include "common.hpp"
#include "kernels.hpp"

namespace seed {

namespace {

constexpr int kMaxCols = 64;

// Sum over the 256 threads of a workgroup; every thread gets it. Must be reached by all threads.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

}  // namespace

template <int DK, int DV, int FDT, bool DIAG>
__global__ __launch_bounds__(256) void k_energy(const EnergyArgs A) {
  constexpr int LDF = (DK > DV ? DK : DV) + 1;
  __shared__ float F[kMaxCols][LDF];             // the true columns of U, then of V
  __shared__ float G[kMaxCols][kMaxCols + 1];    // U's Gram, upper triangle
  __shared__ float at[DK];
  __shared__ float xs[kMaxCols];
  __shared__ float red[4];
  using FT = stor_t<FDT>;
  const int t = threadIdx.x;
  const int64_t unit = blockIdx.x;
  const int r = A.rank, C = A.slots;
  const float* __restrict__ sc = A.scale + unit * A.scale_len;
  // the unit's column count (unsigned; a count beyond the slots reads as all of them)
  const uint32_t mu = __float_as_uint(sc[A.m_off]);
  const int m = mu > static_cast<uint32_t>(C) ? C : static_cast<int>(mu);
  const FT* __restrict__ Ub = reinterpret_cast<const FT*>(A.U) + unit * static_cast<int64_t>(C) * DK;
  const FT* __restrict__ Vb = reinterpret_cast<const FT*>(A.V) + unit * static_cast<int64_t>(C) * DV;
  const float* __restrict__ vb = A.vbar + static_cast<int64_t>(unit % A.heads) * DV;
  const int npairs = m * (m + 1) / 2;
  // pair p -> (i, j), i <= j, row-major over the upper triangle
  auto pair_of = [m](int p, int& i, int& j) {
    i = 0;
    while (p >= m - i) {
      p -= m - i;
      ++i;
    }
    j = i + p;
  };

  // ---- U: true columns U_true[j] = (column scale c_j, or KDA's Gamma per row) U_s[j] -------
  for (int idx = t; idx < m * DK; idx += 256) {
    const int j = idx / DK, d = idx - j * DK;
    const float s = DIAG ? sc[d] : sc[j < r ? 0 : 1 + j - r];
    F[j][d] = s * to_f32<FDT>(Ub[static_cast<int64_t>(j) * DK + d]);
  }
  __syncthreads();
  // a_true = (slot-0 decay, or Gamma) a_0 + sum_{j >= r} c_j U_true[j]
  for (int d = t; d < DK; d += 256) {
    float acc = (DIAG ? sc[d] : sc[0]) * A.a[unit * DK + d];
    for (int j = r; j < m; ++j) acc = fmaf(sc[A.coef_off + j - r], F[j][d], acc);
    at[d] = acc;
  }
  __syncthreads();
  float pa = 0.f;
  for (int d = t; d < DK; d += 256) pa = fmaf(at[d], at[d], pa);
  if (t < m) {
    float x = 0.f;
    for (int d = 0; d < DK; ++d) x = fmaf(F[t][d], at[d], x);
    xs[t] = x;
  }
  for (int p = t; p < npairs; p += 256) {
    int i, j;
    pair_of(p, i, j);
    float g = 0.f;
    for (int d = 0; d < DK; ++d) g = fmaf(F[i][d], F[j][d], g);
    G[i][j] = g;
  }
  __syncthreads();

  // ---- V: cross term (U^T a) . (V^T vbar) and the content sum_{i,j} G_U G_V -------------------
  for (int idx = t; idx < m * DV; idx += 256) {
    const int j = idx / DV, d = idx - j * DV;
    F[j][d] = to_f32<FDT>(Vb[static_cast<int64_t>(j) * DV + d]);
  }
  __syncthreads();
  float pv = 0.f, px = 0.f, pc = 0.f;
  for (int d = t; d < DV; d += 256) pv = fmaf(vb[d], vb[d], pv);
  if (t < m) {
    float y = 0.f;
    for (int d = 0; d < DV; ++d) y = fmaf(F[t][d], vb[d], y);
    px = xs[t] * y;
  }
  for (int p = t; p < npairs; p += 256) {
    int i, j;
    pair_of(p, i, j);
    float g = 0.f;
    for (int d = 0; d < DV; ++d) g = fmaf(F[i][d], F[j][d], g);
    pc = fmaf(i == j ? 1.f : 2.f, G[i][j] * g, pc);
  }
  const float sa = block_sum(pa, red);
  const float sv = block_sum(pv, red);
  const float cross = block_sum(px, red);
  const float content = block_sum(pc, red);
  if (t == 0) {
    const float sink = sa * sv;
    A.out[unit * 3 + 0] = sink + 2.f * cross + content;
    A.out[unit * 3 + 1] = sink;
    A.out[unit * 3 + 2] = content;
  }
}

namespace {
using EnergyFn = void (*)(const EnergyArgs);

template <int DK, int DV>
EnergyFn pick_energy_dt(int fdt, bool diag) {
  switch (fdt) {
    case SEED_F32: return diag ? k_energy<DK, DV, 0, true> : k_energy<DK, DV, 0, false>;
    case SEED_BF16: return diag ? k_energy<DK, DV, 1, true> : k_energy<DK, DV, 1, false>;
    case SEED_F16: return diag ? k_energy<DK, DV, 2, true> : k_energy<DK, DV, 2, false>;
    default: return nullptr;
  }
}

EnergyFn pick_energy(const seed_shape& sh) {
  const bool diag = sh.kind == SEED_KDA;
  if (sh.rank + sh.period > kMaxCols) return nullptr;
  if (sh.d_k == 128 && sh.d_v == 128) return pick_energy_dt<128, 128>(sh.factor_dtype, diag);
  if (sh.d_k == 128 && sh.d_v == 64) return pick_energy_dt<128, 64>(sh.factor_dtype, diag);
  if (sh.d_k == 64 && sh.d_v == 128) return pick_energy_dt<64, 128>(sh.factor_dtype, diag);
  if (sh.d_k == 64 && sh.d_v == 64) return pick_energy_dt<64, 64>(sh.factor_dtype, diag);
  return nullptr;
}
}  // namespace

hipError_t launch_energy(const seed_shape& sh, const EnergyArgs& a, hipStream_t s) {
  bool used = false;
  const hipError_t e = launch_energy_wave(sh, a, s, &used);   // 16-bit factors
  if (used) return e;
  EnergyFn fn = pick_energy(sh);
  if (!fn) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(a.units)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace seed
