// Dense-state decode step: the uncompressed baseline.
//
// Every step loads and stores the whole d_k x d_v fp32 state of every head (pages titled
// "Shallow Encoding Emits Deep Memories", picx.dev summary, "Introduction and Theoretical
// Foundation"). The recurrences are the dense forms whose factorisation is Lemma 2 (picx.dev
// summary, "Exact Update (Lemma 2)"):
//   GDN / KDA: S+ = G S + beta kappa (v - (G S)^T kappa)^T,  G = g I or Diag(alpha)
//   Mamba-2:   S+ = g S + beta kappa v^T
// and o = S+^T q.
//
// Design (gfx950): one 256-thread workgroup per unit. Each thread keeps its share of S in
// registers (64 floats at 128 x 128), so S is read from HBM exactly once and written exactly
// once. A wave-wide load covers two or four whole rows (1 KiB contiguous). The two column
// reductions S_d^T kappa and S_d^T q are summed across row groups through LDS; the rank-one
// write S_d + kappa w^T is then applied to the registers and stored.
#include "common.hpp"
#include "kernels.hpp"

namespace seed {

template <int KIND, int DK, int DV, int IDT>
__global__ __launch_bounds__(256) void k_dense(const DenseArgs A) {
  using IT = stor_t<IDT>;
  constexpr int CS = DV / 4;        // 16-byte column slices per row
  constexpr int RG = 256 / CS;      // row groups
  constexpr int RPT = DK / RG;      // rows per thread
  constexpr bool DELTA = (KIND != SEED_MAMBA2);
  constexpr bool DIAG = (KIND == SEED_KDA);
  static_assert(DK % RG == 0, "rows per thread");

  __shared__ float4 red_k[RG][CS];
  __shared__ float4 red_q[RG][CS];
  __shared__ float kq_sh;

  const int64_t unit = blockIdx.x;
  const int t = threadIdx.x;
  const int cs = t % CS, rg = t / CS;
  float4* __restrict__ Sb = reinterpret_cast<float4*>(A.S + unit * DK * DV);

  float4 Sr[RPT];
#pragma unroll
  for (int ii = 0; ii < RPT; ++ii) Sr[ii] = Sb[(rg + RG * ii) * CS + cs];

  const IT* qp = reinterpret_cast<const IT*>(A.q) + unit * DK;
  const IT* kp = reinterpret_cast<const IT*>(A.k) + unit * DK;
  const float beta = A.beta[unit];
  float gsc = 0.f;
  if constexpr (!DIAG) gsc = A.g[unit];

  // kappa . q by the first wave
  if (t < kWave) {
    float p = 0.f;
    for (int i = t; i < DK; i += kWave) p += to_f32<IDT>(kp[i]) * to_f32<IDT>(qp[i]);
    p = group_sum<64>(p);
    if (t == 0) kq_sh = p;
  }

  float4 pk = make_float4(0.f, 0.f, 0.f, 0.f), pq = pk;
  float kap[RPT];
#pragma unroll
  for (int ii = 0; ii < RPT; ++ii) {
    const int i = rg + RG * ii;
    const float gi = DIAG ? A.g[unit * DK + i] : gsc;
    float4 x = Sr[ii];
    x.x *= gi; x.y *= gi; x.z *= gi; x.w *= gi;  // S_d = G S
    Sr[ii] = x;
    const float ki = to_f32<IDT>(kp[i]);
    const float qi = to_f32<IDT>(qp[i]);
    kap[ii] = ki;
    if constexpr (DELTA) { pk.x += ki * x.x; pk.y += ki * x.y; pk.z += ki * x.z; pk.w += ki * x.w; }
    pq.x += qi * x.x; pq.y += qi * x.y; pq.z += qi * x.z; pq.w += qi * x.w;
  }
  if constexpr (DELTA) red_k[rg][cs] = pk;
  red_q[rg][cs] = pq;
  __syncthreads();

  float4 sk = make_float4(0.f, 0.f, 0.f, 0.f), sq = sk;
#pragma unroll
  for (int g2 = 0; g2 < RG; ++g2) {
    if constexpr (DELTA) {
      const float4 a = red_k[g2][cs];
      sk.x += a.x; sk.y += a.y; sk.z += a.z; sk.w += a.w;
    }
    const float4 b = red_q[g2][cs];
    sq.x += b.x; sq.y += b.y; sq.z += b.z; sq.w += b.w;
  }
  float vv[4];
  load_f32<IDT, 4>(reinterpret_cast<const IT*>(A.v) + unit * DV + 4 * cs, vv);
  // w = beta (v - S_d^T kappa) (delta kinds) or beta v (Mamba-2)
  float4 w;
  w.x = beta * (vv[0] - (DELTA ? sk.x : 0.f));
  w.y = beta * (vv[1] - (DELTA ? sk.y : 0.f));
  w.z = beta * (vv[2] - (DELTA ? sk.z : 0.f));
  w.w = beta * (vv[3] - (DELTA ? sk.w : 0.f));

#pragma unroll
  for (int ii = 0; ii < RPT; ++ii) {
    float4 x = Sr[ii];
    const float ki = kap[ii];
    x.x += ki * w.x; x.y += ki * w.y; x.z += ki * w.z; x.w += ki * w.w;
    Sb[(rg + RG * ii) * CS + cs] = x;
  }
  if (rg == 0) {
    const float kq = kq_sh;
    const float o[4] = {sq.x + kq * w.x, sq.y + kq * w.y, sq.z + kq * w.z, sq.w + kq * w.w};
    store_f32<IDT, 4>(reinterpret_cast<IT*>(A.o) + unit * DV + 4 * cs, o);
  }
}

namespace {
using DenseFn = void (*)(const DenseArgs);

template <int KIND, int DK, int DV>
DenseFn pick_io(int io) {
  return io == SEED_BF16 ? k_dense<KIND, DK, DV, 1> : k_dense<KIND, DK, DV, 0>;
}

template <int KIND>
DenseFn pick_dims(int dk, int dv, int io) {
  if (dk == 128 && dv == 128) return pick_io<KIND, 128, 128>(io);
  if (dk == 128 && dv == 64) return pick_io<KIND, 128, 64>(io);
  if (dk == 64 && dv == 128) return pick_io<KIND, 64, 128>(io);
  if (dk == 64 && dv == 64) return pick_io<KIND, 64, 64>(io);
  return nullptr;
}

DenseFn pick_dense(const seed_shape& sh) {
  switch (sh.kind) {
    case SEED_GDN: return pick_dims<SEED_GDN>(sh.d_k, sh.d_v, sh.io_dtype);
    case SEED_KDA: return pick_dims<SEED_KDA>(sh.d_k, sh.d_v, sh.io_dtype);
    case SEED_MAMBA2: return pick_dims<SEED_MAMBA2>(sh.d_k, sh.d_v, sh.io_dtype);
    default: return nullptr;
  }
}
}  // namespace

hipError_t launch_dense(const seed_shape& sh, const DenseArgs& a, hipStream_t s) {
  DenseFn fn = pick_dense(sh);
  if (!fn) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(a.units)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace seed
