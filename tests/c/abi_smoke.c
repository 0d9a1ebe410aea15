/*
 * The C ABI from plain C: a prefill-end compression, a window of decode steps, a compression
 * and a chunked update on a small GDN state (fp32 factors and inputs), through libseed.so and
 * the HIP runtime's C API only. Checks every status, that the column count in the state
 * follows the calls, and that the read-outs are finite and not all zero. Prints "abi_smoke ok".
 * Built by tests/test_c_abi.py; run there on a GPU.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "seed.h"

#define CHECK_HIP(x)                                                            \
  do {                                                                          \
    hipError_t e_ = (x);                                                        \
    if (e_ != hipSuccess) {                                                     \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
      return 1;                                                                 \
    }                                                                           \
  } while (0)
#define CHECK_SEED(x)                                                                   \
  do {                                                                                  \
    int s_ = (x);                                                                       \
    if (s_ != SEED_OK) {                                                                \
      fprintf(stderr, "%s:%d: %s (%d)\n", __FILE__, __LINE__, seed_status_string(s_), s_); \
      return 1;                                                                         \
    }                                                                                   \
  } while (0)

static uint64_t lcg = 12345u;
static float urand(void) {  /* uniform in [-1, 1) */
  lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
  return (float)((lcg >> 40) & 0xFFFFFF) / 8388608.0f - 1.0f;
}

static void *dev_from(const float *host, size_t n) {
  void *d = NULL;
  if (hipMalloc(&d, n * sizeof(float)) != hipSuccess) return NULL;
  if (hipMemcpy(d, host, n * sizeof(float), hipMemcpyHostToDevice) != hipSuccess) return NULL;
  return d;
}

int main(void) {
  seed_shape sh;
  memset(&sh, 0, sizeof sh);
  sh.kind = SEED_GDN;
  sh.batch = 2;
  sh.heads = 2;
  sh.d_k = 64;
  sh.d_v = 64;
  sh.rank = 8;
  sh.period = 8;
  sh.factor_dtype = SEED_F32;
  sh.io_dtype = SEED_F32;
  sh.rounding = SEED_ROUND_NEAREST;
  const int units = sh.batch * sh.heads, dk = sh.d_k, dv = sh.d_v, C = sh.rank + sh.period;
  const int32_t sl = seed_scale_len(&sh);
  if (sl <= 0 || seed_state_bytes(&sh) == 0) {
    fprintf(stderr, "size queries failed\n");
    return 1;
  }

  /* dense states: a strong mean direction plus noise, and the per-head direction vbar */
  float *S = malloc(sizeof(float) * units * dk * dv), *vb = malloc(sizeof(float) * sh.heads * dv);
  for (int i = 0; i < sh.heads * dv; ++i) vb[i] = 1.0f + 0.1f * urand();
  for (int u = 0; u < units; ++u)
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) S[(u * dk + i) * dv + j] = 0.5f * urand() * vb[(u % sh.heads) * dv + j] + 0.1f * urand();
  float *dS = dev_from(S, (size_t)units * dk * dv), *dvb = dev_from(vb, (size_t)sh.heads * dv);

  seed_state st;
  CHECK_HIP(hipMalloc((void **)&st.a, sizeof(float) * units * dk));
  CHECK_HIP(hipMalloc(&st.U, sizeof(float) * units * C * dk));
  CHECK_HIP(hipMalloc(&st.V, sizeof(float) * units * C * dv));
  CHECK_HIP(hipMalloc((void **)&st.scale, sizeof(float) * units * sl));
  CHECK_HIP(hipMemset(st.scale, 0, sizeof(float) * units * sl));
  CHECK_SEED(seed_state_from_dense(&sh, dS, dvb, &st, NULL, 0, NULL));

  /* one window of decode steps, then a compression */
  const int L = 4;
  float *q = malloc(sizeof(float) * units * L * dk), *k = malloc(sizeof(float) * units * L * dk);
  float *v = malloc(sizeof(float) * units * L * dv), *beta = malloc(sizeof(float) * units * L);
  float *g = malloc(sizeof(float) * units * L);
  float *dq, *dk_, *dvv, *dbeta, *dg, *dout;
  CHECK_HIP(hipMalloc((void **)&dout, sizeof(float) * units * L * dv));
  for (int m = sh.rank; m < C; ++m) {
    for (int i = 0; i < units * dk; ++i) { q[i] = 0.125f * urand(); k[i] = 0.125f * urand(); }
    for (int i = 0; i < units * dv; ++i) v[i] = urand();
    for (int i = 0; i < units; ++i) { beta[i] = 0.5f + 0.25f * urand(); g[i] = 0.95f + 0.04f * urand(); }
    dq = dev_from(q, (size_t)units * dk); dk_ = dev_from(k, (size_t)units * dk); dvv = dev_from(v, (size_t)units * dv);
    dbeta = dev_from(beta, units); dg = dev_from(g, units);
    CHECK_SEED(seed_decode_step(&sh, &st, m, dq, dk_, dvv, dbeta, dg, dvb, dout, NULL));
    CHECK_HIP(hipDeviceSynchronize());
    hipFree(dq); hipFree(dk_); hipFree(dvv); hipFree(dbeta); hipFree(dg);
  }
  CHECK_SEED(seed_compress(&sh, &st, C, NULL, 0, NULL));

  /* a chunk of L tokens: [batch][L][heads][d] inputs */
  for (int i = 0; i < units * L * dk; ++i) { q[i] = 0.125f * urand(); k[i] = 0.125f * urand(); }
  for (int i = 0; i < units * L * dv; ++i) v[i] = urand();
  for (int i = 0; i < units * L; ++i) { beta[i] = 0.5f + 0.25f * urand(); g[i] = 0.95f + 0.04f * urand(); }
  dq = dev_from(q, (size_t)units * L * dk); dk_ = dev_from(k, (size_t)units * L * dk);
  dvv = dev_from(v, (size_t)units * L * dv); dbeta = dev_from(beta, (size_t)units * L); dg = dev_from(g, (size_t)units * L);
  CHECK_SEED(seed_decode_chunk(&sh, &st, sh.rank, L, dq, dk_, dvv, dbeta, dg, dvb, dout, NULL));
  CHECK_HIP(hipDeviceSynchronize());

  float *out = malloc(sizeof(float) * units * L * dv), *sc = malloc(sizeof(float) * units * sl);
  CHECK_HIP(hipMemcpy(out, dout, sizeof(float) * units * L * dv, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(sc, st.scale, sizeof(float) * units * sl, hipMemcpyDeviceToHost));
  double norm = 0.0;
  for (int i = 0; i < units * L * dv; ++i) {
    if (!isfinite(out[i])) { fprintf(stderr, "non-finite read-out at %d\n", i); return 1; }
    norm += (double)out[i] * out[i];
  }
  if (norm == 0.0) { fprintf(stderr, "all read-outs zero\n"); return 1; }
  for (int u = 0; u < units; ++u) {
    uint32_t cnt;
    memcpy(&cnt, &sc[u * sl + sl - 1], sizeof cnt);   /* the column count, last in the scale vector */
    if (cnt != (uint32_t)(sh.rank + L)) { fprintf(stderr, "unit %d holds %u columns\n", u, cnt); return 1; }
  }
  /* an argument error is reported, not launched */
  if (seed_decode_step(&sh, &st, C, dq, dk_, dvv, dbeta, dg, dvb, dout, NULL) != SEED_ERR_ARG) return 1;
  printf("abi_smoke ok: %s\n", seed_version());
  return 0;
}
