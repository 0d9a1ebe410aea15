/*
 * Host-side validation of the C ABI, built with AddressSanitizer and UndefinedBehaviorSanitizer
 * against the ABI's own source (api.cpp) and launcher stand-ins (launch_stubs.cpp) by
 * tests/test_abi_sanitize.py. No GPU is used: every device pointer is a stand-in that the ABI
 * must reject or pass on without reading. Checks that each entry point returns the documented
 * status for malformed calls and launches nothing, that well-formed calls reach exactly one
 * launcher, and that the size queries agree with the state layout. Prints "abi_validate ok".
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "seed.h"

extern int seed_stub_launches;

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)
/* a malformed call: the status, and no launch */
#define REJECT(call, status)                        \
  do {                                              \
    int before_ = seed_stub_launches;               \
    int s_ = (call);                                \
    EXPECT(s_ == (status));                         \
    EXPECT(seed_stub_launches == before_);          \
  } while (0)
/* a well-formed call: OK and exactly one launch */
#define ACCEPT(call)                                \
  do {                                              \
    int before_ = seed_stub_launches;               \
    int s_ = (call);                                \
    EXPECT(s_ == SEED_OK);                          \
    EXPECT(seed_stub_launches == before_ + 1);      \
  } while (0)

static seed_shape shape(int kind, int fdt, int idt) {
  seed_shape sh;
  memset(&sh, 0, sizeof sh);
  sh.kind = kind;
  sh.batch = 4;
  sh.heads = 2;
  sh.d_k = 128;
  sh.d_v = 128;
  sh.rank = 16;
  sh.period = 16;
  sh.factor_dtype = fdt;
  sh.io_dtype = idt;
  sh.rounding = SEED_ROUND_NEAREST;
  return sh;
}

int main(void) {
  /* stand-in device pointers: never dereferenced on the host */
  void *p = (void *)(uintptr_t)0x1000;
  float *fp = (float *)p;
  seed_state st = {fp, p, p, fp};
  seed_state nost = {NULL, p, p, fp};
  seed_shape sh = shape(SEED_GDN, SEED_BF16, SEED_BF16);

  /* size queries */
  EXPECT(seed_scale_len(&sh) == 1 + 16 + 16 + 2);
  EXPECT(seed_state_bytes(&sh) == 4 * 128 + 2 * 32 * 256 + 4 * 35);
  EXPECT(seed_workspace_bytes(&sh, SEED_OP_COMPRESS) == 0);
  EXPECT(seed_state_bytes(NULL) == 0 && seed_scale_len(NULL) == 0);
  {
    seed_shape bad = sh;
    bad.d_k = 96;
    EXPECT(seed_state_bytes(&bad) == 0);
    bad = sh;
    bad.rank = 40;
    bad.period = 40;
    EXPECT(seed_scale_len(&bad) == 0);
  }
  EXPECT(strlen(seed_status_string(SEED_ERR_ARG)) > 0 && strlen(seed_status_string(12345)) > 0);
  EXPECT(strstr(seed_version(), "libseed") != NULL);

  /* decode step */
  ACCEPT(seed_decode_step(&sh, &st, 16, p, p, p, fp, fp, fp, p, NULL));
  REJECT(seed_decode_step(NULL, &st, 16, p, p, p, fp, fp, fp, p, NULL), SEED_ERR_ARG);
  REJECT(seed_decode_step(&sh, NULL, 16, p, p, p, fp, fp, fp, p, NULL), SEED_ERR_ARG);
  REJECT(seed_decode_step(&sh, &nost, 16, p, p, p, fp, fp, fp, p, NULL), SEED_ERR_ARG);
  REJECT(seed_decode_step(&sh, &st, 15, p, p, p, fp, fp, fp, p, NULL), SEED_ERR_ARG);
  REJECT(seed_decode_step(&sh, &st, 32, p, p, p, fp, fp, fp, p, NULL), SEED_ERR_ARG);
  REJECT(seed_decode_step(&sh, &st, 16, NULL, p, p, fp, fp, fp, p, NULL), SEED_ERR_ARG);
  REJECT(seed_decode_step(&sh, &st, 16, p, p, p, fp, fp, NULL, p, NULL), SEED_ERR_ARG);
  REJECT(seed_decode_step(&sh, &st, 16, p, p, p, fp, fp, fp, NULL, NULL), SEED_ERR_ARG);
  {
    seed_shape b = sh;
    b.kind = 7;
    REJECT(seed_decode_step(&b, &st, 16, p, p, p, fp, fp, fp, p, NULL), SEED_ERR_ARG);
    b = sh;
    b.batch = 0;
    REJECT(seed_decode_step(&b, &st, 16, p, p, p, fp, fp, fp, p, NULL), SEED_ERR_ARG);
    b = sh;
    b.batch = 1 << 20;
    b.heads = 1 << 12;  /* more than 2^31 units */
    REJECT(seed_decode_step(&b, &st, 16, p, p, p, fp, fp, fp, p, NULL), SEED_ERR_UNSUPPORTED);
    b = sh;
    b.d_v = 96;
    REJECT(seed_decode_step(&b, &st, 16, p, p, p, fp, fp, fp, p, NULL), SEED_ERR_UNSUPPORTED);
    b = sh;
    b.rank = 40;
    b.period = 30;
    REJECT(seed_decode_step(&b, &st, 40, p, p, p, fp, fp, fp, p, NULL), SEED_ERR_UNSUPPORTED);
    b = sh;
    b.io_dtype = SEED_F16;
    REJECT(seed_decode_step(&b, &st, 16, p, p, p, fp, fp, fp, p, NULL), SEED_ERR_UNSUPPORTED);
    b = sh;
    b.factor_dtype = 9;
    REJECT(seed_decode_step(&b, &st, 16, p, p, p, fp, fp, fp, p, NULL), SEED_ERR_ARG);
    b = shape(SEED_GDN, SEED_F32, SEED_F32);
    b.rounding = SEED_ROUND_STOCHASTIC;   /* stochastic rounding of fp32 factors */
    REJECT(seed_decode_step(&b, &st, 16, p, p, p, fp, fp, fp, p, NULL), SEED_ERR_ARG);
    b.rounding = 2;
    REJECT(seed_decode_step(&b, &st, 16, p, p, p, fp, fp, fp, p, NULL), SEED_ERR_ARG);
  }
  ACCEPT(seed_decode_step_ragged(&sh, &st, NULL, p, p, p, fp, fp, fp, p, NULL));
  REJECT(seed_decode_step_ragged(&sh, &st, NULL, p, p, NULL, fp, fp, fp, p, NULL), SEED_ERR_ARG);

  /* the normed decode step */
  {
    seed_head_norm nrm = {fp, NULL, 1e-6f, 0};
    ACCEPT(seed_decode_step_normed(&sh, &st, 16, p, p, p, fp, fp, fp, &nrm, p, NULL));
    ACCEPT(seed_decode_step_ragged_normed(&sh, &st, NULL, p, p, p, fp, fp, fp, &nrm, p, NULL));
    REJECT(seed_decode_step_normed(&sh, &st, 16, p, p, p, fp, fp, fp, NULL, p, NULL), SEED_ERR_ARG);
    nrm.weight = NULL;
    REJECT(seed_decode_step_normed(&sh, &st, 16, p, p, p, fp, fp, fp, &nrm, p, NULL), SEED_ERR_ARG);
    nrm.weight = fp;
    nrm.eps = -1.0f;
    REJECT(seed_decode_step_normed(&sh, &st, 16, p, p, p, fp, fp, fp, &nrm, p, NULL), SEED_ERR_ARG);
    nrm.eps = NAN;
    REJECT(seed_decode_step_normed(&sh, &st, 16, p, p, p, fp, fp, fp, &nrm, p, NULL), SEED_ERR_ARG);
    nrm.eps = INFINITY;
    REJECT(seed_decode_step_normed(&sh, &st, 16, p, p, p, fp, fp, fp, &nrm, p, NULL), SEED_ERR_ARG);
    nrm.eps = 1e-6f;
    nrm.gate_first = 3;
    REJECT(seed_decode_step_normed(&sh, &st, 16, p, p, p, fp, fp, fp, &nrm, p, NULL), SEED_ERR_ARG);
  }

  /* compression */
  ACCEPT(seed_compress(&sh, &st, 32, NULL, 0, NULL));
  {
    int before = seed_stub_launches;
    EXPECT(seed_compress(&sh, &st, 16, NULL, 0, NULL) == SEED_OK);   /* m <= r: nothing to do */
    EXPECT(seed_stub_launches == before);
  }
  REJECT(seed_compress(&sh, &st, 33, NULL, 0, NULL), SEED_ERR_ARG);
  REJECT(seed_compress(&sh, &st, -1, NULL, 0, NULL), SEED_ERR_ARG);
  REJECT(seed_compress(&sh, &nost, 32, NULL, 0, NULL), SEED_ERR_ARG);
  ACCEPT(seed_compress_ragged(&sh, &st, 32, NULL, 0, NULL));
  REJECT(seed_compress_ragged(&sh, &st, 16, NULL, 0, NULL), SEED_ERR_ARG);
  REJECT(seed_compress_ragged(&sh, &st, 33, NULL, 0, NULL), SEED_ERR_ARG);
  {
    const int32_t *units = (const int32_t *)p;
    ACCEPT(seed_compress_units(&sh, &st, units, 5, NULL, 0, NULL));
    int before = seed_stub_launches;
    EXPECT(seed_compress_units(&sh, &st, units, 0, NULL, 0, NULL) == SEED_OK);
    EXPECT(seed_stub_launches == before);
    REJECT(seed_compress_units(&sh, &st, NULL, 5, NULL, 0, NULL), SEED_ERR_ARG);
    REJECT(seed_compress_units(&sh, &st, units, -1, NULL, 0, NULL), SEED_ERR_ARG);
  }

  /* prefill-end compression, dense step, chunk, diagnostics */
  ACCEPT(seed_state_from_dense(&sh, fp, fp, &st, NULL, 0, NULL));
  REJECT(seed_state_from_dense(&sh, NULL, fp, &st, NULL, 0, NULL), SEED_ERR_ARG);
  REJECT(seed_state_from_dense(&sh, fp, NULL, &st, NULL, 0, NULL), SEED_ERR_ARG);
  ACCEPT(seed_dense_decode_step(&sh, fp, p, p, p, fp, fp, p, NULL));
  REJECT(seed_dense_decode_step(&sh, NULL, p, p, p, fp, fp, p, NULL), SEED_ERR_ARG);
  ACCEPT(seed_decode_chunk(&sh, &st, 16, 8, p, p, p, fp, fp, fp, p, NULL));
  REJECT(seed_decode_chunk(&sh, &st, 16, 0, p, p, p, fp, fp, fp, p, NULL), SEED_ERR_ARG);
  REJECT(seed_decode_chunk(&sh, &st, 16, 33, p, p, p, fp, fp, fp, p, NULL), SEED_ERR_ARG);
  REJECT(seed_decode_chunk(&sh, &st, 28, 8, p, p, p, fp, fp, fp, p, NULL), SEED_ERR_ARG);  /* no room */
  REJECT(seed_decode_chunk(&sh, &st, 16, 17, p, p, p, fp, fp, fp, p, NULL), SEED_ERR_ARG); /* len > T */
  {
    seed_shape k = shape(SEED_KDA, SEED_BF16, SEED_BF16);
    k.period = 32;
    REJECT(seed_decode_chunk(&k, &st, 16, 20, p, p, p, fp, fp, fp, p, NULL), SEED_ERR_UNSUPPORTED);
  }
  ACCEPT(seed_decode_chunk_ragged(&sh, &st, NULL, 8, p, p, p, fp, fp, fp, p, NULL));
  ACCEPT(seed_state_energy(&sh, &st, fp, fp, NULL));
  REJECT(seed_state_energy(&sh, &st, NULL, fp, NULL), SEED_ERR_ARG);
  ACCEPT(seed_state_spectrum(&sh, &st, fp, NULL));
  {
    seed_shape f = shape(SEED_GDN, SEED_F32, SEED_F32);
    REJECT(seed_state_spectrum(&f, &st, fp, NULL), SEED_ERR_UNSUPPORTED);
  }

  /* stream helpers: argument errors before any runtime call */
  {
    void *s = p;
    uint32_t mask = 1u, zero = 0u;
    EXPECT(seed_stream_create_cu_masked(1, NULL, &s) == SEED_ERR_ARG);
    EXPECT(seed_stream_create_cu_masked(0, &mask, &s) == SEED_ERR_ARG);
    EXPECT(seed_stream_create_cu_masked(65, &mask, &s) == SEED_ERR_ARG);
    EXPECT(seed_stream_create_cu_masked(1, &zero, &s) == SEED_ERR_ARG);
    EXPECT(seed_stream_create_cu_masked(1, &mask, NULL) == SEED_ERR_ARG);
    EXPECT(seed_stream_destroy(NULL) == SEED_ERR_ARG);
  }

  if (failures) {
    fprintf(stderr, "abi_validate: %d failures\n", failures);
    return 1;
  }
  printf("abi_validate ok (%d launches reached)\n", seed_stub_launches);
  return 0;
}
