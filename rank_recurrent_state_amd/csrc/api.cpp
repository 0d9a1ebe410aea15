// C ABI of libseed: argument validation, size queries and dispatch to the gfx950 kernels.
// Every entry point validates on the host before anything is enqueued, never synchronises and
// allocates nothing.
#include <hip/hip_runtime.h>

#include "../../include/seed.h"
#include "kernels.hpp"

namespace seed {
int32_t from_dense_iterations();
bool chunk_supported_len(const seed_shape& sh, int32_t len);  // chunk.hip: KDA takes up to 16 tokens
}

namespace {

bool dtype_ok(int32_t d) { return d == SEED_F32 || d == SEED_BF16 || d == SEED_F16; }
bool dim_ok(int32_t d) { return d == 64 || d == 128; }
size_t dt_bytes(int32_t d) { return d == SEED_F32 ? 4 : 2; }

// 0: valid; SEED_ERR_ARG: malformed; SEED_ERR_UNSUPPORTED: well formed but not compiled.
int check_shape(const seed_shape* sh) {
  if (!sh) return SEED_ERR_ARG;
  if (sh->kind != SEED_GDN && sh->kind != SEED_KDA && sh->kind != SEED_MAMBA2) return SEED_ERR_ARG;
  if (sh->batch <= 0 || sh->heads <= 0 || sh->d_k <= 0 || sh->d_v <= 0) return SEED_ERR_ARG;
  if (sh->rank <= 0 || sh->period <= 0) return SEED_ERR_ARG;
  if (!dtype_ok(sh->factor_dtype) || !dtype_ok(sh->io_dtype)) return SEED_ERR_ARG;
  if (sh->rounding != SEED_ROUND_NEAREST && sh->rounding != SEED_ROUND_STOCHASTIC) return SEED_ERR_ARG;
  // stochastic rounding applies to the 16-bit factor formats
  if (sh->rounding == SEED_ROUND_STOCHASTIC && sh->factor_dtype == SEED_F32) return SEED_ERR_ARG;
  if (sh->io_dtype == SEED_F16) return SEED_ERR_UNSUPPORTED;  // fp16 is a factor format only
  if (!dim_ok(sh->d_k) || !dim_ok(sh->d_v)) return SEED_ERR_UNSUPPORTED;
  if (sh->rank + sh->period > 64) return SEED_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(sh->batch) * sh->heads > (int64_t{1} << 31) - 1) return SEED_ERR_UNSUPPORTED;
  return SEED_OK;
}

int64_t units_of(const seed_shape* sh) { return static_cast<int64_t>(sh->batch) * sh->heads; }

// Per-unit scale buffer: the lazy decay scales (1 + T slot scales, or KDA's d_k channel scales),
// then the T sink coefficients of the window's columns.
int32_t coef_off(const seed_shape* sh) {
  return sh->kind == SEED_KDA ? sh->d_k : 1 + sh->period;
}

// decay scales, T sink coefficients, the compression-window count, the column count
int32_t scale_len(const seed_shape* sh) { return coef_off(sh) + sh->period + 2; }

bool state_ok(const seed_state* st) {
  return st && st->a && st->U && st->V && st->scale;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SEED_OK : SEED_ERR_HIP; }

seed::CompressArgs compress_args(const seed_shape* sh, const seed_state* st, int32_t m) {
  seed::CompressArgs a{};
  a.units = units_of(sh);
  a.heads = sh->heads;
  a.m = m;
  a.rank = sh->rank;
  a.slots = sh->rank + sh->period;
  a.scale_len = scale_len(sh);
  a.coef_off = coef_off(sh);
  a.win_off = coef_off(sh) + sh->period;
  a.m_off = a.win_off + 1;
  a.rounding = sh->rounding;
  a.rng_key = sh->rng_key;
  a.ragged = 0;
  a.a = st->a;
  a.U = st->U;
  a.V = st->V;
  a.scale = st->scale;
  a.S = nullptr;
  a.vbar = nullptr;
  a.iters = seed::from_dense_iterations();
  return a;
}

// The decode step's arguments; ragged calls take every unit's m from its state.
seed::StepArgs step_args(const seed_shape* sh, const seed_state* st, int32_t m, const uint8_t* active,
                         bool ragged) {
  seed::StepArgs a{};
  a.units = units_of(sh);
  a.heads = sh->heads;
  a.m = m;
  a.rank = sh->rank;
  a.slots = sh->rank + sh->period;
  a.scale_len = scale_len(sh);
  a.coef_off = coef_off(sh);
  a.win_off = coef_off(sh) + sh->period;
  a.m_off = a.win_off + 1;
  a.rounding = sh->rounding;
  a.rng_key = sh->rng_key;
  a.ragged = ragged ? 1 : 0;
  a.active = active;
  a.a = st->a;
  a.U = st->U;
  a.V = st->V;
  a.scale = st->scale;
  return a;
}

int decode_call(const seed_shape* sh, const seed_state* st, int32_t m, const uint8_t* active, bool ragged,
                const void* q, const void* k, const void* v, const float* beta, const float* g,
                const float* vbar, void* o, void* stream, const seed_head_norm* norm = nullptr,
                bool normed = false) {
  const int c = check_shape(sh);
  if (c != SEED_OK) return c;
  if (!state_ok(st) || !q || !k || !v || !beta || !g || !vbar || !o) return SEED_ERR_ARG;
  if (normed && (!norm || !norm->weight || !(norm->eps >= 0.f) || !(norm->eps < 3.0e38f) ||
                 (norm->gate_first != 0 && norm->gate_first != 1)))
    return SEED_ERR_ARG;
  if (!ragged && (m < sh->rank || m >= sh->rank + sh->period)) return SEED_ERR_ARG;
  if (!seed::decode_supported(*sh)) return SEED_ERR_UNSUPPORTED;
  seed::StepArgs a = step_args(sh, st, m, active, ragged);
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.g = g;
  a.vbar = vbar;
  a.o = o;
  if (normed) {
    a.norm_w = norm->weight;
    a.norm_gate = norm->gate;
    a.norm_eps = norm->eps;
    a.norm_gate_first = norm->gate_first;
  }
  return hip_status(seed::launch_decode(*sh, a, static_cast<hipStream_t>(stream)));
}

int compress_call(const seed_shape* sh, const seed_state* st, int32_t m, bool ragged, void* ws,
                  size_t ws_bytes, void* stream) {
  const int c = check_shape(sh);
  if (c != SEED_OK) return c;
  if (!state_ok(st)) return SEED_ERR_ARG;
  if (ragged ? (m <= sh->rank || m > sh->rank + sh->period) : (m < 0 || m > sh->rank + sh->period))
    return SEED_ERR_ARG;
  if (ws_bytes < seed_workspace_bytes(sh, SEED_OP_COMPRESS)) return SEED_ERR_WORKSPACE;
  (void)ws;
  if (!seed::compress_supported(*sh)) return SEED_ERR_UNSUPPORTED;
  if (!ragged && m <= sh->rank) return SEED_OK;
  seed::CompressArgs a = compress_args(sh, st, m);
  a.ragged = ragged ? 1 : 0;
  return hip_status(seed::launch_compress(*sh, a, static_cast<hipStream_t>(stream)));
}

int chunk_call(const seed_shape* sh, const seed_state* st, int32_t m, const uint8_t* active, bool ragged,
               int32_t len, const void* q, const void* k, const void* v, const float* beta, const float* g,
               const float* vbar, void* o, void* stream) {
  const int c = check_shape(sh);
  if (c != SEED_OK) return c;
  if (!state_ok(st) || !q || !k || !v || !beta || !g || !vbar || !o) return SEED_ERR_ARG;
  if (len < 1 || len > seed::chunk_max_tokens()) return SEED_ERR_ARG;
  if (!ragged && (m < sh->rank || m + len > sh->rank + sh->period)) return SEED_ERR_ARG;
  if (len > sh->period) return SEED_ERR_ARG;
  if (!seed::chunk_supported_len(*sh, len)) return SEED_ERR_UNSUPPORTED;
  seed::StepArgs a = step_args(sh, st, m, active, ragged);
  a.len = len;
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.g = g;
  a.vbar = vbar;
  a.o = o;
  return hip_status(seed::launch_decode_chunk(*sh, a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

size_t seed_state_bytes(const seed_shape* sh) {
  if (check_shape(sh) != SEED_OK) return 0;
  const size_t slots = static_cast<size_t>(sh->rank + sh->period);
  const size_t f = dt_bytes(sh->factor_dtype);
  return 4 * static_cast<size_t>(sh->d_k) + f * slots * (sh->d_k + sh->d_v) +
         4 * static_cast<size_t>(scale_len(sh));
}

int32_t seed_scale_len(const seed_shape* sh) {
  if (check_shape(sh) != SEED_OK) return 0;
  return scale_len(sh);
}

size_t seed_workspace_bytes(const seed_shape* sh, int32_t op) {
  (void)sh;
  (void)op;
  return 0;  // both operations keep their intermediates in LDS
}

int32_t seed_from_dense_iterations(void) { return seed::from_dense_iterations(); }

int seed_state_from_dense(const seed_shape* sh, const float* S, const float* vbar,
                          const seed_state* st, void* ws, size_t ws_bytes, void* stream) {
  const int c = check_shape(sh);
  if (c != SEED_OK) return c;
  if (!S || !vbar || !state_ok(st)) return SEED_ERR_ARG;
  if (ws_bytes < seed_workspace_bytes(sh, SEED_OP_FROM_DENSE)) return SEED_ERR_WORKSPACE;
  (void)ws;
  seed::CompressArgs a = compress_args(sh, st, sh->rank);
  a.S = S;
  a.vbar = vbar;
  return hip_status(seed::launch_from_dense(*sh, a, static_cast<hipStream_t>(stream)));
}

int seed_decode_step(const seed_shape* sh, const seed_state* st, int32_t m, const void* q,
                     const void* k, const void* v, const float* beta, const float* g,
                     const float* vbar, void* o, void* stream) {
  return decode_call(sh, st, m, nullptr, false, q, k, v, beta, g, vbar, o, stream);
}

int seed_decode_step_normed(const seed_shape* sh, const seed_state* st, int32_t m, const void* q,
                            const void* k, const void* v, const float* beta, const float* g,
                            const float* vbar, const seed_head_norm* norm, void* o, void* stream) {
  return decode_call(sh, st, m, nullptr, false, q, k, v, beta, g, vbar, o, stream, norm, true);
}

int seed_decode_step_ragged_normed(const seed_shape* sh, const seed_state* st, const uint8_t* active,
                                   const void* q, const void* k, const void* v, const float* beta,
                                   const float* g, const float* vbar, const seed_head_norm* norm, void* o,
                                   void* stream) {
  return decode_call(sh, st, 0, active, true, q, k, v, beta, g, vbar, o, stream, norm, true);
}

int seed_decode_step_ragged(const seed_shape* sh, const seed_state* st, const uint8_t* active,
                            const void* q, const void* k, const void* v, const float* beta,
                            const float* g, const float* vbar, void* o, void* stream) {
  return decode_call(sh, st, 0, active, true, q, k, v, beta, g, vbar, o, stream);
}


int seed_decode_chunk(const seed_shape* sh, const seed_state* st, int32_t m, int32_t len, const void* q,
                      const void* k, const void* v, const float* beta, const float* g, const float* vbar,
                      void* o, void* stream) {
  return chunk_call(sh, st, m, nullptr, false, len, q, k, v, beta, g, vbar, o, stream);
}

int seed_decode_chunk_ragged(const seed_shape* sh, const seed_state* st, const uint8_t* active, int32_t len,
                             const void* q, const void* k, const void* v, const float* beta, const float* g,
                             const float* vbar, void* o, void* stream) {
  return chunk_call(sh, st, 0, active, true, len, q, k, v, beta, g, vbar, o, stream);
}

int32_t seed_chunk_max_tokens(void) { return seed::chunk_max_tokens(); }

int seed_compress_ragged(const seed_shape* sh, const seed_state* st, int32_t min_m, void* ws,
                         size_t ws_bytes, void* stream) {
  return compress_call(sh, st, min_m, true, ws, ws_bytes, stream);
}

int seed_compress_units(const seed_shape* sh, const seed_state* st, const int32_t* units, int32_t count,
                        void* ws, size_t ws_bytes, void* stream) {
  const int c = check_shape(sh);
  if (c != SEED_OK) return c;
  if (!state_ok(st) || count < 0 || (count > 0 && !units)) return SEED_ERR_ARG;
  if (ws_bytes < seed_workspace_bytes(sh, SEED_OP_COMPRESS)) return SEED_ERR_WORKSPACE;
  (void)ws;
  if (!seed::compress_supported(*sh)) return SEED_ERR_UNSUPPORTED;
  if (count == 0) return SEED_OK;
  seed::CompressArgs a = compress_args(sh, st, sh->rank + 1);
  a.ragged = 1;  // each listed unit at its own column count, when it holds columns beyond r
  a.list = units;
  a.list_len = count;
  return hip_status(seed::launch_compress(*sh, a, static_cast<hipStream_t>(stream)));
}

int seed_compress(const seed_shape* sh, const seed_state* st, int32_t m, void* ws, size_t ws_bytes,
                  void* stream) {
  return compress_call(sh, st, m, false, ws, ws_bytes, stream);
}

int seed_state_energy(const seed_shape* sh, const seed_state* st, const float* vbar, float* out,
                      void* stream) {
  const int c = check_shape(sh);
  if (c != SEED_OK) return c;
  if (!state_ok(st) || !vbar || !out) return SEED_ERR_ARG;
  seed::EnergyArgs a{};
  a.units = units_of(sh);
  a.heads = sh->heads;
  a.rank = sh->rank;
  a.slots = sh->rank + sh->period;
  a.scale_len = scale_len(sh);
  a.coef_off = coef_off(sh);
  a.m_off = coef_off(sh) + sh->period + 1;
  a.a = st->a;
  a.U = st->U;
  a.V = st->V;
  a.scale = st->scale;
  a.vbar = vbar;
  a.out = out;
  return hip_status(seed::launch_energy(*sh, a, static_cast<hipStream_t>(stream)));
}

int seed_state_spectrum(const seed_shape* sh, const seed_state* st, float* out, void* stream) {
  const int c = check_shape(sh);
  if (c != SEED_OK) return c;
  if (!state_ok(st) || !out) return SEED_ERR_ARG;
  // the one-wavefront compression kernel's eigen phase: 16-bit factors, r <= 32
  if (sh->factor_dtype == SEED_F32 || sh->rank > SEED_SPECTRUM_LEN - 1) return SEED_ERR_UNSUPPORTED;
  seed::CompressArgs a = compress_args(sh, st, 0);
  a.spectrum = out;
  return hip_status(seed::launch_spectrum(*sh, a, static_cast<hipStream_t>(stream)));
}

int seed_dense_decode_step(const seed_shape* sh, float* S, const void* q, const void* k,
                           const void* v, const float* beta, const float* g, void* o,
                           void* stream) {
  const int c = check_shape(sh);
  if (c != SEED_OK) return c;
  if (!S || !q || !k || !v || !beta || !g || !o) return SEED_ERR_ARG;
  seed::DenseArgs a{};
  a.units = units_of(sh);
  a.S = S;
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.g = g;
  a.o = o;
  return hip_status(seed::launch_dense(*sh, a, static_cast<hipStream_t>(stream)));
}

int seed_stream_create_cu_masked(uint32_t mask_words, const uint32_t* cu_mask, void** stream) {
  if (!stream || !cu_mask || mask_words == 0 || mask_words > 64) return SEED_ERR_ARG;
  *stream = nullptr;
  uint32_t any = 0;
  for (uint32_t i = 0; i < mask_words; ++i) any |= cu_mask[i];
  if (any == 0) return SEED_ERR_ARG;
  hipStream_t s = nullptr;
  if (hipExtStreamCreateWithCUMask(&s, mask_words, cu_mask) != hipSuccess) {
    (void)hipGetLastError();
    return SEED_ERR_HIP;
  }
  *stream = s;
  return SEED_OK;
}

int seed_stream_destroy(void* stream) {
  if (!stream) return SEED_ERR_ARG;
  return hip_status(hipStreamDestroy(static_cast<hipStream_t>(stream)));
}

const char* seed_status_string(int status) {
  switch (status) {
    case SEED_OK: return "ok";
    case SEED_ERR_ARG: return "invalid argument";
    case SEED_ERR_UNSUPPORTED: return "shape or dtype not supported by this build";
    case SEED_ERR_WORKSPACE: return "workspace missing or too small";
    case SEED_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

const char* seed_version(void) { return "libseed 0.1 (gfx950)"; }

}  // extern "C"
