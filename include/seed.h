/*
 * seed.h - C ABI of the sink + rank-r recurrent decode state library (libseed.so, gfx950).
 *
 * Method (pages titled "Shallow Encoding Emits Deep Memories"):
 *   - picx.dev summary, "SEED Architecture": each linear-attention / state-space head's
 *     d_k x d_v recurrent state is held as S = a vbar^T + U V^T, where vbar (d_v) is a fixed
 *     per-head direction, a (d_k) is the sink coefficient and U (d_k x m), V (d_v x m) are
 *     content factors with r <= m <= r + T columns.
 *   - picx.dev summary, "Exact Update (Lemma 2)": one decode step decays and projects a,
 *     decays U and appends one column to each factor, exactly.
 *   - thelatestinai.com figures & tables, overview table: the read-out and the update work on
 *     the factors, and a compression brings them back to rank r every T steps; a state that
 *     leaves the prefill is brought to the sink + rank-r form once.
 *
 * Kinds. kind selects the recurrence; the arguments map as
 *     kind            g (decay)                 beta      kappa (key)   v (value)   q (query)
 *     SEED_GDN        alpha, one per unit       beta      k             v           q
 *     SEED_KDA        alpha, d_k per unit       beta      k             v           q
 *     SEED_MAMBA2     exp(dt*A), one per unit   dt        B             x           C
 * with the dense recurrences
 *     GDN / KDA:  S+ = G S + beta kappa (v - (G S)^T kappa)^T,   G = g I or Diag(alpha)
 *     Mamba-2:    S+ = g S + beta kappa v^T
 * and the read-out o = S+^T q after the update.
 *
 * Conventions (every entry point):
 *   - Units. A call processes units = batch * heads independent (request, head) states, unit
 *     u = b * heads + h. Per-head constants (vbar) are indexed by h = u % heads. A layer stack
 *     is driven with one call per layer.
 *   - Memory. Every pointer is a device pointer owned by the caller. The library allocates
 *     nothing, keeps no pointer after a call returns and holds no mutable global state.
 *   - Streams. stream is a hipStream_t (NULL = the null stream). Every call only enqueues work
 *     on it and never synchronises. Calls on different streams that touch disjoint buffers may
 *     run concurrently.
 *   - Errors. Functions return SEED_OK (0) or a negative status. Argument errors are detected
 *     on the host before anything is launched, and then nothing is written. SEED_ERR_HIP
 *     reports a launch failure from the HIP runtime. Device-side faults surface, as with any
 *     HIP kernel, at the next synchronising call. seed_status_string() names a status.
 *   - Column count m. The caller keeps m (uniform over the batch): seed_state_from_dense
 *     leaves m = r; seed_decode_step takes m (r <= m < r + T) and leaves m + 1;
 *     seed_compress takes m and leaves r (nothing is done when m <= r).
 *   - Data types. factor_dtype selects the storage of U and V: fp32, or bf16 or IEEE fp16, both
 *     rounded to nearest-even (the reduced-precision factor formats of the pages' appendix
 *     table on number formats and rounding); io_dtype the storage of q, k, v and o. The factor /
 *     io pairs are fp32 / fp32, bf16 / bf16 and fp16 / bf16. a, scale, beta, g, vbar and dense
 *     states are always fp32. Arithmetic is fp32 throughout. With fp16 factors, KDA folds a key
 *     channel's cumulative gate into the stored columns once it falls below 2^-12 (2^-40 for
 *     the other formats), so that the stored key kappa / Gamma stays within fp16's range;
 *     values beyond that range (65504) are not checked and become infinities.
 *   - Rounding. rounding selects how the 16-bit factor stores round (the appendix table on number
 *     formats and rounding measures both): SEED_ROUND_NEAREST (nearest, ties to even) or
 *     SEED_ROUND_STOCHASTIC, which rounds x away from zero with probability equal to its
 *     fractional distance f between the format's two neighbouring values: exactly when the
 *     element's 16-bit draw r satisfies r < 65536 f. The draws come from Philox4x32-10 (Salmon et
 *     al., SC'11) with key (rng_key, 0) and counter (element / 8, site << 16 | aux << 8 | slot,
 *     unit, window); element e of the group of 8 takes half e % 2 of output word (e % 8) / 2.
 *     site: 0 the decode step's U column, 1 its V column, 2 / 3 a compression's U' / V',
 *     4 / 5 the prefill-end U / V, 6 a KDA gate fold rewriting a U column during the decode step
 *     with m columns (aux = m; 0 elsewhere). unit is the index within the call's own batch, and
 *     window the unit's compression-window count (below), so that every store of a trajectory
 *     draws fresh bits; states that share unit indices and windows (layers, say) should take
 *     different keys. Stochastic rounding with fp32 factors is SEED_ERR_ARG.
 *   - Supported shapes: d_k, d_v in {64, 128}; rank >= 1, period >= 1, rank + period <= 64.
 *     Other shapes return SEED_ERR_UNSUPPORTED.
 */
#ifndef SEED_H
#define SEED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SEED_OK = 0,
  SEED_ERR_ARG = -1,          /* null pointer, bad m, non-positive size, unknown enum       */
  SEED_ERR_UNSUPPORTED = -2,  /* shape or dtype not compiled into this library             */
  SEED_ERR_WORKSPACE = -3,    /* workspace pointer null or smaller than seed_workspace_bytes */
  SEED_ERR_HIP = -4           /* the HIP runtime refused a launch                          */
};

enum { SEED_GDN = 0, SEED_KDA = 1, SEED_MAMBA2 = 2 };
enum { SEED_F32 = 0, SEED_BF16 = 1, SEED_F16 = 2 };
enum { SEED_ROUND_NEAREST = 0, SEED_ROUND_STOCHASTIC = 1 };
enum { SEED_OP_COMPRESS = 0, SEED_OP_FROM_DENSE = 1 };

typedef struct seed_shape {
  int32_t kind;          /* SEED_GDN, SEED_KDA or SEED_MAMBA2                                */
  int32_t batch, heads;  /* units = batch * heads                                            */
  int32_t d_k, d_v;      /* d_k: key side (Mamba-2 d_state), the side of a; d_v: value side   */
  int32_t rank, period;  /* r and T: compression back to r columns every T steps             */
  int32_t factor_dtype;  /* SEED_F32, SEED_BF16 or SEED_F16: storage of U and V              */
  int32_t io_dtype;      /* SEED_F32 or SEED_BF16: storage of q, k, v and o                  */
  int32_t rounding;      /* SEED_ROUND_NEAREST or SEED_ROUND_STOCHASTIC: factor stores        */
  uint32_t rng_key;      /* key of the stochastic-rounding draws (ignored when nearest)       */
} seed_shape;

/*
 * Factored state. With C = r + T column slots per unit, s = seed_scale_len(shape) and
 * s0 = 1 + T (GDN, Mamba-2) or d_k (KDA):
 *   a      float [units][d_k]      sink at the last compression (a_0).
 *   U      [units][C][d_k]         slot j holds column j of U, contiguous over d_k (factor_dtype).
 *   V      [units][C][d_v]         slot j holds column j of V, contiguous over d_v (factor_dtype).
 *   scale  float [units][s]        s = s0 + T + 2: the lazy decay of U (scale[0 .. s0)), so that U
 *          is never rewritten by a decay, then the sink coefficients c (scale[s0 .. s0 + T)), then
 *          the compression-window count (scale[s0 + T]) and the unit's column count m
 *          (scale[s0 + T + 1]), both the bits of a uint32:
 *            GDN, Mamba-2: the true column j of U is scale[0] * U[j] for j < r and
 *              scale[1 + j - r] * U[j] for j >= r; the true sink is
 *              a_true = scale[0] * a + sum_{r <= j < m} c[j - r] * U_true[:, j].
 *            KDA: the true column j of U is scale[0 .. d_k) (elementwise, per key channel) times
 *              U[j], for every j; a_true = scale[0 .. d_k) . (a + sum_{r <= j < m} c[j - r] U[j]).
 *          The sink is thus kept lazily like the decay: a decode step appends the new column's
 *          coefficient instead of rewriting a. seed_state_from_dense and seed_compress leave
 *          a = a_true, the decay scales at 1 and the coefficients at 0; seed_state_from_dense
 *          sets the window count to 0 and every compression that runs adds one. Every call
 *          keeps the column count: r after seed_state_from_dense and a compression, one more
 *          after each decode step.
 * The true state is a_true vbar^T + sum_{j<m} U_true[:, j] V[:, j]^T.
 */
typedef struct seed_state {
  float *a;
  void *U;
  void *V;
  float *scale;
} seed_state;

/* Bytes of one unit's state buffers for this shape (a + U + V + scale, all C slots), or 0 if
 * the shape is invalid. Host-only, pure. */
size_t seed_state_bytes(const seed_shape *shape);

/* Length s of one unit's scale vector (decay scales 1 + T, or d_k for KDA, then T sink
 * coefficients), or 0 if the shape is invalid. */
int32_t seed_scale_len(const seed_shape *shape);

/* Workspace bytes that an operation needs (op = SEED_OP_COMPRESS or SEED_OP_FROM_DENSE);
 * 0 means the operation needs none. Host-only, pure. */
size_t seed_workspace_bytes(const seed_shape *shape, int32_t op);

/*
 * Prefill-end compression of dense states into the factored form (leaves m = r).
 *   S      float [units][d_k][d_v] dense states, row i = key channel i (read only).
 *   vbar   float [heads][d_v], every row non-zero (only its direction matters).
 *   state  written: a = S vbar / |vbar|^2 (Lemma 1's sink split); U, V = the best rank-r
 *          approximation of the content C = S - a vbar^T, with sqrt(sigma_i) on both factors,
 *          and zero columns where C has rank below r; scales reset to 1.
 *   ws     workspace of seed_workspace_bytes(shape, SEED_OP_FROM_DENSE) bytes (may be NULL
 *          when that is 0).
 * When min(d_k, d_v) <= 64 the truncation is exact up to rounding (a factored core of the
 * smaller side). For 128 x 128 states it is a one-sided Jacobi SVD of C in fp64: sweeps of plane
 * rotations over all column pairs, stopping at the first sweep in which every pair is orthogonal
 * to 1e-8 of the product of their lengths (at most seed_from_dense_iterations() sweeps).
 * Source: thelatestinai.com figures & tables, overview table (states leaving the prefill are
 * compressed to the sink plus rank-r factors); picx.dev summary, Lemma 1.
 */
int seed_state_from_dense(const seed_shape *shape, const float *S, const float *vbar,
                          const seed_state *state, void *ws, size_t ws_bytes, void *stream);

/* The most one-sided Jacobi sweeps seed_state_from_dense runs on a 128 x 128 state (it stops at
 * the first sweep that rotates no column pair). */
int32_t seed_from_dense_iterations(void);

/*
 * One factored decode step for every unit: read-out and exact update (Lemma 2).
 *   m      columns held before the step, rank <= m < rank + period.
 *   q, k   [units][d_k] (io_dtype); v [units][d_v] (io_dtype).
 *   beta   float [units]. g: float [units] (GDN, Mamba-2) or float [units][d_k] (KDA).
 *   vbar   float [heads][d_v].
 *   o      written, [units][d_v] (io_dtype): o = vbar (a+^T q) + V+ (U+^T q).
 *   state  the scales take the decay, column m of U receives the key, column m of V receives
 *          beta (eps - V (G U)^T kappa) (GDN, KDA) or beta eps (Mamba-2), and the sink
 *          coefficient of column m is beta (omega - kappa^T G a_true) (GDN, KDA) or beta omega
 *          (Mamba-2), with omega = v^T vbar / |vbar|^2 and eps = v - omega vbar; a itself is not
 *          written (Lemma 2's sink update a+ = G a + coef kappa, kept lazily). KDA: a key
 *          channel whose cumulative gate (its scale) would fall below 2^-40 is folded into
 *          the stored columns first (that row of U is multiplied by it, the scale restarts at
 *          1, and a carries the same factor), so that the new column k / scale stays finite;
 *          the true state is unchanged.
 * Afterwards the caller holds m + 1 columns (also recorded as every unit's column count in the
 * state). Source: picx.dev summary, "Exact Update (Lemma 2)" and "SEED Architecture".
 */
int seed_decode_step(const seed_shape *shape, const seed_state *state, int32_t m,
                     const void *q, const void *k, const void *v, const float *beta,
                     const float *g, const float *vbar, void *o, void *stream);

/*
 * Head normalisation of the read-out, applied by the decode step before o is written. The sink
 * part of the read-out, vbar (a^T q), is a bias along the head's fixed direction inside the
 * norm, and its energy sets part of the gain 1 / rms the content receives (picx.dev summary,
 * "Theoretical and Practical Implications", practical implications: the state sink acts as a
 * bias and gain through the head's normalization). With x = o, or o * silu(gate) when
 * gate_first:
 *     o <- weight[h] * x / sqrt(mean over d_v of x^2 + eps)      (then * silu(gate) when a gate
 *                                                                   is given and !gate_first)
 * silu(z) = z / (1 + exp(-z)).
 *   weight      float [heads][d_v] (required).
 *   gate        [units][d_v] in io_dtype, or NULL for no gate.
 *   eps         >= 0 and finite.
 *   gate_first  0: gate after the norm (Gated DeltaNet / KDA output norm); 1: before it (the gated
 *               norm of Mamba-2).
 */
typedef struct seed_head_norm {
  const float *weight;
  const void *gate;
  float eps;
  int32_t gate_first;
} seed_head_norm;

/*
 * seed_decode_step with the head normalisation above fused into its epilogue: o receives the
 * normalised read-out (the raw read-out is not stored). The state update is that of
 * seed_decode_step. SEED_ERR_ARG for a NULL norm or weight, eps negative or not finite, or
 * gate_first other than 0 or 1. It adds one wave reduction and the weight and gate loads per
 * unit; the factors are read once, as without it.
 */
int seed_decode_step_normed(const seed_shape *shape, const seed_state *state, int32_t m,
                            const void *q, const void *k, const void *v, const float *beta,
                            const float *g, const float *vbar, const seed_head_norm *norm, void *o,
                            void *stream);

/*
 * The decode step for a ragged batch: every unit takes its own column count m from its state
 * (see the scale buffer above), as requests that joined at different times hold different
 * counts. A unit runs the step of seed_decode_step with that m, and its count goes one up, when
 *   - active is NULL or active[u] != 0 (active: uint8 [units], device memory), and
 *   - rank <= m < rank + period (a unit that holds rank + period columns is full: compress it
 *     first, with seed_compress_ragged).
 * Any other unit is left untouched and its row of o is not written. Arguments otherwise as for
 * seed_decode_step. Source: the step of seed_decode_step; serving with a batch whose requests
 * differ in length is the continuous batching of the pages' throughput section.
 */
int seed_decode_step_ragged(const seed_shape *shape, const seed_state *state,
                            const uint8_t *active, const void *q, const void *k, const void *v,
                            const float *beta, const float *g, const float *vbar, void *o,
                            void *stream);

/* seed_decode_step_ragged with the head normalisation of seed_decode_step_normed. */
int seed_decode_step_ragged_normed(const seed_shape *shape, const seed_state *state,
                                   const uint8_t *active, const void *q, const void *k, const void *v,
                                   const float *beta, const float *g, const float *vbar,
                                   const seed_head_norm *norm, void *o, void *stream);

/* Floats per unit written by seed_state_spectrum. */
#define SEED_SPECTRUM_LEN 33

/*
 * Rank-energy spectrum of the content, per unit at its own column count m (taken from the
 * state): out[u][i] for i < 32 is sigma_i^2, the i-th largest squared singular value of
 * U V^T (true, decayed columns; zero past its rank), and out[u][32] is |U V^T|_F^2 = sum over
 * all i of sigma_i^2. So out[u][32] - sum_{i<k} out[u][i] is the energy that a rank-k
 * truncation would drop. The sink a vbar^T is not part of it (its share: seed_state_energy).
 *   out    float [units][SEED_SPECTRUM_LEN], device memory, written.
 * Reads the state and writes nothing else. 16-bit factors with rank <= 32 (the compression
 * kernel's core, stopped after its eigenvalues); otherwise SEED_ERR_UNSUPPORTED.
 * Source: picx.dev summary, key finding 2 (after the sink the remaining content is low-rank),
 * and thelatestinai.com figures & tables, overview table (the rest of the state is low-rank).
 */
int seed_state_spectrum(const seed_shape *shape, const seed_state *state, float *out, void *stream);

/*
 * Compression of listed units: units[0 .. count-1] (int32, device memory) name the units to
 * compress, each at its own column count m (taken from the state), as seed_compress does for
 * one unit; a listed unit with m <= rank, or an index outside [0, units), is skipped. One
 * wavefront (or workgroup) is launched per listed unit, so a serving loop that knows which
 * requests filled their slots this step compresses only those (seed_compress_ragged instead
 * starts one per unit of the batch and lets the others leave). A unit listed twice races with
 * itself: list each at most once. count = 0 does nothing. ws as for seed_compress.
 * Source: as seed_compress; compress-when-full serving of requests of different lengths.
 */
int seed_compress_units(const seed_shape *shape, const seed_state *state, const int32_t *units,
                        int32_t count, void *ws, size_t ws_bytes, void *stream);

/*
 * Chunked update: len consecutive tokens of every unit in one call.
 * It appends the len columns and writes the len read-outs that len calls of seed_decode_step
 * would give for the same inputs (equal in exact arithmetic; fp32 arithmetic in another order).
 * Each token's value residual is found by a forward substitution over the chunk:
 * (I + A) [c | W] = beta (omega - gamma a~ . kappa | eps - gamma V U~^T kappa), with
 * A[t][s] = beta_t Gamma(t,s) kappa_t . kappa_s (s < t) and Gamma(t,s) the product of the gates
 * after token s up to token t (Mamba-2: A = 0; KDA: the gates are per key channel, so
 * kappa_t . kappa_s is weighted by each channel's product of gates).
 *   m      columns held before the chunk, rank <= m and m + len <= rank + period.
 *   len    tokens, 1 <= len <= 32 (KDA: 16; a longer KDA chunk is SEED_ERR_UNSUPPORTED).
 *   q, k   [batch][len][heads][d_k] (io_dtype), v [batch][len][heads][d_v]: token t of unit
 *          (b, h) is row (b len + t) heads + h, the layout of a projection over a batch of
 *          sequences.
 *   beta   float [batch][len][heads]. g: float [batch][len][heads] (GDN, Mamba-2) or
 *          [batch][len][heads][d_k] (KDA).
 *   vbar   float [heads][d_v].
 *   o      written, [batch][len][heads][d_v] (io_dtype): token t's read-out S_t^T q_t.
 *   state  as after len decode steps: the keys become columns m .. m + len - 1 of U (decay
 *          scale: the gates of the later tokens), W columns m .. of V, c their sink
 *          coefficients; the scales held before take the product of all len gates; the column
 *          count becomes m + len. KDA: a channel whose scale would fall below the floor of
 *          seed_decode_step is folded into the stored columns and a as there.
 * Stochastic rounding takes the draws the decode steps would take for the same stores (site,
 * slot m + t, unit, window count, element; a KDA fold: site 6 with aux = m, the count before the
 * chunk).
 * Source: picx.dev summary, "Exact Update (Lemma 2)" applied token after token, and
 * "Theoretical and Practical Implications", Lemma 1 (each part follows the head's recurrence).
 */
int seed_decode_chunk(const seed_shape *shape, const seed_state *state, int32_t m, int32_t len,
                      const void *q, const void *k, const void *v, const float *beta,
                      const float *g, const float *vbar, void *o, void *stream);

/*
 * The chunked update for a ragged batch: every unit takes its own column count m from its
 * state, as seed_decode_step_ragged does, and runs the chunk of seed_decode_chunk from it when
 *   - active is NULL or active[u] != 0 (active: uint8 [units], device memory), and
 *   - rank <= m and m + len <= rank + period (the chunk fits the unit's free slots).
 * Any other unit is left untouched and its rows of o are not written. len <= period, else
 * SEED_ERR_ARG. Arguments otherwise as for seed_decode_chunk. Source: the chunk of
 * seed_decode_chunk; requests of different lengths in one batch (continuous batching).
 */
int seed_decode_chunk_ragged(const seed_shape *shape, const seed_state *state, const uint8_t *active,
                             int32_t len, const void *q, const void *k, const void *v,
                             const float *beta, const float *g, const float *vbar, void *o,
                             void *stream);

/* The largest len seed_decode_chunk takes. */
int32_t seed_chunk_max_tokens(void);

/*
 * Compression of the content back to rank r (leaves m = r; nothing is done when m <= r).
 * The content U V^T (m columns) is replaced by its best rank-r approximation, with
 * sqrt(sigma_i) on both factors; a becomes a_true, the decay scales 1 and the sink
 * coefficients 0. Method: lazy decay
 * folded into U; column pairs balanced; Grams G_U = U^T U and G_V = V^T V; pivoted Cholesky
 * G_U ~ L L^T; the (k x k, k <= m) core B = L^T G_V L, whose eigenvalues are sigma_i^2; the
 * top r eigenpairs give U' = U X_U and V' = V X_V. The core's eigenpairs come from a
 * Householder tridiagonalisation, Sturm-count multisection and twisted factorisations in
 * fp32 for bf16 factors with r <= 32, and otherwise from cyclic Jacobi (fp64 for fp32
 * factors, fp32 for bf16 factors).
 * ws as for seed_state_from_dense with SEED_OP_COMPRESS.
 * Source: picx.dev summary, "Open-Loop Error Bound (Corollary 4)" (periodic compressions)
 * and thelatestinai.com figures & tables, overview table (compression back to rank r).
 */
int seed_compress(const seed_shape *shape, const seed_state *state, int32_t m, void *ws,
                  size_t ws_bytes, void *stream);

/*
 * Compression of the units whose own column count m_u (from the state) satisfies
 * m_u >= min_m, with rank < min_m <= rank + period: each is compressed as by seed_compress with
 * m = m_u and left with count rank; the other units are not touched. min_m = rank + period
 * compresses exactly the full units ("compress when full"), so that a ragged batch compresses
 * each unit every period steps, on the step it fills. SEED_ERR_ARG for min_m outside that range.
 */
int seed_compress_ragged(const seed_shape *shape, const seed_state *state, int32_t min_m,
                         void *ws, size_t ws_bytes, void *stream);

/*
 * Energy of every unit's state (a diagnostic): with S~ = a_true vbar^T + U_true V^T over the
 * unit's own column count (kept in the state),
 *   out[u][0] = |S~|_F^2,  out[u][1] = |a_true vbar^T|_F^2 (the sink),  out[u][2] = |U V^T|_F^2.
 * The sink's share of the energy, out[u][1] / out[u][0], summed over heads first when pooled,
 * is the statistic the pages report for trained models.
 *   vbar   float [heads][d_v];  out  float [units][3], written.
 * Source: picx.dev summary, key finding 2 and "Introduction and Theoretical Foundation" (the
 * state sink holds most of the state energy).
 */
int seed_state_energy(const seed_shape *shape, const seed_state *state, const float *vbar,
                      float *out, void *stream);

/*
 * Dense-state step (the uncompressed baseline): S <- the dense recurrence of `kind`, then
 * o = S^T q.
 *   S      float [units][d_k][d_v], read once and written once.
 *   q, k, v, beta, g, o as for seed_decode_step (factor_dtype, rank and period are ignored).
 * Source: picx.dev summary, "Introduction and Theoretical Foundation" (every decode step
 * loads and stores the whole state) and "Exact Update (Lemma 2)".
 */
int seed_dense_decode_step(const seed_shape *shape, float *S, const void *q, const void *k,
                           const void *v, const float *beta, const float *g, void *o,
                           void *stream);

/*
 * Streams restricted to a set of compute units, for schedules that run the HBM-bound decode and
 * the arithmetic-bound compression side by side on disjoint parts of the chip. These are the
 * library's own HIP runtime calls, so the stream belongs to the runtime that launches the
 * kernels.
 *   cu_mask     mask_words (1 .. 64) words; bit i of word w selects compute unit 32 w + i; at
 *               least one bit set. The runtime may refuse masks it cannot honour (on MI355X,
 *               masks that split an XCD's block of 32 compute units were refused).
 *   *stream     receives the new hipStream_t (NULL on failure). It has the default priority.
 * Returns SEED_ERR_ARG for a null pointer, an empty mask or a bad word count, SEED_ERR_HIP when
 * the runtime refuses. The caller owns the stream and releases it with seed_stream_destroy
 * after the work queued on it has finished.
 */
int seed_stream_create_cu_masked(uint32_t mask_words, const uint32_t *cu_mask, void **stream);

/* Destroys a stream made by seed_stream_create_cu_masked (SEED_ERR_ARG for NULL). */
int seed_stream_destroy(void *stream);

/* Static text for a status code. */
const char *seed_status_string(int status);

/* Library version string. */
const char *seed_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SEED_H */
