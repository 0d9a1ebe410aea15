// Internal launch interface between the C ABI (api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/seed.h"

namespace seed {

struct StepArgs {
  int64_t units;
  int32_t heads;
  int32_t m;          // columns held before the step
  int32_t rank;       // r
  int32_t slots;      // r + T: column slots per unit
  int32_t scale_len;  // per-unit floats of the scale buffer: decay scales, sink coefficients, window
                      // count, column count
  int32_t coef_off;   // where the T sink coefficients start: 1 + T (GDN, Mamba-2) or d_k (KDA)
  int32_t win_off;    // the compression-window count (a uint32 in the float buffer): coef_off + T
  int32_t m_off;      // the unit's column count m (a uint32 in the float buffer): win_off + 1
  int32_t rounding;   // 0: nearest-even factor stores; 1: stochastic
  uint32_t rng_key;   // key of the stochastic-rounding draws
  int32_t ragged;     // 1: every unit's m is its own column count; 0: m above for all
  const uint8_t* active;  // ragged: units with active[u] == 0 are skipped (nullptr: none)
  int32_t len;        // chunked update: tokens per call (q, k, v, beta, g, o are [batch][len][heads])
  float* a;
  void* U;
  void* V;
  float* scale;
  const void* q;
  const void* k;
  const void* v;
  const float* beta;
  const float* g;
  const float* vbar;
  void* o;
  // head-normalisation epilogue of the read-out (decode step only): norm_w == nullptr leaves o
  // as the read-out; otherwise o becomes norm_w[head] * x / sqrt(mean(x^2) + norm_eps), with x
  // the read-out (times silu(norm_gate) first when norm_gate_first), times silu(norm_gate)
  // after when a gate is given and !norm_gate_first
  const float* norm_w;      // [heads][d_v]
  const void* norm_gate;    // [units][d_v] in the io dtype, or nullptr
  float norm_eps;
  int32_t norm_gate_first;
};

struct DenseArgs {
  int64_t units;
  float* S;
  const void* q;
  const void* k;
  const void* v;
  const float* beta;
  const float* g;
  void* o;
};

struct CompressArgs {
  int64_t units;
  int32_t heads;
  int32_t m;          // columns held (> r)
  int32_t rank;
  int32_t slots;
  int32_t scale_len;
  int32_t coef_off;
  int32_t win_off;
  int32_t m_off;
  int32_t rounding;
  uint32_t rng_key;
  int32_t ragged;     // 1: compress the units whose own count is >= m (and > r); 0: all, at m
  float* a;
  void* U;
  void* V;
  float* scale;
  const float* S;     // from_dense only: dense states
  const float* vbar;  // from_dense only
  int32_t iters;      // from_dense only: subspace iterations (128 x 128 states)
  float* spectrum;    // spectrum mode only ([units][33]): the state is read, not written
  const int32_t* list;  // list mode: block b compresses unit list[b] (ragged semantics); nullptr: block b is unit b
  int32_t list_len;     // list mode: the number of blocks
};

// Blocks of a compression launch: one per listed unit, or one per unit.
inline int64_t compress_blocks(const CompressArgs& a) { return a.list != nullptr ? a.list_len : a.units; }

struct EnergyArgs {
  int64_t units;
  int32_t heads;
  int32_t rank;
  int32_t slots;
  int32_t scale_len;
  int32_t coef_off;
  int32_t m_off;
  const float* a;
  const void* U;
  const void* V;
  const float* scale;
  const float* vbar;
  float* out;         // [units][3]: |S~|^2, |a vbar^T|^2, |U V^T|^2
};

// Each returns hipSuccess or the launch error. Shapes are validated by the caller.
hipError_t launch_decode(const seed_shape& sh, const StepArgs& a, hipStream_t s);
hipError_t launch_dense(const seed_shape& sh, const DenseArgs& a, hipStream_t s);
hipError_t launch_compress(const seed_shape& sh, const CompressArgs& a, hipStream_t s);
hipError_t launch_from_dense(const seed_shape& sh, const CompressArgs& a, hipStream_t s);
hipError_t launch_energy(const seed_shape& sh, const EnergyArgs& a, hipStream_t s);
// The energy diagnostic for 16-bit factors (one wavefront per unit, MFMA Grams); *used tells
// whether it took the call.
hipError_t launch_energy_wave(const seed_shape& sh, const EnergyArgs& a, hipStream_t s, bool* used);
// One-wavefront-per-unit compression with the core in registers (bf16 factors, r <= 32,
// r + T <= 64); *used tells whether it took the call.
hipError_t launch_compress_wave(const seed_shape& sh, const CompressArgs& a, hipStream_t s, bool* used);

// The chunked update of len tokens per unit (scalar-decay kinds, nearest rounding).
hipError_t launch_decode_chunk(const seed_shape& sh, const StepArgs& a, hipStream_t s);
int32_t chunk_max_tokens();
// The content spectrum (spectrum mode of the one-wavefront compression kernel).
hipError_t launch_spectrum(const seed_shape& sh, const CompressArgs& a, hipStream_t s);

// Whether a compiled instance exists for this shape (host-side dispatch tables).
bool decode_supported(const seed_shape& sh);
bool compress_supported(const seed_shape& sh);
bool chunk_supported(const seed_shape& sh);

}  // namespace seed
