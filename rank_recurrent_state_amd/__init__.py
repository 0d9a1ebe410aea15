"""Sink + rank-r recurrent decode state on MI355X (gfx950).

The library (libseed.so, hand-written HIP kernels behind a C ABI declared in include/seed.h)
holds each Gated DeltaNet, Kimi Delta Attention or Mamba-2 head's recurrent state as a sink
a vbar^T plus rank-r factors U V^T, runs the fused read-out + exact update per decode step (or
per chunk of tokens), compresses back to rank r every T steps, and provides the dense-state step as a baseline.

This package is the thin Python binding over that C ABI (rank_recurrent_state_amd._lib). The
binding is loaded on first use of any of its names, and raises ImportError if libseed.so has
not been built (python -m rank_recurrent_state_amd.build): there is no fallback path.
"""
import importlib

_NAMES = {
    "EXPORTS", "LIB_PATH", "SEED_BF16", "SEED_ERR_ARG", "SEED_ERR_HIP", "SEED_ERR_UNSUPPORTED",
    "SEED_ERR_WORKSPACE", "SEED_F16", "SEED_F32", "SEED_GDN", "SEED_KDA", "SEED_MAMBA2", "SEED_OK",
    "SEED_OP_COMPRESS", "SEED_OP_FROM_DENSE", "SEED_ROUND_NEAREST", "SEED_ROUND_STOCHASTIC",
    "SeedError", "State", "make_shape",
    "column_counts", "seed_compress", "seed_compress_ragged", "seed_decode_step",
    "seed_decode_step_ragged", "seed_dense_decode_step", "seed_from_dense_iterations",
    "seed_state_energy", "seed_decode_chunk", "seed_chunk_max_tokens", "seed_state_spectrum",
    "seed_decode_chunk_ragged", "seed_compress_units",
    "SEED_SPECTRUM_LEN", "CUMaskedStream", "hip_runtimes_mapped", "seed_head_norm",
    "seed_decode_step_normed", "seed_decode_step_ragged_normed",
    "seed_scale_len", "seed_shape", "seed_state", "seed_state_bytes", "seed_state_from_dense",
    "seed_status_string", "seed_version", "seed_workspace_bytes",
}


_OVERLAP = {"OverlappedStack", "StaggeredStack", "partition_streams", "under_profiler"}


def __getattr__(name):
    if name in _NAMES:
        return getattr(importlib.import_module("._lib", __name__), name)
    if name in _OVERLAP:
        return getattr(importlib.import_module(".overlap", __name__), name)
    raise AttributeError(name)


__all__ = sorted(_NAMES | _OVERLAP)
