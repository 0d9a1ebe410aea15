"""Parity at the workloads' full sizes, in the launch configuration the benchmark times.

Every unit of a layer goes through the HIP kernels: a dense prefill of the workload's length,
the prefill-end compression, a full compression window of decode steps, the compression, and
two more decode steps. The fp64 oracle checks a seeded sample of units call by call
(teacher-forced: it starts each call from the GPU's own state), with the first and last unit
always in the sample. Inputs are drawn on the device by the same seeded generators as the
benchmark's. gdn-stack36 is checked on one layer (4,096 units): a benchmark launch, with its
bf16 factors and again with fp16 factors (bf16 inputs).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import synth
from gpu_util import (check_compress_call, check_decode_call, check_from_dense_call, out_tolerance,
                      tolerance, torch_dtype)

pytestmark = pytest.mark.gpu

FULL = ["gdn-layer", "kda-layer", "mamba2-layer", "gdn-stack36", "gdn-stack36:fp16"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_recurrent_state_amd as rrs

    name, _, fmt = name.partition(":")
    w = synth.WORKLOADS[name]
    if fmt == "fp16":
        w = dataclasses.replace(w, factor_dtype=synth.F16)
    units = w.batch * w.heads
    seed = 3000 + sorted(synth.WORKLOADS).index(name)
    sh = rrs.make_shape(w.kind, w.batch, w.heads, w.d_k, w.d_v, w.rank, w.period, w.factor_dtype,
                        w.io_dtype)
    io = torch_dtype(w.io_dtype)
    ds = synth.DeviceStream(w, seed, "cuda", units=units)
    vbar = ds.vbar(0)
    vbar_np = vbar.double().cpu().numpy()
    tol = tolerance(w)
    tol_o = out_tolerance(w)
    rng = np.random.default_rng(seed)
    sample = sorted({0, units - 1, *rng.choice(units, size=10, replace=False).tolist()})
    print(f"\n[{name}] {units} units, prefill {w.prefill}, sample {sample}", flush=True)

    S = torch.zeros((units, w.d_k, w.d_v), dtype=torch.float32, device="cuda")
    o = torch.empty((units, w.d_v), dtype=io, device="cuda")
    for _ in range(w.prefill):
        x = ds.step(io)
        rrs.seed_dense_decode_step(sh, S, x["q"], x["k"], x["v"], x["beta"], x["g"], o)
    torch.cuda.synchronize()

    st, err, ties = check_from_dense_call(rrs, sh, S, vbar, vbar_np, w.heads, sample, w.factor_dtype)
    print(f"[{name}] from_dense worst {err:.2e} (near-ties {ties})", flush=True)
    assert err <= tol
    del S

    m = w.rank
    worst_S = worst_o = worst_c = 0.0
    for t in range(w.period + 2):
        x = ds.step(io)
        eS, eo = check_decode_call(rrs, sh, st, m, x, vbar, vbar_np, w.heads, sample, o)
        worst_S, worst_o = max(worst_S, eS), max(worst_o, eo)
        assert eS <= tol and eo <= tol_o, f"{name} decode step {t}: S {eS} o {eo}"
        m += 1
        if m == w.rank + w.period:
            ec, ties = check_compress_call(rrs, sh, st, m, vbar_np, w.heads, sample, w.factor_dtype)
            worst_c = max(worst_c, ec)
            print(f"[{name}] compress: {ties} near-ties of {len(sample)}, product error vs the "
                  f"oracle's truncation {check_compress_call.last_raw:.2e}", flush=True)
            assert ec <= tol, f"{name} compress: {ec}"
            m = w.rank
    torch.cuda.synchronize()
    print(f"[{name}] decode S {worst_S:.2e} o {worst_o:.2e}, compress {worst_c:.2e}", flush=True)
