"""Parity at the workloads' full sizes, in the launch configuration the benchmark times.

Every unit of a layer goes through the HIP kernels: a dense prefill of the workload's length,
the prefill-end compression, and the workload's whole decode trajectory with its periodic
compressions (the fp16 variant of the layer stack: two compression windows and two more steps).
A seeded sample of 64 units (the first and last always among them) is checked three ways:

* The prefill. The oracle runs the same dense recurrence in fp64 on the exact inputs the device
  buffers held, and its state is compared with the GPU's fp32 one (a sanity check of S_0).
* Every call, teacher-forced. The oracle applies the same operation to the GPU's state before
  the call (Lemma 2 step, compression, prefill-end compression) and the GPU's state after it is
  held to the format's tolerance, the sink included after every compression.
* The free-running trajectory. The exact dense recurrence runs in fp64 from the GPU's prefill
  state, beside the GPU's compressed trajectory (never reset). Corollary 4 of the picx.dev
  summary bounds their distance: the error of one compression decays by at most g per step and
  errors add, so |S~_t - S_t|_F <= sum_j (prod over the steps after compression j of g) eps_j
  (eps_j the GPU's own compression errors |S~_before - S~_after|_F, the prefill-end one
  included; g the step's bound on |Phi_t|_2). That is the corollary's eps_bar / (1 - g_bar^W)
  with each step's own decay in place of the largest one. The check adds the format's rounding
  allowance, tol |S_t|_F.

Inputs are drawn on the device by the same seeded generators as the benchmark's. gdn-stack36 is
checked on one layer (4,096 units): a benchmark launch, with its bf16 factors, and again with
fp16 factors (bf16 inputs).
"""
from __future__ import annotations

import dataclasses
import time

import numpy as np
import pytest

import oracle as orc
import synth
from gpu_util import (compare_compression, host_state, out_tolerance, rel_out, relF, tolerance,
                      torch_dtype)

pytestmark = pytest.mark.gpu

FULL = ["gdn-layer", "kda-layer", "mamba2-layer", "gdn-stack36", "gdn-stack36:fp16"]
SAMPLE = 64


def _host(x: dict, idx, keys=("q", "k", "v", "beta", "g")):
    return {k: x[k].index_select(0, idx).float().cpu().double().numpy() for k in keys}


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_recurrent_state_amd as rrs

    name, _, fmt = name.partition(":")
    w = synth.WORKLOADS[name]
    if fmt == "fp16":
        w = dataclasses.replace(w, factor_dtype=synth.F16, steps=2 * w.period + 2)
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
    sample = sorted({0, units - 1, *rng.choice(np.arange(1, units - 1), size=SAMPLE - 2, replace=False).tolist()})
    assert len(sample) == SAMPLE
    idx = torch.as_tensor(sample, device="cuda")
    vbs = [vbar_np[u % w.heads] for u in sample]
    t0 = time.time()
    print(f"\n[{name}{':' + fmt if fmt else ''}] {units} units, prefill {w.prefill}, {w.steps} steps, "
          f"{SAMPLE} sampled units", flush=True)

    # ---- dense prefill on the GPU; the oracle follows it in fp64 on the sample ----
    S = torch.zeros((units, w.d_k, w.d_v), dtype=torch.float32, device="cuda")
    o = torch.empty((units, w.d_v), dtype=io, device="cuda")
    S_orc = [np.zeros((w.d_k, w.d_v)) for _ in sample]
    for t in range(w.prefill):
        x = ds.step(io)
        rrs.seed_dense_decode_step(sh, S, x["q"], x["k"], x["v"], x["beta"], x["g"], o)
        hx = _host(x, idx)
        for i in range(SAMPLE):
            S_orc[i], _ = orc.dense_step(w.kind, S_orc[i], hx["q"][i], hx["k"][i], hx["v"][i],
                                         hx["beta"][i], hx["g"][i])
    S0 = S.index_select(0, idx).double().cpu().numpy()
    e_pre = max(relF(S0[i], S_orc[i]) for i in range(SAMPLE))
    print(f"[{name}] prefill S_0 fp32 vs fp64 oracle: {e_pre:.2e} ({time.time() - t0:.1f} s)", flush=True)
    assert e_pre <= 1e-5

    # ---- prefill-end compression ----
    st = rrs.State.empty(sh)
    rrs.seed_state_from_dense(sh, S, vbar, st)
    del S
    post = host_state(sh, st, sample, w.rank)
    worst_fd = sink_fd = 0.0
    ties = 0
    exact = [S0[i].copy() for i in range(SAMPLE)]  # the exact trajectory, from the GPU's S_0
    bound = np.zeros(SAMPLE)                       # the free-running bound, per unit
    for i in range(SAMPLE):
        a_o, _, _, _ = orc.from_dense(S0[i], vbs[i], w.rank)
        _, C = orc.sink_split(S0[i], vbs[i])
        kind, err, _, sk = compare_compression(C, post[i][0], vbs[i], post[i][1], post[i][2], w.rank,
                                               w.factor_dtype, a_ref=a_o)
        worst_fd, sink_fd = max(worst_fd, err), max(sink_fd, sk)
        ties += kind == "optimal"
        bound[i] = np.linalg.norm(orc.reconstruct(*post[i][:1], vbs[i], *post[i][1:]) - S0[i])
    print(f"[{name}] from_dense worst {worst_fd:.2e}, sink {sink_fd:.2e} (near-ties {ties})", flush=True)
    assert worst_fd <= tol and sink_fd <= tol

    # ---- the decode trajectory with its compressions ----
    m = w.rank
    worst_S = worst_o = worst_c = sink_c = 0.0
    free_ratio = free_rel = 0.0
    ties = ncomp = 0
    for t in range(1, w.steps + 1):
        x = ds.step(io)
        rrs.seed_decode_step(sh, st, m, x["q"], x["k"], x["v"], x["beta"], x["g"], vbar, o)
        hx = _host(x, idx)
        og = o.index_select(0, idx).double().cpu().numpy()
        nxt = host_state(sh, st, sample, m + 1)
        for i in range(SAMPLE):
            X = {k: hx[k][i] for k in hx}
            a1, U1, V1, o1 = orc.factored_step(w.kind, *post[i], vbs[i], X["q"], X["k"], X["v"], X["beta"], X["g"])
            S1 = orc.reconstruct(a1, vbs[i], U1, V1)
            Sg = orc.reconstruct(nxt[i][0], vbs[i], nxt[i][1], nxt[i][2])
            eS, eo = relF(Sg, S1), rel_out(og[i], o1, S1, X["q"])
            worst_S, worst_o = max(worst_S, eS), max(worst_o, eo)
            assert eS <= tol and eo <= tol_o, f"{name} step {t} unit {sample[i]}: S {eS} o {eo}"
            exact[i], _ = orc.dense_step(w.kind, exact[i], X["q"], X["k"], X["v"], X["beta"], X["g"])
            bound[i] *= orc.decay_bound(w.kind, X["g"])
        post = nxt
        m += 1
        if m == w.rank + w.period:
            rrs.seed_compress(sh, st, m)
            nxt = host_state(sh, st, sample, w.rank)
            for i in range(SAMPLE):
                kind, err, _, sk = compare_compression((post[i][1], post[i][2]), nxt[i][0], vbs[i], nxt[i][1],
                                                       nxt[i][2], w.rank, w.factor_dtype, a_ref=post[i][0])
                worst_c, sink_c = max(worst_c, err), max(sink_c, sk)
                ties += kind == "optimal"
                assert err <= tol, f"{name} compression after step {t} unit {sample[i]}: {kind} {err} sink {sk}"
                bound[i] += np.linalg.norm(orc.reconstruct(*nxt[i][:1], vbs[i], *nxt[i][1:])
                                           - orc.reconstruct(*post[i][:1], vbs[i], *post[i][1:]))
            post = nxt
            ncomp += 1
            m = w.rank
        # free running: the GPU's compressed trajectory against the exact one
        for i in range(SAMPLE):
            Sg = orc.reconstruct(post[i][0], vbs[i], post[i][1], post[i][2])
            dist, nS = np.linalg.norm(Sg - exact[i]), np.linalg.norm(exact[i])
            free_rel = max(free_rel, dist / nS)
            ratio = dist / (bound[i] + tol * nS)
            free_ratio = max(free_ratio, ratio)
            assert ratio <= 1.0, (f"{name} step {t} unit {sample[i]}: free-running distance {dist:.3e} beyond "
                                  f"the compressions' bound {bound[i]:.3e} + {tol} |S|")
        if t % 128 == 0 or t == w.steps:
            print(f"[{name}] step {t}/{w.steps}: decode S {worst_S:.2e} o {worst_o:.2e}, compress {worst_c:.2e} "
                  f"sink {sink_c:.2e} ({ncomp} compressions, near-ties {ties}), free-running rel {free_rel:.2e} "
                  f"at {free_ratio:.3f} of its bound ({time.time() - t0:.0f} s)", flush=True)
    torch.cuda.synchronize()
    assert ncomp == w.steps // w.period
