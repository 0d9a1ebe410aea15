"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Protocol (per call, teacher-forced): the GPU state before a call is read back in fp64 and the
oracle applies the same operation (Lemma 2 step, compression, prefill-end compression, dense
step) to it with the same inputs; the GPU's state after the call and its output are compared
with the oracle's: rel-Frobenius on the reconstructed S~ = a vbar^T + U V^T and rel-L2 on o.
Tolerances: 1e-5 for fp32 factors, 2e-2 for bf16 and 2.5e-3 for fp16 factors (fp32 arithmetic
throughout). Compressions whose relative gap (sigma_r - sigma_{r+1}) / sigma_1 is below 1e-3
(fp32), 5e-2 (bf16) or 1e-2 (fp16) have several correct answers; they are checked by the Eckart-Young optimality
criterion instead. The free-running trajectory is compared as well.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle as orc
import synth
from gpu_util import (compare_compression, host_inputs, host_state, out_tolerance, rel_out, relF,
                      shape_of, to_device_inputs, tolerance, torch_dtype)

pytestmark = pytest.mark.gpu


def _rrs():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_recurrent_state_amd as rrs
    return rrs, torch


def _squeeze(xs, units):
    return xs


def run_parity(w: synth.Workload, seed: int, steps: int, check_units=None, report=None,
               free_running=True, x_override=None):
    """Dense prefill, prefill-end compression, decode steps with periodic compressions, all on
    the GPU, checked call by call against the oracle on `check_units`."""
    rrs, torch = _rrs()
    sh = shape_of(w)
    n = w.units
    check = list(range(n)) if check_units is None else list(check_units)
    tol = tolerance(w)
    tol_o = out_tolerance(w)
    hc = synth.head_consts(w, seed)
    vbar_np = hc.vbar
    vbar = torch.tensor(vbar_np, dtype=torch.float32, device="cuda")
    heads_of = [u % w.heads for u in check]
    gen = synth.rng(seed)
    io = torch_dtype(w.io_dtype)
    rep = {"dense": 0.0, "from_dense": [], "step_S": 0.0, "step_o": 0.0, "compress": [],
           "free_S": 0.0, "free_o": 0.0, "ties": 0}

    # dense prefill on the GPU; the oracle follows the same inputs on the checked units
    S = torch.zeros((n, w.d_k, w.d_v), dtype=torch.float32, device="cuda")
    o = torch.empty((n, w.d_v), dtype=io, device="cuda")
    S_orc = [np.zeros((w.d_k, w.d_v)) for _ in check]
    for t in range(w.prefill):
        x = synth.step_inputs(w, hc, gen, n)
        dx = to_device_inputs(x, w.io_dtype)
        rrs.seed_dense_decode_step(sh, S, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], o)
        hx = host_inputs(dx, check)
        og = o.index_select(0, torch.as_tensor(check, device="cuda")).double().cpu().numpy()
        for i, u in enumerate(check):
            S_orc[i], oo = orc.dense_step(w.kind, S_orc[i], hx[i]["q"], hx[i]["k"], hx[i]["v"],
                                          hx[i]["beta"], hx[i]["g"])
            if t == w.prefill - 1:
                rep["dense"] = max(rep["dense"], rel_out(og[i], oo, S_orc[i], hx[i]["q"]))
    Sg = S.index_select(0, torch.as_tensor(check, device="cuda")).double().cpu().numpy()
    for i in range(len(check)):
        rep["dense"] = max(rep["dense"], relF(Sg[i], S_orc[i]))

    # prefill-end compression (teacher-forced on the GPU's own dense states)
    st = rrs.State.empty(sh)
    rrs.seed_state_from_dense(sh, S, vbar, st)
    post = host_state(sh, st, check, w.rank)
    free = []
    for i, u in enumerate(check):
        vb = vbar_np[heads_of[i]]
        a_o, U_o, V_o, _ = orc.from_dense(Sg[i], vb, w.rank)
        _, C = orc.sink_split(Sg[i], vb)
        kind, err, raw, sink = compare_compression(C, post[i][0], vb, post[i][1], post[i][2], w.rank,
                                                   w.factor_dtype, a_ref=a_o)
        rep["from_dense"].append((kind, err, raw, sink))
        rep["ties"] += kind == "optimal"
        assert err <= tol, f"from_dense unit {u}: {kind} {err}"
        free.append([a_o, U_o, V_o])

    # decode steps with periodic compressions
    m = w.rank
    for t in range(1, steps + 1):
        x = synth.step_inputs(w, hc, gen, n) if x_override is None else x_override(t, n)
        dx = to_device_inputs(x, w.io_dtype)
        pre = host_state(sh, st, check, m)
        rrs.seed_decode_step(sh, st, m, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], vbar, o)
        post = host_state(sh, st, check, m + 1)
        og = o.index_select(0, torch.as_tensor(check, device="cuda")).double().cpu().numpy()
        hx = host_inputs(dx, check)
        for i, u in enumerate(check):
            vb = vbar_np[heads_of[i]]
            X = hx[i]
            a1, U1, V1, o1 = orc.factored_step(w.kind, *pre[i], vb, X["q"], X["k"], X["v"], X["beta"], X["g"])
            S1 = orc.reconstruct(a1, vb, U1, V1)
            eS = relF(orc.reconstruct(*post[i][:1], vb, *post[i][1:]), S1)
            eo = rel_out(og[i], o1, S1, X["q"])
            rep["step_S"] = max(rep["step_S"], eS)
            rep["step_o"] = max(rep["step_o"], eo)
            assert eS <= tol and eo <= tol_o, f"decode step {t} unit {u}: S {eS} o {eo}"
            if free_running:
                fa, fU, fV, fo = orc.factored_step(w.kind, *free[i], vb, X["q"], X["k"], X["v"], X["beta"], X["g"])
                free[i] = [fa, fU, fV]
                rep["free_S"] = max(rep["free_S"], relF(orc.reconstruct(*post[i][:1], vb, *post[i][1:]),
                                                        orc.reconstruct(fa, vb, fU, fV)))
                rep["free_o"] = max(rep["free_o"], rel_out(og[i], fo, orc.reconstruct(fa, vb, fU, fV), X["q"]))
        m += 1
        if m == w.rank + w.period:
            pre = host_state(sh, st, check, m)
            rrs.seed_compress(sh, st, m)
            post = host_state(sh, st, check, w.rank)
            for i, u in enumerate(check):
                vb = vbar_np[heads_of[i]]
                kind, err, raw, sink = compare_compression((pre[i][1], pre[i][2]), post[i][0], vb,
                                                           post[i][1], post[i][2], w.rank, w.factor_dtype,
                                                           a_ref=pre[i][0])
                rep["compress"].append((kind, err, raw, sink))
                rep["ties"] += kind == "optimal"
                assert err <= tol, f"compress after step {t} unit {u}: {kind} {err}"
                if free_running:
                    fU, fV, _ = orc.compress(free[i][1], free[i][2], w.rank)
                    free[i][1], free[i][2] = fU, fV
            m = w.rank
    torch.cuda.synchronize()
    if report is not None:
        report.update(rep)
    return rep


def _summary(name, rep):
    fd = max((e[2] for e in rep["from_dense"]), default=0.0)
    cp = max((e[2] for e in rep["compress"]), default=0.0)
    sk = max((e[3] for e in rep["from_dense"] + rep["compress"]), default=0.0)
    print(f"\n[{name}] dense {rep['dense']:.2e} from_dense {fd:.2e} step S {rep['step_S']:.2e} "
          f"o {rep['step_o']:.2e} compress {cp:.2e} sink {sk:.2e} free S {rep['free_S']:.2e} "
          f"o {rep['free_o']:.2e} near-ties {rep['ties']}", flush=True)


def test_gdn_tiny_full_trajectory():
    """The small single-head GDN workload in full: d 64, r 8, T 8, 64 steps, fp32."""
    w = synth.WORKLOADS["gdn-tiny"]
    rep = run_parity(w, seed=1001, steps=w.steps)
    _summary("gdn-tiny", rep)
    assert rep["dense"] <= 1e-5
    assert len(rep["compress"]) == w.steps // w.period
    if rep["ties"] == 0:
        assert rep["free_S"] <= 1e-5 and rep["free_o"] <= 1e-5


SMALL = [
    # kind, d_k, d_v, r, T, factor dtype, batch, heads
    (synth.GDN, 128, 128, 16, 16, synth.F32, 3, 5),
    (synth.GDN, 128, 128, 16, 16, synth.BF16, 3, 5),
    (synth.KDA, 128, 128, 8, 8, synth.F32, 2, 3),
    (synth.KDA, 128, 128, 32, 32, synth.BF16, 2, 3),
    (synth.MAMBA2, 128, 64, 16, 16, synth.F32, 3, 3),
    (synth.MAMBA2, 128, 64, 16, 16, synth.BF16, 3, 3),
    (synth.GDN, 64, 128, 4, 12, synth.F32, 1, 7),
    (synth.GDN, 64, 64, 24, 40, synth.BF16, 2, 3),
    # the 32-wide compression kernel (r + T <= 32) with d_k = 64, at its largest rank, and the
    # 64-wide one at r + T = 33
    (synth.KDA, 64, 64, 8, 24, synth.BF16, 2, 3),
    (synth.GDN, 64, 128, 12, 20, synth.BF16, 3, 2),
    (synth.GDN, 128, 128, 31, 1, synth.BF16, 2, 2),
    (synth.MAMBA2, 128, 64, 17, 16, synth.BF16, 2, 3),
    # bf16 factors with r > 32: the workgroup compression kernel with an fp32 Jacobi core
    (synth.GDN, 128, 64, 40, 8, synth.BF16, 2, 2),
    # fp16 factors (bf16 inputs): both wave-compression widths, d_k = 64, and r > 32
    (synth.GDN, 128, 128, 16, 16, synth.F16, 3, 5),
    (synth.KDA, 128, 128, 32, 32, synth.F16, 2, 3),
    (synth.MAMBA2, 128, 64, 16, 16, synth.F16, 3, 3),
    (synth.GDN, 64, 128, 12, 20, synth.F16, 3, 2),
    (synth.GDN, 128, 64, 40, 8, synth.F16, 2, 2),
]

DT_NAMES = {synth.F32: "fp32", synth.BF16: "bf16", synth.F16: "fp16"}


@pytest.mark.parametrize("kind,dk,dv,r,T,fdt,batch,heads", SMALL)
def test_small_multi_unit(kind, dk, dv, r, T, fdt, batch, heads):
    """Several units (a ragged last workgroup), more than one compression window."""
    io = synth.BF16 if fdt == synth.F16 else fdt
    w = synth.Workload("small", kind, batch, heads, dk, dv, r, T, 2 * T + 3, 48, fdt, io)
    rep = run_parity(w, seed=2000 + kind * 10 + dk + r, steps=w.steps)
    _summary(f"{synth.KIND_NAMES[kind]} {dk}x{dv} r{r} T{T} {DT_NAMES[fdt]}", rep)
    if fdt == synth.F32:
        assert rep["dense"] <= 1e-5


@pytest.mark.parametrize("kind", [synth.GDN, synth.KDA, synth.MAMBA2])
@pytest.mark.parametrize("dk,dv", [(128, 128), (128, 64), (64, 128), (64, 64)])
@pytest.mark.parametrize("io", [synth.F32, synth.BF16])
def test_dense_step_teacher_forced(kind, dk, dv, io):
    rrs, torch = _rrs()
    w = synth.Workload("dense", kind, 3, 3, dk, dv, 8, 8, 1, 1, io, io)
    sh = shape_of(w)
    n = w.units
    gen = synth.rng(77 + kind + dk + dv + io)
    hc = synth.head_consts(w, 77)
    S0 = torch.tensor(gen.standard_normal((n, dk, dv)) * 0.3, dtype=torch.float32, device="cuda")
    S = S0.clone()
    x = synth.step_inputs(w, hc, gen, n)
    dx = to_device_inputs(x, io)
    o = torch.empty((n, dv), dtype=torch_dtype(io), device="cuda")
    rrs.seed_dense_decode_step(sh, S, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], o)
    hx = host_inputs(dx, range(n))
    S0h, Sh, oh = S0.double().cpu().numpy(), S.double().cpu().numpy(), o.double().cpu().numpy()
    tol_o = 1e-5 if io == synth.F32 else 8e-3   # o is stored in the io dtype
    for u in range(n):
        Sr, orr = orc.dense_step(kind, S0h[u], hx[u]["q"], hx[u]["k"], hx[u]["v"], hx[u]["beta"], hx[u]["g"])
        assert relF(Sh[u], Sr) <= 1e-6
        assert rel_out(oh[u], orr, Sr, hx[u]["q"]) <= tol_o
