"""The decode step with the head normalisation fused into its epilogue, against the oracle.

picx.dev summary, "Theoretical and Practical Implications", practical implications: the state
sink acts as a bias and gain through the head's normalization. seed_decode_step_normed writes
weight[h] * x / sqrt(mean(x^2) + eps) (x the read-out, gated before or after) in place of the
read-out. Checked per call, teacher-forced: the state after the call is bit for bit the state a
plain seed_decode_step leaves from the same state and inputs (the epilogue touches only o), and
o matches the oracle's head_norm of the oracle's Lemma 2 read-out from the GPU's state before
the call, at the read-out's tolerance.
"""
import numpy as np
import pytest

import oracle as orc
import synth
from gpu_util import host_inputs, host_state, out_tolerance, relF, shape_of, to_device_inputs, torch_dtype

pytestmark = pytest.mark.gpu

CASES = [
    # kind, d_k, d_v, r, T, factor dtype, gate: None / "after" / "first"
    (synth.GDN, 128, 128, 16, 16, synth.BF16, "after"),
    (synth.GDN, 128, 128, 16, 16, synth.F32, None),
    (synth.KDA, 128, 128, 8, 8, synth.F32, "after"),
    (synth.MAMBA2, 128, 64, 16, 16, synth.BF16, "first"),
    (synth.MAMBA2, 128, 64, 16, 16, synth.F16, None),
    (synth.GDN, 64, 64, 8, 8, synth.BF16, "first"),
]


def _setup(kind, dk, dv, r, T, fdt, seed):
    import torch
    import rank_recurrent_state_amd as rrs
    io = synth.BF16 if fdt == synth.F16 else fdt
    w = synth.Workload("norm", kind, 3, 4, dk, dv, r, T, T, 24, fdt, io)
    sh = shape_of(w)
    hc = synth.head_consts(w, seed)
    gen = synth.rng(seed)
    vbar = torch.tensor(hc.vbar, dtype=torch.float32, device="cuda")
    S = torch.zeros((w.units, dk, dv), dtype=torch.float32, device="cuda")
    o = torch.empty((w.units, dv), dtype=torch_dtype(io), device="cuda")
    for _ in range(w.prefill):
        d = to_device_inputs(synth.step_inputs(w, hc, gen, w.units), io)
        rrs.seed_dense_decode_step(sh, S, d["q"], d["k"], d["v"], d["beta"], d["g"], o)
    st = rrs.State.empty(sh)
    rrs.seed_state_from_dense(sh, S, vbar, st)
    return rrs, torch, w, sh, hc, gen, vbar, st, o


@pytest.mark.parametrize("kind,dk,dv,r,T,fdt,gate", CASES)
def test_normed_step_matches_oracle(kind, dk, dv, r, T, fdt, gate):
    rrs, torch, w, sh, hc, gen, vbar, st, o = _setup(kind, dk, dv, r, T, fdt, 4100 + kind * 7 + dk + r)
    n = w.units
    wgen = np.random.default_rng(9)
    weight_np = wgen.uniform(0.5, 1.5, (w.heads, dv))
    weight = torch.tensor(weight_np, dtype=torch.float32, device="cuda")
    eps = 1e-5
    tol = out_tolerance(w)
    worst = 0.0
    m = r
    for step in range(T - 1):
        x = synth.step_inputs(w, hc, gen, n)
        dx = to_device_inputs(x, w.io_dtype)
        z = None
        if gate is not None:
            z = torch.tensor(wgen.standard_normal((n, dv)) * 2.0, dtype=torch.float32,
                             device="cuda").to(torch_dtype(w.io_dtype)).contiguous()
        pre = host_state(sh, st, range(n), m)
        plain = rrs.State(*[t.clone() for t in st.tensors()])
        o_plain = torch.empty_like(o)
        rrs.seed_decode_step(sh, plain, m, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], vbar, o_plain)
        rrs.seed_decode_step_normed(sh, st, m, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], vbar, o, weight,
                                    gate=z, eps=eps, gate_first=(gate == "first"))
        for a_, b_ in zip(st.tensors(), plain.tensors()):
            assert torch.equal(a_, b_), "the epilogue changed the state"
        hx = host_inputs(dx, range(n))
        og = o.double().cpu().numpy()
        zh = None if z is None else z.double().cpu().numpy()
        for u in range(n):
            h = u % w.heads
            X = hx[u]
            _, _, _, o1 = orc.factored_step(kind, *pre[u], hc.vbar[h], X["q"], X["k"], X["v"], X["beta"], X["g"])
            y = orc.head_norm(o1, weight_np[h], eps, gate=None if zh is None else zh[u], gate_first=(gate == "first"))
            e = relF(og[u], y)
            worst = max(worst, e)
            assert e <= tol, f"step {step} unit {u}: {e}"
        m += 1
    torch.cuda.synchronize()
    print(f"\n[head norm {synth.KIND_NAMES[kind]} {dk}x{dv} {gate}] worst {worst:.2e} (tolerance {tol})", flush=True)


def test_ragged_normed_and_argument_errors():
    rrs, torch, w, sh, hc, gen, vbar, st, o = _setup(synth.GDN, 128, 128, 8, 8, synth.BF16, 4321)
    n = w.units
    weight_np = np.linspace(0.5, 1.5, w.heads * 128).reshape(w.heads, 128)
    weight = torch.tensor(weight_np, dtype=torch.float32, device="cuda")
    x = synth.step_inputs(w, hc, gen, n)
    dx = to_device_inputs(x, w.io_dtype)
    active = torch.tensor([u % 3 != 1 for u in range(n)], dtype=torch.uint8, device="cuda")
    pre = host_state(sh, st, range(n), w.rank)
    o.fill_(7.0)
    rrs.seed_decode_step_ragged_normed(sh, st, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], vbar, o, weight,
                                       eps=1e-6, active=active)
    counts = rrs.column_counts(sh, st).numpy()
    hx = host_inputs(dx, range(n))
    og = o.double().cpu().numpy()
    for u in range(n):
        if u % 3 == 1:
            assert counts[u] == w.rank and np.all(og[u] == 7.0)   # skipped: untouched
            continue
        assert counts[u] == w.rank + 1
        X = hx[u]
        _, _, _, o1 = orc.factored_step(w.kind, *pre[u], hc.vbar[u % w.heads], X["q"], X["k"], X["v"], X["beta"], X["g"])
        assert relF(og[u], orc.head_norm(o1, weight_np[u % w.heads], 1e-6)) <= out_tolerance(w)
    with pytest.raises(rrs.SeedError):   # eps must be >= 0
        rrs.seed_decode_step_normed(sh, st, w.rank + 1, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], vbar, o,
                                    weight, eps=-1.0)
    with pytest.raises(rrs.SeedError):   # gate_first must be 0 or 1
        rrs.seed_decode_step_normed(sh, st, w.rank + 1, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], vbar, o,
                                    weight, gate_first=2)
