"""GPU parity of the content spectrum (seed_state_spectrum, through the C ABI) against the oracle.

Per unit, at its own column count: the 32 largest squared singular values of U V^T and the total
|U V^T|_F^2, against oracle.content_spectrum of the same stored state read back in fp64 (true,
decayed columns). Both sides see the same stored bits, so the difference is the kernel's fp32
arithmetic: its Grams, pivoted Cholesky, core B = L^T G_V L and the eigenvalues of B. Each
eigenvalue is held to 1e-4 of the largest (fp32 carries about 1e-7 of the entries of B, and the
core is formed by two products of 64-term sums), the total to 1e-4 relative. The state must be
left bit for bit as it was.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle as orc
import synth
from gpu_util import host_state, to_device_inputs, torch_dtype

pytestmark = pytest.mark.gpu

TOL_EIG = 1e-4
TOL_TOTAL = 1e-4


def _rrs():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_recurrent_state_amd as rrs
    return rrs, torch


def _state(kind, dk, dv, r, T, fdt, steps, seed, batch=2, heads=3):
    rrs, torch = _rrs()
    w = synth.Workload("spec", kind, batch, heads, dk, dv, r, T, 2 * T, 24, fdt, synth.BF16)
    sh = rrs.make_shape(kind, batch, heads, dk, dv, r, T, fdt, synth.BF16)
    hc = synth.head_consts(w, seed)
    gen = synth.rng(seed)
    vbar = torch.tensor(hc.vbar, dtype=torch.float32, device="cuda")
    S = torch.zeros((w.units, dk, dv), dtype=torch.float32, device="cuda")
    o = torch.empty((w.units, dv), dtype=torch.bfloat16, device="cuda")
    for _ in range(w.prefill):
        dx = to_device_inputs(synth.step_inputs(w, hc, gen, w.units), synth.BF16)
        rrs.seed_dense_decode_step(sh, S, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], o)
    st = rrs.State.empty(sh)
    rrs.seed_state_from_dense(sh, S, vbar, st)
    for t in range(steps):
        dx = to_device_inputs(synth.step_inputs(w, hc, gen, w.units), synth.BF16)
        rrs.seed_decode_step(sh, st, r + t, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], vbar, o)
    return rrs, torch, w, sh, st


def _check(rrs, torch, sh, st, m):
    before = [t.clone() for t in st.tensors()]
    out = rrs.seed_state_spectrum(sh, st)
    torch.cuda.synchronize()
    for x, y in zip(before, st.tensors()):
        assert torch.equal(x, y), "the spectrum wrote to the state"
    got = out.double().cpu().numpy()
    units = list(range(sh.units))
    hs = host_state(sh, st, units, m)
    worst_e = worst_t = 0.0
    for i in range(len(units)):
        _, U, V = hs[i]
        spec, tot = orc.content_spectrum(U, V, k=32)
        lam1 = max(spec[0], 1e-30)
        worst_e = max(worst_e, float(np.max(np.abs(got[i, :32] - spec))) / lam1)
        worst_t = max(worst_t, abs(got[i, 32] - tot) / max(tot, 1e-30))
        assert np.all(np.diff(got[i, :32]) <= 1e-6 * lam1), "not in decreasing order"
    return worst_e, worst_t


CASES = {
    # kind, d_k, d_v, r, T, factors, decode steps after the prefill-end compression
    "gdn-n32:bf16": (synth.GDN, 128, 128, 16, 16, synth.BF16, 9),
    "gdn-n64:bf16": (synth.GDN, 128, 128, 32, 32, synth.BF16, 31),
    "kda-n64:fp16": (synth.KDA, 128, 128, 32, 32, synth.F16, 20),
    "mamba2-n32:bf16": (synth.MAMBA2, 128, 64, 16, 16, synth.BF16, 12),
    "gdn-rank-only:bf16": (synth.GDN, 64, 64, 16, 16, synth.BF16, 0),
}


@pytest.mark.parametrize("case", list(CASES))
def test_spectrum_against_oracle(case):
    kind, dk, dv, r, T, fdt, steps = CASES[case]
    rrs, torch, w, sh, st = _state(kind, dk, dv, r, T, fdt, steps, seed=300 + kind)
    e, t = _check(rrs, torch, sh, st, r + steps)
    print(f"[spectrum] {case} m={r + steps}: eigenvalues {e:.2e} of the largest, total {t:.2e}", flush=True)
    assert e <= TOL_EIG and t <= TOL_TOTAL


def test_spectrum_ragged_counts():
    """Units at different column counts (a staggered batch): each at its own."""
    rrs, torch, w, sh, st = _state(synth.GDN, 128, 128, 16, 16, synth.BF16, 0, seed=7, batch=4)
    hc = synth.head_consts(w, 7)
    gen = synth.rng(99)
    vbar = torch.tensor(hc.vbar, dtype=torch.float32, device="cuda")
    o = torch.empty((w.units, w.d_v), dtype=torch.bfloat16, device="cuda")
    B, H = w.batch, w.heads
    for t in range(12):
        dx = to_device_inputs(synth.step_inputs(w, hc, gen, w.units), synth.BF16)
        act = torch.tensor([1 if (u // H) * 3 >= t else 0 for u in range(w.units)], dtype=torch.uint8,
                           device="cuda")
        rrs.seed_decode_step_ragged(sh, st, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], vbar, o, active=act)
    m = rrs.column_counts(sh, st).numpy()
    assert len(set(m.tolist())) > 1
    e, tt = _check(rrs, torch, sh, st, m)
    print(f"[spectrum] ragged counts {sorted(set(m.tolist()))}: {e:.2e}, total {tt:.2e}", flush=True)
    assert e <= TOL_EIG and tt <= TOL_TOTAL
