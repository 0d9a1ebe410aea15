"""Edge cases of the HIP path against the fp64 oracle, through the C ABI.

beta = 0 (pure decay), g = 0 (complete forgetting), a zero state, a repeated key across a whole
compression window (duplicate U columns), the no-op compression at m = r, and the scale of vbar
(only its direction matters) -- each for fp32, bf16 and fp16 factors where it applies (fp16
factors with bf16 inputs).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle as orc
import synth
from gpu_util import (check_compress_call, check_decode_call, check_from_dense_call, host_state,
                      out_tolerance, relF, tolerance, to_device_inputs, torch_dtype)

pytestmark = pytest.mark.gpu

KINDS = [synth.GDN, synth.KDA, synth.MAMBA2]


def _setup(kind, fdt, seed, prefill=24, batch=2, heads=3, r=8, T=8):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_recurrent_state_amd as rrs

    dv = 64 if kind == synth.MAMBA2 else 128
    io = synth.BF16 if fdt == synth.F16 else fdt
    w = synth.Workload("edge", kind, batch, heads, 128, dv, r, T, 2 * T, prefill, fdt, io)
    sh = rrs.make_shape(kind, batch, heads, 128, dv, r, T, fdt, io)
    hc = synth.head_consts(w, seed)
    gen = synth.rng(seed)
    vbar = torch.tensor(hc.vbar, dtype=torch.float32, device="cuda")
    n = w.units
    S = torch.zeros((n, w.d_k, w.d_v), dtype=torch.float32, device="cuda")
    o = torch.empty((n, w.d_v), dtype=torch_dtype(io), device="cuda")
    for _ in range(prefill):
        d = to_device_inputs(synth.step_inputs(w, hc, gen, n), io)
        rrs.seed_dense_decode_step(sh, S, d["q"], d["k"], d["v"], d["beta"], d["g"], o)
    return rrs, w, sh, hc, gen, vbar, S, o


def _window(rrs, w, sh, hc, gen, vbar, st, o, make, steps):
    """Decode `steps` steps with inputs from make(t, x) and check every call, compressing at
    r + T columns."""
    n = w.units
    units = list(range(n))
    tol = tolerance(w)
    tol_o = out_tolerance(w)
    m = w.rank
    for t in range(steps):
        x = make(t, synth.step_inputs(w, hc, gen, n))
        dx = to_device_inputs(x, w.io_dtype)
        eS, eo = check_decode_call(rrs, sh, st, m, dx, vbar, hc.vbar, w.heads, units, o)
        assert eS <= tol and eo <= tol_o, f"step {t}: S {eS} o {eo}"
        m += 1
        if m == w.rank + w.period:
            ec, _ = check_compress_call(rrs, sh, st, m, hc.vbar, w.heads, units, w.factor_dtype)
            assert ec <= tol, f"compress after step {t}: {ec}"
            m = w.rank
    return m


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("fdt", [synth.F32, synth.BF16, synth.F16])
def test_beta_zero_is_pure_decay(kind, fdt):
    rrs, w, sh, hc, gen, vbar, S, o = _setup(kind, fdt, 41)
    st, _, _ = check_from_dense_call(rrs, sh, S, vbar, hc.vbar, w.heads, range(w.units), fdt)

    def make(t, x):
        x["beta"] = np.zeros_like(x["beta"])
        if kind == synth.MAMBA2:
            # Mamba-2's own gates reach exp(-48) per step: with nothing written, an fp32 state
            # would underflow within two steps and the relative error would compare zeros
            x["g"] = 0.9 + 0.1 * gen.random(x["g"].shape)
        return x
    _window(rrs, w, sh, hc, gen, vbar, st, o, make, w.period + 2)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("fdt", [synth.F32, synth.BF16, synth.F16])
def test_zero_decay_forgets_everything(kind, fdt):
    rrs, w, sh, hc, gen, vbar, S, o = _setup(kind, fdt, 43)
    st, _, _ = check_from_dense_call(rrs, sh, S, vbar, hc.vbar, w.heads, range(w.units), fdt)

    def make(t, x):
        if t in (2, w.period - 1):
            x["g"] = np.zeros_like(x["g"])
        return x
    _window(rrs, w, sh, hc, gen, vbar, st, o, make, w.period + 3)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("fdt", [synth.F32, synth.BF16, synth.F16])
def test_zero_state(kind, fdt):
    rrs, w, sh, hc, gen, vbar, S, o = _setup(kind, fdt, 47, prefill=0)
    st, err, _ = check_from_dense_call(rrs, sh, S, vbar, hc.vbar, w.heads, range(w.units), fdt)
    assert float(st.a.abs().max()) == 0.0
    _window(rrs, w, sh, hc, gen, vbar, st, o, lambda t, x: x, w.period + 1)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("fdt", [synth.F32, synth.BF16, synth.F16])
def test_repeated_key_window(kind, fdt):
    """The same key every step: the T new U columns are parallel (a rank-deficient Gram)."""
    rrs, w, sh, hc, gen, vbar, S, o = _setup(kind, fdt, 53)
    st, _, _ = check_from_dense_call(rrs, sh, S, vbar, hc.vbar, w.heads, range(w.units), fdt)
    key = {}

    def make(t, x):
        if "k" not in key:
            key["k"] = x["k"].copy()
        x["k"] = key["k"].copy()
        return x
    _window(rrs, w, sh, hc, gen, vbar, st, o, make, w.period + 2)


@pytest.mark.parametrize("fdt", [synth.F32, synth.BF16, synth.F16])
def test_compress_at_rank_is_a_no_op(fdt):
    import torch
    rrs, w, sh, hc, gen, vbar, S, o = _setup(synth.GDN, fdt, 59)
    st, _, _ = check_from_dense_call(rrs, sh, S, vbar, hc.vbar, w.heads, range(w.units), fdt)
    before = [t.clone() for t in st.tensors()]
    rrs.seed_compress(sh, st, w.rank)
    rrs.seed_compress(sh, st, 0)
    torch.cuda.synchronize()
    for b, a in zip(before, st.tensors()):
        assert torch.equal(b, a)


@pytest.mark.parametrize("kind", KINDS)
def test_vbar_scale_does_not_matter(kind):
    """Only the direction of vbar matters: a run with 3 vbar reconstructs the same S~ and o."""
    import torch
    rrs, w, sh, hc, gen, vbar, S, o = _setup(kind, synth.F32, 61)
    n = w.units
    st1 = rrs.State.empty(sh)
    st3 = rrs.State.empty(sh)
    rrs.seed_state_from_dense(sh, S, vbar, st1)
    rrs.seed_state_from_dense(sh, S, 3.0 * vbar, st3)
    o3 = torch.empty_like(o)
    m = w.rank
    for t in range(w.period + 1):
        dx = to_device_inputs(synth.step_inputs(w, hc, gen, n), w.io_dtype)
        rrs.seed_decode_step(sh, st1, m, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], vbar, o)
        rrs.seed_decode_step(sh, st3, m, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], 3.0 * vbar, o3)
        assert relF(o3.double().cpu().numpy(), o.double().cpu().numpy()) <= 1e-5
        m += 1
        if m == w.rank + w.period:
            rrs.seed_compress(sh, st1, m)
            rrs.seed_compress(sh, st3, m)
            m = w.rank
    h1 = host_state(sh, st1, range(n), m)
    h3 = host_state(sh, st3, range(n), m)
    for u in range(n):
        vb = hc.vbar[u % w.heads]
        S1 = orc.reconstruct(h1[u][0], vb, h1[u][1], h1[u][2])
        S3 = orc.reconstruct(h3[u][0], 3.0 * vb, h3[u][1], h3[u][2])
        assert relF(S3, S1) <= 1e-5
