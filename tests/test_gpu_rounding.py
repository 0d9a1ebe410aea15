"""Stochastic rounding of the 16-bit factor stores, through the C ABI, against the oracle.

* Bit for bit: the decode step's new U column is the key (GDN) or kappa / Gamma (KDA), a value
  the oracle reproduces exactly in fp32 from the step's key and the Gamma the step stored. Each
  stored element must equal the oracle's stochastic rounding of that value with the oracle's own
  Philox4x32-10 draws for the same key, unit, window, site, slot and element.
* The compression-window count starts at 0 after the prefill-end compression and goes one up
  per compression.
* Whole trajectories (prefill-end compression, decode, compression) stay within the format's
  tolerance of the fp64 oracle, teacher-forced per call.
* The draws depend on the key: a run is reproduced exactly by the same key, not by another.
"""
from __future__ import annotations

import numpy as np
import pytest

import synth
from gpu_util import (check_compress_call, check_decode_call, check_from_dense_call, out_tolerance,
                      tolerance, to_device_inputs, torch_dtype)
from oracle import rounding as rd

pytestmark = pytest.mark.gpu

FMT = {synth.BF16: rd.BF16, synth.F16: rd.FP16}


def _rrs():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_recurrent_state_amd as rrs
    return rrs, torch


def _setup(kind, fdt, key, r=8, T=8, batch=2, heads=3, prefill=24, seed=71):
    rrs, torch = _rrs()
    dv = 64 if kind == synth.MAMBA2 else 128
    w = synth.Workload("sr", kind, batch, heads, 128, dv, r, T, 2 * T, prefill, fdt, synth.BF16)
    sh = rrs.make_shape(kind, batch, heads, 128, dv, r, T, fdt, synth.BF16,
                        rounding=rrs.SEED_ROUND_STOCHASTIC, rng_key=key)
    hc = synth.head_consts(w, seed)
    gen = synth.rng(seed)
    vbar = torch.tensor(hc.vbar, dtype=torch.float32, device="cuda")
    S = torch.zeros((w.units, 128, dv), dtype=torch.float32, device="cuda")
    o = torch.empty((w.units, dv), dtype=torch.bfloat16, device="cuda")
    for _ in range(prefill):
        d = to_device_inputs(synth.step_inputs(w, hc, gen, w.units), synth.BF16)
        rrs.seed_dense_decode_step(sh, S, d["q"], d["k"], d["v"], d["beta"], d["g"], o)
    return rrs, torch, w, sh, hc, gen, vbar, S, o


def _window_count(st, sh):
    """The compression-window count: the scale buffer's second-to-last float (a uint32), before
    the column count."""
    sc = np.ascontiguousarray(st.scale.detach().cpu().numpy()[:, -2])
    return sc.view(np.uint32).astype(np.int64)


def _bits(t, fdt):
    """Raw 16-bit codes of a bf16 / fp16 tensor (numpy int64)."""
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().astype(np.int64) & 0xFFFF


def _codes(vals, fmt):
    """16-bit codes of float64 values that are exactly representable in fmt."""
    if fmt == rd.FP16:
        return vals.astype(np.float16).view(np.uint16).astype(np.int64)
    return (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.int64)


@pytest.mark.parametrize("kind", [synth.GDN, synth.KDA])
@pytest.mark.parametrize("fdt", [synth.BF16, synth.F16])
def test_decode_u_column_bit_exact(kind, fdt):
    key = 0x5EED1234
    rrs, torch, w, sh, hc, gen, vbar, S, o = _setup(kind, fdt, key)
    st = rrs.State.empty(sh)
    rrs.seed_state_from_dense(sh, S, vbar, st)
    n, r, T = w.units, w.rank, w.period
    assert np.all(_window_count(st, sh) == 0)
    fmt = FMT[fdt]
    m = r
    windows_seen = set()
    d_idx = np.arange(w.d_k)
    rounded_up = 0
    for t in range(T + 4):
        x = synth.step_inputs(w, hc, gen, n)
        if kind == synth.KDA and t == 2:
            x["g"][0] = 0.0          # unit 0 forgets: its Gamma folds into the stored columns
        dx = to_device_inputs(x, synth.BF16)
        win = _window_count(st, sh)
        rrs.seed_decode_step(sh, st, m, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], vbar, o)
        torch.cuda.synchronize()
        kf = dx["k"].float().cpu().numpy().astype(np.float32)
        got = _bits(st.U[:, m, :], fdt)
        gam = st.scale[:, :w.d_k].cpu().numpy().astype(np.float32)
        for u in range(n):
            val = kf[u] / gam[u] if kind == synth.KDA else kf[u]      # fp32 quotient (IEEE)
            r16 = rd.sr_bits(key, u, int(win[u]), rd.SITE_DECODE_U, m, d_idx)
            exp = _codes(rd.round_stochastic(val.astype(np.float32), fmt, r16), fmt)
            assert np.array_equal(got[u], exp), f"step {t} unit {u}: {np.count_nonzero(got[u] != exp)} codes differ"
            rounded_up += int(np.count_nonzero(exp != _codes(rd.neighbors(val.astype(np.float32), fmt)[0], fmt)))
            windows_seen.add(int(win[u]))
        m += 1
        if m == r + T:
            rrs.seed_compress(sh, st, m)
            torch.cuda.synchronize()
            assert np.all(_window_count(st, sh) == win + 1)
            m = r
    assert windows_seen == {0, 1}
    if kind == synth.KDA:
        assert rounded_up > 0    # the draws did take quotients away from zero somewhere


@pytest.mark.parametrize("kind", [synth.GDN, synth.KDA, synth.MAMBA2])
@pytest.mark.parametrize("fdt", [synth.BF16, synth.F16])
def test_trajectory_within_tolerance(kind, fdt):
    rrs, torch, w, sh, hc, gen, vbar, S, o = _setup(kind, fdt, 777 + kind, r=16, T=16)
    units = list(range(w.units))
    st, err, _ = check_from_dense_call(rrs, sh, S, vbar, hc.vbar, w.heads, units, fdt)
    tol, tol_o = tolerance(w), out_tolerance(w)
    assert err <= tol
    m = w.rank
    for t in range(w.period + 3):
        dx = to_device_inputs(synth.step_inputs(w, hc, gen, w.units), synth.BF16)
        eS, eo = check_decode_call(rrs, sh, st, m, dx, vbar, hc.vbar, w.heads, units, o)
        assert eS <= tol and eo <= tol_o, f"step {t}: S {eS} o {eo}"
        m += 1
        if m == w.rank + w.period:
            ec, _ = check_compress_call(rrs, sh, st, m, hc.vbar, w.heads, units, fdt)
            assert ec <= tol, f"compress after step {t}: {ec}"
            m = w.rank


def _run(kind, fdt, key, steps):
    rrs, torch, w, sh, hc, gen, vbar, S, o = _setup(kind, fdt, key, seed=91)
    st = rrs.State.empty(sh)
    rrs.seed_state_from_dense(sh, S, vbar, st)
    m = w.rank
    for _ in range(steps):
        dx = to_device_inputs(synth.step_inputs(w, hc, gen, w.units), synth.BF16)
        rrs.seed_decode_step(sh, st, m, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], vbar, o)
        m += 1
        if m == w.rank + w.period:
            rrs.seed_compress(sh, st, m)
            m = w.rank
    torch.cuda.synchronize()
    return [t.clone() for t in st.tensors()]


@pytest.mark.parametrize("fdt", [synth.BF16, synth.F16])
def test_draws_follow_the_key(fdt):
    import torch
    a = _run(synth.KDA, fdt, 1, 11)
    b = _run(synth.KDA, fdt, 1, 11)
    c = _run(synth.KDA, fdt, 2, 11)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert not torch.equal(a[1], c[1]) and not torch.equal(a[2], c[2])   # U and V
