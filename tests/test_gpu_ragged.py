"""Ragged batches through the C ABI: every unit steps from its own column count and is
compressed on the step it fills, checked call by call against the fp64 oracle.

The units are staggered first: an active mask holds unit u out of the first decode steps until
its count is r + (u mod T), so that later every step fills and compresses a different subset.
Then every call is compared with the oracle (teacher-forced, at each unit's own count): the
stepped units by Lemma 2, the compressed ones by the exact truncation; units a call must not
touch (inactive, or not full) are compared bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle as orc
import synth
from gpu_util import (compare_compression, host_inputs, host_state, out_tolerance, rel_out, relF,
                      to_device_inputs, tolerance, torch_dtype)

pytestmark = pytest.mark.gpu


def _rrs():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_recurrent_state_amd as rrs
    return rrs, torch


def _setup(kind, fdt, r, T, batch, heads, prefill=32, seed=131):
    rrs, torch = _rrs()
    dv = 64 if kind == synth.MAMBA2 else 128
    io = synth.BF16 if fdt == synth.F16 else fdt
    w = synth.Workload("ragged", kind, batch, heads, 128, dv, r, T, 3 * T, prefill, fdt, io)
    sh = rrs.make_shape(kind, batch, heads, 128, dv, r, T, fdt, io)
    hc = synth.head_consts(w, seed)
    gen = synth.rng(seed)
    vbar = torch.tensor(hc.vbar, dtype=torch.float32, device="cuda")
    S = torch.zeros((w.units, 128, dv), dtype=torch.float32, device="cuda")
    o = torch.empty((w.units, dv), dtype=torch_dtype(io), device="cuda")
    for _ in range(prefill):
        d = to_device_inputs(synth.step_inputs(w, hc, gen, w.units), io)
        rrs.seed_dense_decode_step(sh, S, d["q"], d["k"], d["v"], d["beta"], d["g"], o)
    st = rrs.State.empty(sh)
    rrs.seed_state_from_dense(sh, S, vbar, st)
    return rrs, torch, w, sh, hc, gen, vbar, st, o


def _snapshot(st, units):
    import torch
    idx = torch.as_tensor(units, device=st.a.device)
    return [t.index_select(0, idx).clone() for t in st.tensors()]


def _decode_checked(rrs, torch, w, sh, hc, gen, vbar, st, o, active):
    """One ragged decode step, checked per unit; returns the counts after it."""
    n = w.units
    tol, tol_o = tolerance(w), out_tolerance(w)
    m0 = rrs.column_counts(sh, st).numpy()
    units = list(range(n))
    steps = [u for u in units if active[u] and sh.rank <= m0[u] < sh.rank + sh.period]
    still = [u for u in units if u not in steps]
    pre = host_state(sh, st, steps, m0[steps]) if steps else []
    keep = _snapshot(st, still) if still else None
    o.fill_(7.0)
    o_keep = o.clone()
    dx = to_device_inputs(synth.step_inputs(w, hc, gen, n), w.io_dtype)
    act = torch.as_tensor(np.asarray(active, dtype=np.uint8), device="cuda")
    rrs.seed_decode_step_ragged(sh, st, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], vbar, o, active=act)
    m1 = rrs.column_counts(sh, st).numpy()
    assert np.array_equal(m1[steps], m0[steps] + 1) and np.array_equal(m1[still], m0[still])
    if steps:
        post = host_state(sh, st, steps, m1[steps])
        og = o.double().cpu().numpy()
        hx = host_inputs(dx, steps)
        for i, u in enumerate(steps):
            vb = hc.vbar[u % w.heads]
            X = hx[i]
            a1, U1, V1, o1 = orc.factored_step(w.kind, *pre[i], vb, X["q"], X["k"], X["v"], X["beta"], X["g"])
            S1 = orc.reconstruct(a1, vb, U1, V1)
            eS = relF(orc.reconstruct(post[i][0], vb, post[i][1], post[i][2]), S1)
            eo = rel_out(og[u], o1, S1, X["q"])
            assert eS <= tol and eo <= tol_o, f"unit {u} at m {m0[u]}: S {eS} o {eo}"
    if still:
        for a_, b_ in zip(keep, _snapshot(st, still)):
            assert torch.equal(a_, b_)
        idx = torch.as_tensor(still, device="cuda")
        assert torch.equal(o.index_select(0, idx), o_keep.index_select(0, idx))
    return m1


def _compress_checked(rrs, torch, w, sh, hc, st, min_m):
    """One ragged compression, checked per unit; returns the number of units compressed."""
    n = w.units
    tol = tolerance(w)
    m0 = rrs.column_counts(sh, st).numpy()
    full = [u for u in range(n) if m0[u] >= min_m and m0[u] > sh.rank]
    rest = [u for u in range(n) if u not in full]
    pre = host_state(sh, st, full, m0[full]) if full else []
    keep = _snapshot(st, rest) if rest else None
    rrs.seed_compress_ragged(sh, st, min_m)
    m1 = rrs.column_counts(sh, st).numpy()
    assert np.all(m1[full] == sh.rank) and np.array_equal(m1[rest], m0[rest])
    if full:
        post = host_state(sh, st, full, sh.rank)
        for i, u in enumerate(full):
            vb = hc.vbar[u % w.heads]
            kind, err, _, sink = compare_compression((pre[i][1], pre[i][2]), post[i][0], vb, post[i][1],
                                                     post[i][2], sh.rank, w.factor_dtype, a_ref=pre[i][0])
            assert err <= tol, f"unit {u} compressed at m {m0[u]}: {kind} {err} (sink {sink})"
    if rest:
        for a_, b_ in zip(keep, _snapshot(st, rest)):
            assert torch.equal(a_, b_)
    return len(full)


@pytest.mark.parametrize("kind,fdt", [(synth.GDN, synth.BF16), (synth.KDA, synth.F32),
                                      (synth.MAMBA2, synth.BF16), (synth.GDN, synth.F16)])
def test_staggered_trajectory(kind, fdt):
    r, T = 8, 8
    rrs, torch, w, sh, hc, gen, vbar, st, o = _setup(kind, fdt, r, T, batch=3, heads=4)
    n = w.units
    assert np.all(rrs.column_counts(sh, st).numpy() == r)
    phase = np.arange(n) % T
    # stagger: unit u sits out the steps from its phase on, so it ends at r + phase
    for s in range(T - 1):
        _decode_checked(rrs, torch, w, sh, hc, gen, vbar, st, o, active=(phase > s))
    assert np.array_equal(rrs.column_counts(sh, st).numpy(), r + phase)
    compressed = []
    for t in range(2 * T + 2):
        _decode_checked(rrs, torch, w, sh, hc, gen, vbar, st, o, active=np.ones(n, dtype=bool))
        compressed.append(_compress_checked(rrs, torch, w, sh, hc, st, r + T))
    # step t fills and compresses exactly the units of phase T - 1 - t (mod T)
    for t, c in enumerate(compressed):
        assert c == int(np.count_nonzero(phase == (T - 1 - t) % T)), f"step {t}: {c} compressed"
    assert sum(compressed) == 2 * n + int(np.count_nonzero(phase >= T - 2))


def test_full_unit_is_skipped():
    r, T = 8, 8
    rrs, torch, w, sh, hc, gen, vbar, st, o = _setup(synth.GDN, synth.BF16, r, T, batch=2, heads=3)
    n = w.units
    for s in range(T):
        # unit 0 takes every step and fills; the others stop one short of full
        _decode_checked(rrs, torch, w, sh, hc, gen, vbar, st, o,
                        active=np.array([True] + [s < T - 1] * (n - 1)))
    m = rrs.column_counts(sh, st).numpy()
    assert m[0] == r + T and np.all(m[1:] == r + T - 1)
    # a full unit is not stepped again (checked inside: untouched, its row of o not written)
    _decode_checked(rrs, torch, w, sh, hc, gen, vbar, st, o, active=np.ones(n, dtype=bool))
    m = rrs.column_counts(sh, st).numpy()
    assert np.all(m == r + T)
    assert _compress_checked(rrs, torch, w, sh, hc, st, r + T) == n


def test_uniform_calls_keep_the_counts():
    r, T = 8, 8
    rrs, torch, w, sh, hc, gen, vbar, st, o = _setup(synth.KDA, synth.BF16, r, T, batch=2, heads=2)
    assert np.all(rrs.column_counts(sh, st).numpy() == r)
    m = r
    for _ in range(3):
        dx = to_device_inputs(synth.step_inputs(w, hc, gen, w.units), w.io_dtype)
        rrs.seed_decode_step(sh, st, m, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], vbar, o)
        m += 1
    assert np.all(rrs.column_counts(sh, st).numpy() == m)
    # a threshold below r + T compresses early: here every unit, at r + 3 columns
    assert _compress_checked(rrs, torch, w, sh, hc, st, r + 4) == 0
    assert _compress_checked(rrs, torch, w, sh, hc, st, r + 3) == w.units
    m = r
    for _ in range(2):
        dx = to_device_inputs(synth.step_inputs(w, hc, gen, w.units), w.io_dtype)
        rrs.seed_decode_step(sh, st, m, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], vbar, o)
        m += 1
    rrs.seed_compress(sh, st, m)
    assert np.all(rrs.column_counts(sh, st).numpy() == r)


@pytest.mark.parametrize("fdt", [synth.BF16, synth.F32])
def test_compress_units_matches_ragged_scan(fdt):
    """seed_compress_units over the units that are full gives, bit for bit, what
    seed_compress_ragged gives (the same kernel per unit: the one-wave kernel for bf16 factors,
    the workgroup kernel for fp32); units not listed, or listed with m <= r, are left as they
    were."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_recurrent_state_amd as rrs
    from gpu_util import to_device_inputs
    w = synth.Workload("units", synth.GDN, 4, 3, 128, 128, 8, 8, 16, 16, fdt, fdt)
    sh = rrs.make_shape(w.kind, w.batch, w.heads, 128, 128, 8, 8, fdt, fdt)
    hc = synth.head_consts(w, 5)
    gen = synth.rng(5)
    n, H = w.units, w.heads
    vbar = torch.tensor(hc.vbar, dtype=torch.float32, device="cuda")
    S = torch.zeros((n, 128, 128), dtype=torch.float32, device="cuda")
    o = torch.empty((n, 128), dtype=torch.bfloat16 if fdt else torch.float32, device="cuda")
    for _ in range(w.prefill):
        dx = to_device_inputs(synth.step_inputs(w, hc, gen, n), fdt)
        rrs.seed_dense_decode_step(sh, S, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], o)
    st = rrs.State.empty(sh)
    rrs.seed_state_from_dense(sh, S, vbar, st)
    # request b takes 8 - 2 b steps: counts 16 (full), 14, 12, 10
    for t in range(8):
        dx = to_device_inputs(synth.step_inputs(w, hc, gen, n), fdt)
        act = torch.tensor([1 if t < 8 - 2 * (u // H) else 0 for u in range(n)], dtype=torch.uint8, device="cuda")
        rrs.seed_decode_step_ragged(sh, st, dx["q"], dx["k"], dx["v"], dx["beta"], dx["g"], vbar, o, active=act)
    m = rrs.column_counts(sh, st)
    assert sorted(set(m.tolist())) == [10, 12, 14, 16]
    a = rrs.State(*[t.clone() for t in st.tensors()])
    b = rrs.State(*[t.clone() for t in st.tensors()])
    rrs.seed_compress_ragged(sh, a, 16)                      # the full ones
    full = torch.nonzero(m == 16).flatten().to(torch.int32).cuda()
    rrs.seed_compress_units(sh, b, full)
    torch.cuda.synchronize()
    for x, y in zip(a.tensors(), b.tensors()):
        assert torch.equal(x, y)
    # every unit listed: each at its own count (all hold columns beyond r)
    c = rrs.State(*[t.clone() for t in st.tensors()])
    rrs.seed_compress_units(sh, c, torch.arange(n, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(rrs.column_counts(sh, c) == 8)
    # a second call: every count is r now, so nothing changes
    d = rrs.State(*[t.clone() for t in c.tensors()])
    rrs.seed_compress_units(sh, d, torch.arange(n, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    for x, y in zip(c.tensors(), d.tensors()):
        assert torch.equal(x, y)
