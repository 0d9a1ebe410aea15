"""Corollary 4 on the oracle's own compressed trajectories, and the byte accounting.

Corollary 4 (picx.dev summary, "Open-Loop Error Bound (Corollary 4)"): with the same inputs
driving both trajectories, |S~_t - S_t|_F <= eps_bar / (1 - g_bar^W), where eps_bar is the
largest single compression error (the prefill-end one included) and g_bar the largest decay.
W is read as the number of steps between compressions (= T).

The byte accounting is pinned to the pages' state table (tests/golden/state_table.txt).
"""
import os

import numpy as np
import pytest

import oracle as orc
import synth


def _squeeze(xs):
    return [{k: (v[0] if np.ndim(v) else v) for k, v in x.items()} for x in xs]


def _run(kind, dk, dv, r, T, steps, prefill, seed):
    w = synth.Workload("t", kind, 1, 1, dk, dv, r, T, steps, prefill, synth.F32, synth.F32)
    xs = _squeeze(synth.sequence(w, seed, prefill + steps, units=1))
    vbar = synth.head_consts(w, seed).vbar[0]
    S0, _ = orc.run_dense(kind, np.zeros((dk, dv)), xs[:prefill])
    return orc.run_compressed(kind, S0[-1], vbar, xs[prefill:], r, T), xs


@pytest.mark.parametrize("kind,dk,dv,r,T", [
    (orc.GDN, 64, 64, 8, 8),        # the small single-head GDN workload
    (orc.GDN, 32, 32, 4, 4),
    (orc.KDA, 32, 32, 6, 6),
    (orc.MAMBA2, 32, 16, 4, 4),
])
def test_corollary4_bound_holds_along_the_trajectory(kind, dk, dv, r, T):
    res, _ = _run(kind, dk, dv, r, T, steps=64, prefill=32, seed=17 + kind)
    eps_bar = max(res["errs"])
    g_bar = max(res["g_bound"])
    bound = orc.corollary4_bound(eps_bar, g_bar, T)
    errs = [np.linalg.norm(Sc - S) for Sc, S in zip(res["S_c"], res["S"])]
    assert eps_bar > 0
    assert max(errs) <= bound * (1 + 1e-9), (max(errs), bound)
    # the bound does not grow with the number of compressions: errors stay flat in time
    assert len(res["errs"]) == 1 + 64 // T


def test_prefill_error_decays_without_further_compressions():
    # with T beyond the horizon only the prefill-end error exists, and it shrinks by at most
    # g_bar per step: |E_t| <= g_bar^t eps_0
    res, _ = _run(orc.GDN, 16, 16, 3, 1000, steps=40, prefill=24, seed=5)
    eps0 = res["errs"][0]
    g_run = 1.0
    for t, (Sc, S, gb) in enumerate(zip(res["S_c"], res["S"], res["g_bound"]), start=1):
        g_run *= gb
        assert np.linalg.norm(Sc - S) <= g_run * eps0 * (1 + 1e-9)


def test_compressed_trajectory_compress_points_and_sink():
    res, xs = _run(orc.GDN, 16, 16, 4, 4, steps=8, prefill=8, seed=3)
    a, U, V = res["final"]
    assert U.shape[1] == 4 and V.shape[1] == 4


def _table(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "state_table.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            p = line.split()
            rows.append((p[0], *map(float, p[1:5]), *map(int, p[5:8])))
    return rows


def test_state_bytes_reproduce_the_pages_state_table(golden_dir):
    rows = _table(golden_dir)
    assert len(rows) == 5
    for name, dense, at_r, mean, peak, dk, dv, R in rows:
        n0 = dense * 1e6 / (4 * dk * dv)
        fits = []
        for n in range(int(n0) - 3, int(n0) + 4):
            if round(orc.dense_state_bytes(n, dk, dv) / 1e6, 1) != dense:
                continue
            got = [round(orc.state_bytes(n, dk, dv, m) / 1e6, 1) for m in (R, 1.5 * R, 2 * R)]
            if got == [at_r, mean, peak]:
                fits.append(n)
        assert fits, f"{name}: no head count reproduces the printed row"
        # and the compression ratio printed in the summary table (dense / at R)
        assert round(dense / at_r, 1) in (3.9, 2.6, 2.0)


def test_state_bytes_convention_is_discriminating(golden_dir):
    # halving the bytes per value, or counting vbar, must break the fit for the first row
    name, dense, at_r, mean, peak, dk, dv, R = _table(golden_dir)[0]
    n = 1728
    assert round(orc.state_bytes(n, dk, dv, R) / 1e6, 1) == at_r
    assert round(orc.state_bytes(n, dk, dv, R, bytes_per=2) / 1e6, 1) != at_r
    assert round((orc.state_bytes(n, dk, dv, R) + 4 * n * dv) / 1e6, 1) != at_r


def test_corollary4_bound_worked_value():
    # eps_bar / (1 - g_bar^W) at eps_bar = 1, g_bar = 1/2, W = 2 is 1 / (1 - 1/4) = 4/3, worked by
    # hand; the looser forms eps_bar / (1 - g_bar) = 2 and eps_bar / (1 - g_bar)^W = 4 differ
    assert orc.corollary4_bound(1.0, 0.5, 2) == pytest.approx(4.0 / 3.0, rel=1e-15)
    assert orc.corollary4_bound(0.1, 0.9, 8) == pytest.approx(0.1 / (1.0 - 0.43046721), rel=1e-12)
    assert orc.corollary4_bound(3.0, 0.0, 5) == pytest.approx(3.0, rel=1e-15)


def test_corollary4_bound_is_attained_by_coherent_errors():
    """A trajectory on which the bound is tight: every compression drops an error of the same
    size along the same direction, and the exact state keeps accumulating it.

    Mamba-2 head, d_k = 2, d_v = 3, vbar = e3 (so the content lives on e1, e2 and the sink stays
    0), constant decay g, rank r = 1, compression every W = 2 steps. Each window writes e1 e1^T
    (the large direction, always kept) and then b e2 e2^T (always dropped). After window k the
    exact state's e2 e2^T coefficient is b (1 + g^2 + ... + g^(2(k-1))), the compressed state's 0,
    and every compression error is b. So the distance after window k is
    b (1 - g^(2k)) / (1 - g^2), which tends to eps_bar / (1 - g_bar^W) = b / (1 - g^2): the
    geometric series of the decayed errors, summed here step by step by the oracle's own driver.
    """
    g, b, W, K = 0.5, 0.1, 2, 24
    e1, e2, e3 = np.eye(3)
    xs = []
    for _ in range(K):
        xs.append({"q": e1[:2], "k": e1[:2], "v": e1, "beta": 1.0, "g": g})
        xs.append({"q": e1[:2], "k": e2[:2], "v": b * e2, "beta": 1.0, "g": g})
    res = orc.run_compressed(orc.MAMBA2, np.zeros((2, 3)), e3, xs, r=1, T=W)
    errs = res["errs"]
    assert errs[0] == 0.0 and np.allclose(errs[1:], b, rtol=1e-12)
    bound = orc.corollary4_bound(max(errs), max(res["g_bound"]), W)
    dist = [np.linalg.norm(Sc - S) for Sc, S in zip(res["S_c"], res["S"])]
    for k in range(1, K + 1):
        expect = b * (1 - g ** (2 * k)) / (1 - g * g)
        assert dist[2 * k - 1] == pytest.approx(expect, rel=1e-12)
    assert max(dist) <= bound * (1 + 1e-12)
    assert max(dist) >= bound * (1 - 1e-12)          # tight: the sup is the bound itself
    # a bound with g_bar in place of g_bar^W would be loose by a factor 1 + g here
    assert max(dist) / orc.corollary4_bound(max(errs), max(res["g_bound"]), 1) == pytest.approx(1 / (1 + g))
