"""Pins of the oracle's factored step (oracle step O4) against the dense recurrence.

Lemma 2 (picx.dev summary, "Exact Update (Lemma 2)") is an identity: with no compression the
factored state a vbar^T + U V^T equals the dense state after every step. The dense recurrence
is pinned by its closed forms (test_oracle_dense.py), so this pins the factored step.
Lemma 1 (picx.dev summary, "Theoretical and Practical Implications") adds two invariants: the
sink coefficient equals the dense state's projection S vbar / |vbar|^2, and the content stays
orthogonal to vbar.
"""
import numpy as np
import pytest

import oracle as orc
import synth

RNG = np.random.default_rng(99)


def _tiny(kind, dk, dv):
    return synth.Workload("t", kind, 1, 1, dk, dv, 4, 4, 64, 16, synth.F32, synth.F32)


def _relF(A, B):
    return np.linalg.norm(A - B) / max(np.linalg.norm(B), 1e-300)


@pytest.mark.parametrize("kind", [orc.GDN, orc.KDA, orc.MAMBA2])
@pytest.mark.parametrize("dk,dv", [(16, 16), (12, 8)])
def test_lemma2_identity_from_dense_split(kind, dk, dv):
    w = _tiny(kind, dk, dv)
    xs = synth.sequence(w, seed=7 + kind, steps=16 + 64, units=1)
    xs = [{k: (v[0] if np.ndim(v) else v) for k, v in x.items()} for x in xs]
    vbar = synth.head_consts(w, 7 + kind).vbar[0]
    S0, _ = orc.run_dense(kind, np.zeros((dk, dv)), xs[:16])
    S0 = S0[-1]
    # exact split: keep every singular value, so nothing is truncated
    a, U, V, err = orc.from_dense(S0, vbar, min(dk, dv))
    assert err < 1e-12 * np.linalg.norm(S0)
    np.testing.assert_allclose(orc.reconstruct(a, vbar, U, V), S0, atol=1e-12 * np.abs(S0).max())
    Ss, os_ = orc.run_dense(kind, S0, xs[16:])
    traj = orc.run_factored(kind, a, U, V, vbar, xs[16:])
    for t, ((a_t, U_t, V_t, o_t), S_t, od_t) in enumerate(zip(traj, Ss, os_)):
        assert U_t.shape[1] == min(dk, dv) + t + 1
        assert _relF(orc.reconstruct(a_t, vbar, U_t, V_t), S_t) <= 1e-12
        assert np.linalg.norm(o_t - od_t) <= 1e-12 * np.linalg.norm(od_t)


@pytest.mark.parametrize("kind", [orc.GDN, orc.KDA, orc.MAMBA2])
def test_lemma2_identity_from_zero_state(kind):
    dk, dv = 10, 6
    w = _tiny(kind, dk, dv)
    xs = synth.sequence(w, seed=3, steps=64, units=1)
    xs = [{k: (v[0] if np.ndim(v) else v) for k, v in x.items()} for x in xs]
    vbar = RNG.standard_normal(dv) * 3.0            # any non-zero scale: only the direction matters
    Ss, _ = orc.run_dense(kind, np.zeros((dk, dv)), xs)
    traj = orc.run_factored(kind, np.zeros(dk), np.zeros((dk, 0)), np.zeros((dv, 0)), vbar, xs)
    for (a_t, U_t, V_t, _), S_t in zip(traj, Ss):
        assert _relF(orc.reconstruct(a_t, vbar, U_t, V_t), S_t) <= 1e-12
        # Lemma 1: the sink coefficient is the projection of the exact state on vbar
        np.testing.assert_allclose(a_t, S_t @ vbar / (vbar @ vbar), rtol=1e-11,
                                   atol=1e-12 * np.abs(S_t).max())
        # and the content stays orthogonal to vbar
        assert np.linalg.norm(V_t.T @ vbar) <= 1e-12 * max(np.linalg.norm(V_t), 1.0)


@pytest.mark.parametrize("kind", [orc.GDN, orc.KDA, orc.MAMBA2])
def test_zero_decay_factored_step_is_rank_one(kind):
    dk, dv = 8, 5
    a = RNG.standard_normal(dk)
    U = RNG.standard_normal((dk, 3))
    V = RNG.standard_normal((dv, 3))
    vbar = RNG.standard_normal(dv)
    kap = RNG.standard_normal(dk)
    kap /= np.linalg.norm(kap)
    q = RNG.standard_normal(dk)
    v = RNG.standard_normal(dv)
    g = np.zeros(dk) if kind == orc.KDA else 0.0
    a1, U1, V1, o1 = orc.factored_step(kind, a, U, V, vbar, q, kap, v, 0.7, g)
    omega = v @ vbar / (vbar @ vbar)
    eps = v - omega * vbar
    np.testing.assert_allclose(a1, 0.7 * omega * kap, atol=1e-14)
    np.testing.assert_allclose(U1 @ V1.T, 0.7 * np.outer(kap, eps), atol=1e-14)
    np.testing.assert_allclose(o1, 0.7 * (kap @ q) * v, atol=1e-13)


def test_value_along_vbar_only_feeds_the_sink():
    # a value exactly along vbar writes only the sink: eps = 0, so the new V column is
    # -beta V U_d^T kappa (GDN), i.e. only the delta correction
    dk, dv = 6, 4
    vbar = np.array([0.0, 2.0, 0.0, 0.0])
    a = np.zeros(dk)
    U = np.zeros((dk, 0))
    V = np.zeros((dv, 0))
    kap = np.eye(dk)[1]
    a1, U1, V1, o1 = orc.factored_step(orc.GDN, a, U, V, vbar, kap, kap, 3.0 * vbar, 0.5, 0.9)
    np.testing.assert_allclose(a1, 0.5 * 3.0 * kap)
    np.testing.assert_allclose(V1, 0.0)
    np.testing.assert_allclose(o1, 1.5 * vbar)


def test_state_energy_pins():
    """The energy split: a worked 2 x 2 case, Pythagoras when the content is orthogonal to vbar,
    and the sink split of a dense state, whose content is orthogonal to vbar by construction."""
    tot, sink, cont = orc.state_energy([2.0, 0.0], [3.0, 0.0], np.array([[0.0], [1.0]]), np.array([[0.0], [5.0]]))
    assert (tot, sink, cont) == (36.0 + 25.0, 36.0, 25.0)
    g = np.random.default_rng(3)
    vb = g.standard_normal(6)
    V = g.standard_normal((6, 3))
    V -= np.outer(vb, vb @ V) / (vb @ vb)          # columns orthogonal to vbar
    a, U = g.standard_normal(5), g.standard_normal((5, 3))
    tot, sink, cont = orc.state_energy(a, vb, U, V)
    assert tot == pytest.approx(sink + cont, rel=1e-12)
    assert sink == pytest.approx(float(a @ a) * float(vb @ vb), rel=1e-12)
    S = g.standard_normal((5, 6))
    a_s, C = orc.sink_split(S, vb)
    tot, sink, cont = orc.state_energy(a_s, vb, C, np.eye(6))
    assert tot == pytest.approx(float(np.sum(S * S)), rel=1e-12)
    assert tot == pytest.approx(sink + cont, rel=1e-12)
    # a cross term that does not vanish: the total is not the sum of the parts
    tot, sink, cont = orc.state_energy([1.0, 0.0], [1.0, 0.0], np.array([[1.0], [0.0]]), np.array([[1.0], [0.0]]))
    assert (tot, sink, cont) == (4.0, 1.0, 1.0)


def test_content_spectrum_pins():
    """The spectrum of the content: a planted spectrum (random orthonormal singular vectors,
    chosen singular values) comes back exactly; a worked rank-one case; the total is the sum of
    all squared singular values (Frobenius); past the rank the values are at the rounding level,
    and past the matrix's smaller dimension they are zero."""
    g = np.random.default_rng(11)
    sig = np.array([5.0, 3.0, 2.0, 0.5, 0.25])
    Y, _ = np.linalg.qr(g.standard_normal((9, 5)))
    Z, _ = np.linalg.qr(g.standard_normal((7, 5)))
    U = Y * sig                                     # C = Y diag(sig) Z^T, split as U V^T
    spec, tot = orc.content_spectrum(U, Z, k=8)
    np.testing.assert_allclose(spec[:5], sig ** 2, rtol=1e-12)
    assert np.all(spec[5:7] < 1e-24 * float(np.sum(sig ** 2)))   # rank 5: rounding-level values
    assert spec[7] == 0.0                                          # past min(9, 7): zero
    assert tot == pytest.approx(float(np.sum(sig ** 2)), rel=1e-12)
    # rank one: u v^T has the single singular value |u| |v|
    spec, tot = orc.content_spectrum(np.array([[3.0], [4.0]]), np.array([[1.0], [0.0], [0.0]]), k=3)
    np.testing.assert_allclose(spec, [25.0, 0.0, 0.0], atol=1e-12)
    assert tot == pytest.approx(25.0)
    # more columns than the rank: 6 columns spanning 2 directions
    A = g.standard_normal((8, 2)) @ g.standard_normal((2, 6))
    B = g.standard_normal((5, 6))
    spec, tot = orc.content_spectrum(A, B, k=4)
    C = A @ B.T
    assert tot == pytest.approx(float(np.sum(C * C)), rel=1e-12)
    assert spec[0] + spec[1] == pytest.approx(tot, rel=1e-10)
    assert spec[2] < 1e-20 * tot and spec[3] < 1e-20 * tot
