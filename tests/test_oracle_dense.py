"""Pins of the oracle's dense recurrences (oracle step O1) against closed forms.

Each special case below has a value fixed by the mathematics of the recurrence, not by the
oracle's own formula, so that a dropped term, a wrong sign or a transposed operand fails:

* beta = 1 and |kappa| = 1 make a delta-rule step overwrite what the key reads: S+^T kappa = v
  for any decay (GDN and KDA).
* With g = 1, beta = 1, |kappa| = 1, key directions orthogonal to kappa are left untouched.
* beta = 0 leaves only the decay; KDA's gate acts per key channel (per row of the state).
* g = 0 leaves the rank-one state beta kappa v^T.
* Mamba-2 driven by constant inputs from zero sums a geometric series.
"""
import numpy as np
import pytest

import oracle as orc

RNG = np.random.default_rng(1234)


def _unit(n):
    x = RNG.standard_normal(n)
    return x / np.linalg.norm(x)


@pytest.mark.parametrize("kind", [orc.GDN, orc.KDA])
@pytest.mark.parametrize("dk,dv", [(8, 8), (16, 8), (6, 11)])
def test_delta_rule_overwrites_what_the_key_reads(kind, dk, dv):
    S = RNG.standard_normal((dk, dv))
    kap = _unit(dk)
    v = RNG.standard_normal(dv)
    g = RNG.uniform(0.2, 1.0, size=dk) if kind == orc.KDA else 0.37
    Sn, o = orc.dense_step(kind, S, kap, kap, v, 1.0, g)
    np.testing.assert_allclose(Sn.T @ kap, v, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-12)   # reading with q = kappa returns v


@pytest.mark.parametrize("dk,dv", [(8, 8), (12, 5)])
def test_delta_rule_leaves_orthogonal_key_directions(dk, dv):
    S = RNG.standard_normal((dk, dv))
    kap = _unit(dk)
    v = RNG.standard_normal(dv)
    Sn, _ = orc.dense_step(orc.GDN, S, kap, kap, v, 1.0, 1.0)
    x = RNG.standard_normal(dk)
    x -= (x @ kap) * kap                      # x orthogonal to kappa
    np.testing.assert_allclose(x @ Sn, x @ S, atol=1e-12)
    # and the change is rank one along kappa on the key side
    D = Sn - S
    s = np.linalg.svd(D, compute_uv=False)
    assert s[1] < 1e-12 * s[0]
    np.testing.assert_allclose(np.abs(kap @ D), np.linalg.norm(D, axis=0), rtol=1e-10)


def test_beta_zero_is_pure_decay_gdn_mamba2():
    S = RNG.standard_normal((7, 5))
    kap, q, v = _unit(7), _unit(7), RNG.standard_normal(5)
    for kind in (orc.GDN, orc.MAMBA2):
        Sn, o = orc.dense_step(kind, S, q, kap, v, 0.0, 0.625)
        np.testing.assert_array_equal(Sn, 0.625 * S)
        np.testing.assert_allclose(o, 0.625 * (S.T @ q), atol=1e-14)


def test_kda_gate_forgets_one_key_channel():
    dk, dv = 6, 4
    S = RNG.standard_normal((dk, dv))
    alpha = np.ones(dk)
    alpha[2] = 0.0
    Sn, _ = orc.dense_step(orc.KDA, S, _unit(dk), _unit(dk), RNG.standard_normal(dv), 0.0, alpha)
    assert np.all(Sn[2] == 0.0)                              # key channel 2 is forgotten
    np.testing.assert_array_equal(np.delete(Sn, 2, 0), np.delete(S, 2, 0))


@pytest.mark.parametrize("kind", [orc.GDN, orc.KDA, orc.MAMBA2])
def test_zero_decay_leaves_rank_one_write(kind):
    dk, dv = 9, 7
    S = RNG.standard_normal((dk, dv))
    kap, q, v = _unit(dk), _unit(dk), RNG.standard_normal(dv)
    g = np.zeros(dk) if kind == orc.KDA else 0.0
    Sn, o = orc.dense_step(kind, S, q, kap, v, 0.3, g)
    np.testing.assert_allclose(Sn, 0.3 * np.outer(kap, v), atol=1e-15)
    np.testing.assert_allclose(o, 0.3 * (kap @ q) * v, atol=1e-14)


def test_mamba2_constant_inputs_geometric_series():
    dk, dv = 5, 3
    kap = RNG.standard_normal(dk)
    v = RNG.standard_normal(dv)
    q = RNG.standard_normal(dk)
    g, beta = 0.8, 0.45
    S = np.zeros((dk, dv))
    for t in range(1, 30):
        S, o = orc.dense_step(orc.MAMBA2, S, q, kap, v, beta, g)
        closed = beta * np.outer(kap, v) * (1 - g ** t) / (1 - g)
        np.testing.assert_allclose(S, closed, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(o, closed.T @ q, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("kind", [orc.GDN, orc.KDA, orc.MAMBA2])
def test_transition_is_a_contraction_by_the_decay_bound(kind):
    dk, dv = 10, 6
    for _ in range(20):
        kap = _unit(dk)
        beta = RNG.uniform(0, 1)
        g = RNG.uniform(0.5, 1.0, size=dk) if kind == orc.KDA else RNG.uniform(0.5, 1.0)
        v = RNG.standard_normal(dv)
        X = RNG.standard_normal((dk, dv))
        # the step is affine in S: Phi(X) = step(X) - step(0)
        S1, _ = orc.dense_step(kind, X, kap, kap, v, beta, g)
        S0, _ = orc.dense_step(kind, np.zeros_like(X), kap, kap, v, beta, g)
        # spectral norm of the linear map on the key side bounds every column's shrinkage
        assert np.linalg.norm(S1 - S0, 2) <= orc.decay_bound(kind, g) * np.linalg.norm(X, 2) + 1e-12
