"""Pins of the oracle's truncation and compression (oracle steps O2, O3, O5).

The truncation is the plain definition of a compression to rank r: the best rank-r
approximation of the content (Eckart-Young). It is pinned by

* the Eckart-Young closed form |C - C_r|_F^2 = sum_{i>r} sigma_i^2, with the singular values
  cross-checked by an independent route (eigenvalues of C^T C);
* brute force over unit vectors on tiny heads;
* exact-rank inputs, which must be reproduced exactly;
* the sink split's identity S = a vbar^T + C with C vbar = 0 (Lemma 1).
"""
import itertools

import numpy as np
import pytest

import oracle as orc

RNG = np.random.default_rng(2024)


@pytest.mark.parametrize("dk,dv,r", [(12, 9, 3), (9, 12, 4), (16, 16, 8), (5, 5, 5), (6, 4, 6)])
def test_eckart_young_closed_form(dk, dv, r):
    C = RNG.standard_normal((dk, dv))
    U, V, err = orc.truncate(C, r)
    assert U.shape == (dk, r) and V.shape == (dv, r)
    lam = np.sort(np.linalg.eigvalsh(C.T @ C))[::-1]       # independent route to sigma^2
    lam = np.clip(lam, 0, None)
    tail = lam[r:].sum() if r < lam.size else 0.0
    np.testing.assert_allclose(err ** 2, tail, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(np.sum((C - U @ V.T) ** 2), tail, rtol=1e-9, atol=1e-12)
    # balanced factors: U^T U = V^T V = diag(sigma_1..sigma_r)
    kept = min(r, lam.size)
    sig = np.sqrt(lam[:kept])
    np.testing.assert_allclose(np.diag(U.T @ U)[:kept], sig, rtol=1e-9)
    np.testing.assert_allclose(U.T @ U, V.T @ V, atol=1e-10 * sig[0])
    off = U.T @ U - np.diag(np.diag(U.T @ U))
    assert np.abs(off).max() < 1e-10 * sig[0]


def _sphere_grid(d, n):
    if d == 2:
        th = np.linspace(0, np.pi, n, endpoint=False)
        return np.stack([np.cos(th), np.sin(th)], 1)
    th = np.linspace(0, np.pi, n)
    ph = np.linspace(0, 2 * np.pi, 2 * n, endpoint=False)
    T, P = np.meshgrid(th, ph)
    return np.stack([np.sin(T) * np.cos(P), np.sin(T) * np.sin(P), np.cos(T)], -1).reshape(-1, 3)


def _refine_best_z(C, z0, maximise=True):
    # local refinement of the brute-force optimum by random search around it
    z = z0 / np.linalg.norm(z0)
    best = np.linalg.norm(C @ z)
    step = 0.05
    loc = np.random.default_rng(5)
    for _ in range(3000):
        cand = z + step * loc.standard_normal(z.size)
        cand /= np.linalg.norm(cand)
        val = np.linalg.norm(C @ cand)
        if (val > best) if maximise else (val < best):
            z, best = cand, val
        else:
            step *= 0.995
    return z, best


@pytest.mark.parametrize("dk,dv", [(3, 2), (2, 3), (3, 3)])
def test_rank_one_truncation_matches_brute_force(dk, dv):
    for trial in range(3):
        C = RNG.standard_normal((dk, dv))
        # for a unit right vector z, the best approximation C z z^T leaves |C|^2 - |C z|^2
        grid = _sphere_grid(dv, 400)
        vals = np.linalg.norm(grid @ C.T, axis=1)
        z, best = _refine_best_z(C, grid[np.argmax(vals)], maximise=True)
        brute_err = np.sqrt(max(np.sum(C ** 2) - best ** 2, 0.0))
        U, V, err = orc.truncate(C, 1)
        assert abs(err - brute_err) <= 1e-6 * np.linalg.norm(C)
        np.testing.assert_allclose(U @ V.T, np.outer(C @ z, z), atol=1e-5 * np.linalg.norm(C))


def test_rank_two_of_three_matches_brute_force():
    C = RNG.standard_normal((3, 3))
    grid = _sphere_grid(3, 300)
    vals = np.linalg.norm(grid @ C.T, axis=1)
    _, smallest = _refine_best_z(C, grid[np.argmin(vals)], maximise=False)
    _, _, err = orc.truncate(C, 2)
    assert abs(err - smallest) <= 1e-6 * np.linalg.norm(C)


@pytest.mark.parametrize("rank,r", [(3, 3), (3, 5), (0, 2)])
def test_exact_rank_input_is_reproduced(rank, r):
    dk, dv = 10, 7
    C = RNG.standard_normal((dk, rank)) @ RNG.standard_normal((rank, dv))
    U, V, err = orc.truncate(C, r)
    assert U.shape == (dk, r)
    np.testing.assert_allclose(U @ V.T, C, atol=1e-12 * max(1.0, np.abs(C).max()))
    assert err <= 1e-12 * max(1.0, np.linalg.norm(C))
    # columns beyond the rank are zero
    assert np.allclose(U[:, rank:], 0, atol=1e-7) and np.allclose(V[:, rank:], 0, atol=1e-7)


def test_compress_is_truncation_of_the_product():
    dk, dv, m, r = 12, 10, 9, 4
    U = RNG.standard_normal((dk, m))
    V = RNG.standard_normal((dv, m))
    U2, V2, e = orc.compress(U, V, r)
    U3, V3, e3 = orc.truncate(U @ V.T, r)
    np.testing.assert_allclose(U2 @ V2.T, U3 @ V3.T, atol=1e-12)
    assert e == pytest.approx(e3)
    # products, never factors: any invertible mixing M of the r columns gives the same state
    M = RNG.standard_normal((r, r)) + 3 * np.eye(r)
    np.testing.assert_allclose((U2 @ M) @ (V2 @ np.linalg.inv(M).T).T, U2 @ V2.T, atol=1e-10)


@pytest.mark.parametrize("dk,dv", [(8, 8), (8, 5)])
def test_sink_split_identity(dk, dv):
    S = RNG.standard_normal((dk, dv))
    vbar = RNG.standard_normal(dv) * 0.3
    a, C = orc.sink_split(S, vbar)
    np.testing.assert_allclose(np.outer(a, vbar) + C, S, atol=1e-14)
    np.testing.assert_allclose(C @ vbar, 0, atol=1e-13)
    # only the direction of vbar matters
    a2, C2 = orc.sink_split(S, -5.0 * vbar)
    np.testing.assert_allclose(C2, C, atol=1e-13)


def test_optimality_criterion_accepts_ties_and_rejects_worse():
    # sigma = (3, 2, 2, 1): ranks 2 truncations are not unique (sigma_2 = sigma_3)
    Q1, _ = np.linalg.qr(RNG.standard_normal((6, 6)))
    Q2, _ = np.linalg.qr(RNG.standard_normal((5, 5)))
    s = np.array([3.0, 2.0, 2.0, 1.0])
    C = Q1[:, :4] @ np.diag(s) @ Q2[:, :4].T
    r = 2
    Ca = Q1[:, [0, 1]] @ np.diag([3.0, 2.0]) @ Q2[:, [0, 1]].T
    Cb = Q1[:, [0, 2]] @ np.diag([3.0, 2.0]) @ Q2[:, [0, 2]].T
    assert orc.relative_gap(C, r) < 1e-12
    assert orc.truncation_is_optimal(C, Ca, r, 1e-9)
    assert orc.truncation_is_optimal(C, Cb, r, 1e-9)
    worse = Q1[:, [0, 3]] @ np.diag([3.0, 1.0]) @ Q2[:, [0, 3]].T
    assert not orc.truncation_is_optimal(C, worse, r, 1e-3)
    assert not orc.truncation_is_optimal(C, C, r, 1e-3)            # rank 4 > r
    # a small perturbation of the optimum is accepted within delta and rejected beyond it
    P = Ca + 1e-3 * (Q1[:, [0]] @ Q2[:, [1]].T)
    assert orc.truncation_is_optimal(C, P, r, 1e-4)
    assert not orc.truncation_is_optimal(C, P, r, 1e-8)


def test_from_dense_full_rank_is_exact():
    for dk, dv in itertools.product((4, 7), (4, 6)):
        S = RNG.standard_normal((dk, dv))
        vbar = RNG.standard_normal(dv)
        a, U, V, err = orc.from_dense(S, vbar, min(dk, dv))
        np.testing.assert_allclose(orc.reconstruct(a, vbar, U, V), S, atol=1e-12)
        assert err < 1e-12


def test_singular_values_and_gap_of_a_known_spectrum():
    """A matrix built as P diag(s) Q^T with orthogonal P, Q has singular values s (sorted,
    non-negative, sign-free), and its relative gap at rank r is (s_r - s_{r+1}) / s_1."""
    rng = np.random.default_rng(7)
    s = np.array([5.0, -3.0, 2.0, 0.5])          # a negative entry flips one column's sign
    P, _ = np.linalg.qr(rng.standard_normal((6, 6)))
    Q, _ = np.linalg.qr(rng.standard_normal((4, 4)))
    C = P[:, :4] @ np.diag(s) @ Q.T
    got = orc.singular_values(C)
    assert np.allclose(got, [5.0, 3.0, 2.0, 0.5], atol=1e-12)
    assert orc.relative_gap(C, 2) == pytest.approx((3.0 - 2.0) / 5.0, abs=1e-12)
    assert orc.relative_gap(C, 4) == 1.0            # rank <= r
    assert orc.relative_gap(np.zeros((3, 3)), 1) == 1.0
