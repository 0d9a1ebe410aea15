"""Pins of the oracle's chunked update, and of the chunked form the HIP kernel evaluates.

A chunk of tokens is defined by its Lemma 2 steps taken in turn (picx.dev summary, "Exact
Update (Lemma 2)"), so oracle.factored_chunk is that loop. It is pinned here against the dense
recurrence (pinned on its own by its closed forms): after every chunk the factored state
a vbar^T + U V^T equals the dense state, and each read-out equals the dense one.

The HIP kernel does not loop over tokens: it solves one triangular system per chunk (the reading
written out in _chunk_closed_form below, from Lemma 1: the sink coefficient and the content
each follow the head's recurrence). That form is checked against the loop in float64, so the
algebra of the kernel is settled before any GPU run.
"""
import numpy as np
import pytest

import oracle as orc
import synth


def _relF(A, B):
    return np.linalg.norm(A - B) / max(np.linalg.norm(B), 1e-300)


def _inputs(kind, dk, dv, steps, seed):
    w = synth.Workload("t", kind, 1, 1, dk, dv, 4, 4, 64, 16, synth.F32, synth.F32)
    xs = synth.sequence(w, seed=seed, steps=steps, units=1)
    return w, [{k: (v[0] if np.ndim(v) else v) for k, v in x.items()} for x in xs]


def _start_state(kind, dk, dv, seed, m=6):
    """A factored state with m columns, a non-zero sink and unequal column norms."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(dk)
    U = rng.standard_normal((dk, m)) * np.linspace(1.0, 0.2, m)
    V = rng.standard_normal((dv, m))
    vbar = rng.standard_normal(dv) + 2.0
    V -= np.outer(vbar, vbar @ V) / (vbar @ vbar)     # content orthogonal to vbar (Lemma 1)
    return a, U, V, vbar


@pytest.mark.parametrize("kind", [orc.GDN, orc.MAMBA2, orc.KDA])
@pytest.mark.parametrize("L", [1, 5, 17])
def test_chunk_equals_dense_recurrence(kind, L):
    dk, dv = 12, 8
    _, xs = _inputs(kind, dk, dv, L, seed=40 + L)
    a, U, V, vbar = _start_state(kind, dk, dv, seed=L)
    S0 = orc.reconstruct(a, vbar, U, V)
    Ss, os_ = orc.run_dense(kind, S0, xs)
    a1, U1, V1, outs = orc.factored_chunk(kind, a, U, V, vbar, xs)
    assert U1.shape[1] == U.shape[1] + L and V1.shape[1] == V.shape[1] + L
    assert _relF(orc.reconstruct(a1, vbar, U1, V1), Ss[-1]) <= 1e-12
    for o_t, od_t in zip(outs, os_):
        assert np.linalg.norm(o_t - od_t) <= 1e-12 * np.linalg.norm(od_t)


def _chunk_closed_form(kind, a, U, V, vbar, xs):
    """The chunked form of the HIP kernel in float64 (scalar-decay kinds).

    Gamma(t, s) = prod_{s < u <= t} g_u, gamma_t = Gamma(t, -1);
    (I + A) c = beta (omega - gamma a . kappa), (I + A) W = beta (eps - gamma V U^T kappa),
    A[t][s] = beta_t Gamma(t, s) kappa_t . kappa_s for s < t (Mamba-2: A = 0, no state terms);
    o_t = vbar (gamma_t a . q_t + sum_{s<=t} Gamma(t,s) (q_t . kappa_s) c_s)
          + gamma_t V U^T q_t + sum_{s<=t} Gamma(t,s) (q_t . kappa_s) w_s.
    The new columns kappa_s carry the decay Gamma(L-1, s); the old state takes gamma_{L-1}.
    """
    L = len(xs)
    K = np.stack([x["k"] for x in xs])           # L x dk
    Q = np.stack([x["q"] for x in xs])
    Vin = np.stack([x["v"] for x in xs])         # L x dv
    beta = np.array([x["beta"] for x in xs], dtype=float)
    g = np.array([x["g"] for x in xs], dtype=float)
    G = np.zeros((L, L + 1))                     # G[t, s + 1] = Gamma(t, s)
    for t in range(L):
        for s in range(-1, t + 1):
            G[t, s + 1] = np.prod(g[s + 1:t + 1])
    gam = G[:, 0]
    delta = kind != orc.MAMBA2
    omega = Vin @ vbar / (vbar @ vbar)
    eps = Vin - np.outer(omega, vbar)
    A = np.zeros((L, L))
    if delta:
        for t in range(L):
            for s in range(t):
                A[t, s] = beta[t] * G[t, s + 1] * (K[t] @ K[s])
    Rc = beta * (omega - (gam * (K @ a) if delta else 0.0))
    RW = beta[:, None] * (eps - ((gam[:, None] * (K @ U) @ V.T) if delta else 0.0))
    M = np.eye(L) + A
    c = np.linalg.solve(M, Rc)
    W = np.linalg.solve(M, RW)                   # L x dv
    QK = np.array([[G[t, s + 1] * (Q[t] @ K[s]) if s <= t else 0.0 for s in range(L)] for t in range(L)])
    outs = [vbar * (gam[t] * (Q[t] @ a) + QK[t] @ c) + gam[t] * (V @ (U.T @ Q[t])) + QK[t] @ W
            for t in range(L)]
    scale_new = np.array([G[L - 1, s + 1] for s in range(L)])
    U1 = np.concatenate([gam[-1] * U, K.T * scale_new[None, :]], axis=1)
    V1 = np.concatenate([V, W.T], axis=1)
    a1 = gam[-1] * a + K.T @ (scale_new * c)
    return a1, U1, V1, outs


@pytest.mark.parametrize("kind", [orc.GDN, orc.MAMBA2])
@pytest.mark.parametrize("L", [1, 2, 7, 32])
def test_closed_form_equals_token_loop(kind, L):
    dk, dv = 16, 12
    _, xs = _inputs(kind, dk, dv, L, seed=60 + L + kind)
    if L >= 7:
        xs[3]["g"] = 0.0                         # a token that forgets everything before it
    a, U, V, vbar = _start_state(kind, dk, dv, seed=100 + L)
    a1, U1, V1, outs = orc.factored_chunk(kind, a, U, V, vbar, xs)
    b1, X1, Y1, outs2 = _chunk_closed_form(kind, a, U, V, vbar, xs)
    np.testing.assert_allclose(b1, a1, rtol=1e-10, atol=1e-12 * np.abs(a1).max())
    # the appended columns themselves (not only the product): the kernel writes exactly these
    np.testing.assert_allclose(Y1, V1, rtol=1e-9, atol=1e-11 * np.abs(V1).max())
    np.testing.assert_allclose(X1, U1, rtol=1e-12, atol=1e-14)
    for o1, o2 in zip(outs, outs2):
        np.testing.assert_allclose(o2, o1, rtol=1e-9, atol=1e-11 * max(np.abs(o1).max(), 1e-300))
