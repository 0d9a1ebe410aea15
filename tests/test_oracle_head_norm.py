"""Pins of the oracle's head normalisation (picx.dev summary, "Theoretical and Practical
Implications", practical implications: the sink acts as a bias and gain through the head's
normalization). Each pin is fixed by something other than the function's own formula: values
worked by hand, invariances, torch's own rms_norm and sigmoid, and the decomposition of a
factored read-out into its sink and content parts."""
import numpy as np
import pytest

import oracle as orc


def test_constant_vector_worked_by_hand():
    # o = (3, 3, 3, 3): mean square 9, eps 7 -> rms 4 -> y = 3/4 * w
    w = np.array([1.0, 2.0, -1.0, 0.5])
    y = orc.head_norm(np.full(4, 3.0), w, eps=7.0)
    assert np.allclose(y, 0.75 * w, rtol=1e-15, atol=0)
    # o = (1, -1, 1, -1), eps 0: rms 1 -> y = o * w
    o = np.array([1.0, -1.0, 1.0, -1.0])
    assert np.allclose(orc.head_norm(o, w, eps=0.0), o * w, rtol=1e-15)


def test_silu_values():
    assert orc.silu(0.0) == 0.0
    assert orc.silu(np.log(3.0)) == pytest.approx(np.log(3.0) * 0.75, rel=1e-15)   # sigmoid(ln 3) = 3/4
    assert orc.silu(-np.log(3.0)) == pytest.approx(-np.log(3.0) * 0.25, rel=1e-15)
    assert orc.silu(40.0) == pytest.approx(40.0, rel=1e-15)


def test_scale_invariance_and_rms_one():
    rng = np.random.default_rng(3)
    o = rng.standard_normal(128)
    w = rng.uniform(0.5, 1.5, 128)
    y = orc.head_norm(o, np.ones(128), eps=0.0)
    assert np.sqrt(np.mean(y * y)) == pytest.approx(1.0, rel=1e-14)
    assert np.allclose(orc.head_norm(37.0 * o, w, eps=0.0), orc.head_norm(o, w, eps=0.0), rtol=1e-13)
    # eps > 0 breaks the invariance towards small outputs: a tiny read-out stays tiny
    assert np.linalg.norm(orc.head_norm(1e-6 * o, w, eps=1e-2)) < 1e-3


def test_against_torch_rms_norm_and_sigmoid():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    o = rng.standard_normal((6, 64))
    w = rng.uniform(0.5, 1.5, 64)
    z = rng.standard_normal((6, 64))
    ot, wt, zt = (torch.tensor(x, dtype=torch.float64) for x in (o, w, z))
    ref = torch.nn.functional.rms_norm(ot, (64,), wt, eps=1e-5)
    gated_after = ref * zt * torch.sigmoid(zt)
    x = ot * zt * torch.sigmoid(zt)
    gated_first = torch.nn.functional.rms_norm(x, (64,), wt, eps=1e-5)
    for u in range(6):
        assert np.allclose(orc.head_norm(o[u], w, 1e-5), ref[u].numpy(), rtol=1e-13, atol=1e-15)
        assert np.allclose(orc.head_norm(o[u], w, 1e-5, gate=z[u]), gated_after[u].numpy(), rtol=1e-13, atol=1e-15)
        assert np.allclose(orc.head_norm(o[u], w, 1e-5, gate=z[u], gate_first=True), gated_first[u].numpy(),
                           rtol=1e-13, atol=1e-15)


def test_sink_is_a_bias_and_a_gain():
    # A factored read-out o = vbar (a^T q) + V (U^T q), with the content orthogonal to vbar
    # (Lemma 1's split): the normalised output's content part is the content read-out times
    # 1 / rms, and rms^2 = (|content|^2 + (a^T q)^2 |vbar|^2) / d_v, so a stronger sink lowers the
    # content's gain; the vbar part is the sink's fixed-direction bias.
    rng = np.random.default_rng(11)
    dk, dv, m = 16, 8, 3
    vbar = rng.standard_normal(dv)
    vbar /= np.linalg.norm(vbar)
    U = rng.standard_normal((dk, m))
    V = rng.standard_normal((dv, m))
    V -= np.outer(vbar, vbar @ V)                 # content orthogonal to vbar
    q = rng.standard_normal(dk)
    a = rng.standard_normal(dk)
    content = V @ (U.T @ q)
    gains = []
    for s in (0.0, 1.0, 4.0):
        o = orc.readout(orc.reconstruct(s * a, vbar, U, V), q)
        y = orc.head_norm(o, np.ones(dv), eps=0.0)
        bias = s * (a @ q)
        rms = np.sqrt((content @ content + bias * bias) / dv)
        assert np.allclose(y - vbar * (vbar @ y), content / rms, rtol=1e-12, atol=1e-14)
        assert vbar @ y == pytest.approx(bias / rms, rel=1e-12, abs=1e-14)
        gains.append(1.0 / rms)
    assert gains[0] > gains[1] > gains[2]
    # a pure sink state normalises to the fixed direction, whatever its magnitude
    o = orc.readout(orc.reconstruct(a, vbar, U * 0.0, V), q)
    y = orc.head_norm(o, np.ones(dv), eps=0.0)
    assert np.allclose(np.abs(y), np.abs(vbar) * np.sqrt(dv), rtol=1e-12)
