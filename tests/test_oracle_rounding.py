"""Pins of the oracle's rounding to the 16-bit factor formats and of its random source.

Philox4x32-10 is pinned to its published known-answer vectors. Round-to-nearest is pinned to
library conversions (NumPy's fp16, torch's bf16 on the CPU). Stochastic rounding is pinned by
its defining properties: the result is one of the two neighbouring values, representable values
are kept, the probability of rounding away from zero is the fractional distance, and the mean
over all 65,536 draws is the value itself.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

from oracle import rounding as rd

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def _kat():
    rows = []
    with open(GOLDEN) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                w = [int(x, 16) for x in line.split()]
                rows.append((w[:4], w[4:6], w[6:10]))
    return rows


def test_philox_known_answers():
    rows = _kat()
    assert len(rows) == 3
    for ctr, key, out in rows:
        got = rd.philox4x32([np.uint32(c) for c in ctr], key)
        assert [int(x) for x in got] == out


def test_philox_vectorised_matches_scalar_calls():
    ctr = np.arange(37, dtype=np.int64)
    words = rd.philox4x32([ctr, 5, 7, 11], (123, 0))
    for i in (0, 1, 17, 36):
        one = rd.philox4x32([np.uint32(i), np.uint32(5), np.uint32(7), np.uint32(11)], (123, 0))
        assert [int(w[i]) for w in words] == [int(x) for x in one]


def test_sr_bits_layout():
    """Element e of a column takes half (e % 2) of word (e % 8) // 2 of the call for group e // 8."""
    e = np.arange(24)
    r = rd.sr_bits(99, 3, 4, rd.SITE_DECODE_V, 17, e)
    for g in range(3):
        w = rd.philox4x32([np.uint32(g), np.uint32((rd.SITE_DECODE_V << 16) | 17), np.uint32(3),
                           np.uint32(4)], (99, 0))
        for k in range(8):
            word = int(w[k // 2])
            assert r[8 * g + k] == ((word >> (16 * (k % 2))) & 0xFFFF)
    # the aux byte and the site separate otherwise equal counters
    assert not np.array_equal(r, rd.sr_bits(99, 3, 4, rd.SITE_DECODE_U, 17, e))
    assert not np.array_equal(rd.sr_bits(99, 3, 4, rd.SITE_FOLD_U, 17, e, aux=40),
                              rd.sr_bits(99, 3, 4, rd.SITE_FOLD_U, 17, e, aux=41))


def _samples(n=20000, seed=5):
    g = np.random.default_rng(seed)
    x = g.standard_normal(n) * np.exp2(g.integers(-20, 12, n))
    return np.concatenate([x, [0.0, -0.0, 1.0, -1.0, 65504.0, 3.0e-8, -7.0e-6]]).astype(np.float32)


def test_round_nearest_fp16_matches_numpy():
    x = _samples()
    assert np.array_equal(rd.round_nearest(x, rd.FP16), x.astype(np.float16).astype(np.float64))


def test_round_nearest_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    x = _samples()
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(rd.round_nearest(x, rd.BF16), ref)


def test_round_nearest_bf16_ties_to_even():
    one = np.float32(1.0)
    half_ulp = np.float32(2.0 ** -8)   # bf16 keeps 7 fraction bits: its unit at 1 is 2^-7
    assert rd.round_nearest(np.float32(one + half_ulp), rd.BF16) == 1.0
    assert rd.round_nearest(np.float32(one + 3 * half_ulp), rd.BF16) == 1.0 + 2 * 2.0 ** -7


@pytest.mark.parametrize("fmt", [rd.BF16, rd.FP16])
def test_stochastic_rounding_properties(fmt):
    x = _samples(4000)
    lo, hi = rd.neighbors(x, fmt)
    xd = x.astype(np.float64)
    assert np.all(np.abs(lo) <= np.abs(xd)) and np.all(np.abs(xd) <= np.abs(hi))
    g = np.random.default_rng(7)
    r = g.integers(0, 65536, x.shape)
    y = rd.round_stochastic(x, fmt, r)
    assert np.all((y == lo) | (y == hi))
    # representable values are kept whatever the draw
    rep = rd.round_nearest(x, fmt).astype(np.float32)
    for rr in (0, 12345, 65535):
        assert np.array_equal(rd.round_stochastic(rep, fmt, np.full(x.shape, rr)), rep.astype(np.float64))


@pytest.mark.parametrize("fmt", [rd.BF16, rd.FP16])
def test_stochastic_rounding_is_unbiased_over_all_draws(fmt):
    """In the normal range f * 65536 is an integer, so the mean over every draw is exactly x."""
    g = np.random.default_rng(11)
    x = (g.standard_normal(64) * (1.0 if fmt == rd.FP16 else 1e3)).astype(np.float32)
    r = np.arange(65536)
    for xi in x:
        y = rd.round_stochastic(np.full(r.shape, xi, dtype=np.float32), fmt, r)
        assert y.mean() == pytest.approx(float(xi), rel=0, abs=1e-12 * max(1.0, abs(float(xi))))
        lo, hi = rd.neighbors(np.float32(xi), fmt)
        if hi != lo:
            f = (abs(float(xi)) - abs(float(lo))) / (abs(float(hi)) - abs(float(lo)))
            assert np.count_nonzero(y == hi) == int(round(f * 65536))


def test_stochastic_rounding_bf16_matches_the_carry_rule():
    """For bf16 the rule equals adding the draw's complement to the dropped half and carrying:
    hi exactly when r < low16(x)."""
    x = _samples(3000)
    g = np.random.default_rng(13)
    r = g.integers(0, 65536, x.shape)
    low = x.view(np.uint32) & 0xFFFF
    lo, hi = rd.neighbors(x, rd.BF16)
    expect = np.where(r < low, hi, lo)
    assert np.array_equal(rd.round_stochastic(x, rd.BF16, r), expect)
