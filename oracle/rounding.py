"""Reference rounding of fp32 values to the 16-bit factor formats, and the random bits that
stochastic rounding draws.

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the test suite, the package's smoke check and the
benchmark's CPU-baseline leg may import or run it. It shares no code with the HIP path.

Sources:

* thelatestinai.com figures & tables, appendix table on number formats and rounding: the
  factors are stored in fp16 or bf16 with nearest or stochastic rounding. The pages fix neither
  the stochastic rule nor the random source; the readings below are the plainest ones.
* Philox4x32-10: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random numbers:
  as easy as 1, 2, 3", SC'11. A counter-based generator: ten rounds of two 32x32 -> 64-bit
  products with the multipliers 0xD2511F53 and 0xCD9E8D57, the key bumped between rounds by the
  Weyl constants 0x9E3779B9 and 0xBB67AE85.

Readings:

* A value x (fp32) lies between lo, its neighbour in the target format towards zero, and hi,
  the next value of the format away from zero (lo = hi = x when x is representable).
  Round-to-nearest takes the nearer of the two, the one with an even last bit on a tie.
  Stochastic rounding takes hi with probability f = (|x| - |lo|) / (|hi| - |lo|), decided by
  16 random bits r (an integer in [0, 65536)): hi exactly when r < f * 65536. When f * 65536 is
  an integer, which holds for every fp32 value in the normal range of either format, the
  expected result is x.
* The random bits of a stored element come from one Philox4x32-10 call whose key is
  (rng_key, 0) and whose counter words are:
      c0 = the element's index along the column, divided by 8 (the group of 8 elements);
      c1 = site << 16 | aux << 8 | slot (slot: the column slot written; site and aux: below);
      c2 = the unit;
      c3 = the unit's compression-window count (0 after the prefill-end compression, then one
           more after each compression).
  The four output words hold the group's eight 16-bit draws, element e taking the low (e even)
  or high (e odd) half of word (e % 8) // 2. Sites: 0 the decode step's new U column, 1 its new
  V column, 2 a compression's U', 3 its V', 4 the prefill-end U, 5 its V, 6 a KDA gate fold that
  rewrites a U column during decode step m (aux = m; aux is 0 at every other site).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "philox4x32", "sr_bits", "neighbors", "round_nearest", "round_stochastic", "BF16", "FP16",
    "SITE_DECODE_U", "SITE_DECODE_V", "SITE_COMPRESS_U", "SITE_COMPRESS_V", "SITE_FROM_DENSE_U",
    "SITE_FROM_DENSE_V", "SITE_FOLD_U",
]

BF16, FP16 = "bf16", "fp16"
SITE_DECODE_U, SITE_DECODE_V, SITE_COMPRESS_U, SITE_COMPRESS_V = 0, 1, 2, 3
SITE_FROM_DENSE_U, SITE_FROM_DENSE_V, SITE_FOLD_U = 4, 5, 6

_M32 = np.uint64(0xFFFFFFFF)


def _mulhilo(a: int, b):
    p = np.uint64(a) * b.astype(np.uint64)
    return (p >> np.uint64(32)) & _M32, p & _M32


def philox4x32(counter, key, rounds: int = 10):
    """Philox4x32 on arrays: counter is four uint32 arrays (broadcast together), key two uint32
    scalars or arrays. Returns the four output words as uint32 arrays."""
    c = [np.asarray(x, dtype=np.uint64) & _M32 for x in counter]
    c = list(np.broadcast_arrays(*c))
    k0 = np.asarray(key[0], dtype=np.uint64) & _M32
    k1 = np.asarray(key[1], dtype=np.uint64) & _M32
    for i in range(rounds):
        if i > 0:
            k0 = (k0 + np.uint64(0x9E3779B9)) & _M32
            k1 = (k1 + np.uint64(0xBB67AE85)) & _M32
        hi0, lo0 = _mulhilo(0xD2511F53, c[0])
        hi1, lo1 = _mulhilo(0xCD9E8D57, c[2])
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return [x.astype(np.uint32) for x in c]


def sr_bits(rng_key: int, unit, window, site: int, slot, elem, aux: int = 0):
    """The 16-bit draws (as int64) of the elements `elem` (array) of column `slot` of `unit`."""
    elem = np.asarray(elem, dtype=np.int64)
    c0 = elem // 8
    c1 = (np.int64(site) << 16) | (np.int64(aux) << 8) | np.asarray(slot, dtype=np.int64)
    words = philox4x32([c0, c1, np.asarray(unit, dtype=np.int64), np.asarray(window, dtype=np.int64)],
                       (rng_key, 0))
    w = np.stack(np.broadcast_arrays(*words), axis=0).astype(np.int64)   # [4, ...]
    e8 = np.broadcast_to(elem % 8, w.shape[1:])
    pick = np.take_along_axis(w, (e8 // 2)[None, ...], axis=0)[0]
    return np.where(e8 % 2 == 0, pick & 0xFFFF, (pick >> 16) & 0xFFFF)


def _bf16_neighbors(x32):
    """(lo, hi) in bf16 as float64: bf16 is the upper half of the fp32 encoding, so dropping the
    low 16 bits moves towards zero and adding one unit of the upper half moves away from it."""
    b = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lo_b = b & np.uint64(0xFFFF0000)
    exact = lo_b == b
    hi_b = np.where(exact, b, lo_b + np.uint64(0x10000))
    lo = lo_b.astype(np.uint32).view(np.float32).astype(np.float64)
    hi = hi_b.astype(np.uint32).view(np.float32).astype(np.float64)
    return lo, hi


def _fp16_neighbors(x32):
    """(lo, hi) in fp16 as float64, from NumPy's fp16 conversion and nextafter."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    h = x.astype(np.float16)                      # one of the two neighbours
    hd = h.astype(np.float64)
    with np.errstate(over="ignore"):   # the step away from 65504 is the infinity
        toward = np.nextafter(h, np.float16(0)).astype(np.float64)
        away = np.nextafter(h, np.where(x < 0, np.float16(-np.inf), np.float16(np.inf))).astype(np.float64)
    exact = hd == x
    h_is_hi = np.abs(hd) > np.abs(x)
    lo = np.where(exact, x, np.where(h_is_hi, toward, hd))
    hi = np.where(exact, x, np.where(h_is_hi, hd, away))
    return lo, hi


def neighbors(x32, fmt: str):
    """The two values of format fmt around each fp32 value: (towards zero, away from zero)."""
    return _bf16_neighbors(x32) if fmt == BF16 else _fp16_neighbors(x32)


def _last_bit_even(v, fmt):
    if fmt == BF16:
        bits = np.asarray(v, dtype=np.float32).view(np.uint32) >> np.uint32(16)
    else:
        bits = np.asarray(v, dtype=np.float16).view(np.uint16)
    return (bits & 1) == 0


def round_nearest(x32, fmt: str):
    """Round to nearest, ties to even (float64 values of the format)."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    lo, hi = neighbors(x32, fmt)
    dlo, dhi = np.abs(x - lo), np.abs(hi - x)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ~_last_bit_even(lo, fmt))
    return np.where(pick_hi, hi, lo)


def round_stochastic(x32, fmt: str, r16):
    """Stochastic rounding with 16-bit draws r16: hi exactly when r16 < f * 65536."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    lo, hi = neighbors(x32, fmt)
    span = np.abs(hi) - np.abs(lo)
    f = np.where(span > 0, (np.abs(x) - np.abs(lo)) / np.where(span > 0, span, 1.0), 0.0)
    return np.where(np.asarray(r16, dtype=np.float64) < f * 65536.0, hi, lo)
