"""Pins for the oracle's greedy head (token, top probability), independent of numpy.

* ``brute``: pure-Python loops with ``math.exp`` over the rule (first index of
  the largest non-NaN value; 1 / sum exp(x - max) over non-NaN entries);
* closed forms: a constant row (token 0, top 1/V), one high value above a
  constant rest (1 / (1 + (V-1) e^-gap)), two levels with multiplicities,
  -inf masks (1 / number of unmasked equal entries);
* special rows: all NaN, all -inf, NaN beside the maximum, ties;
* invariants: a shift of every logit leaves the token and top probability,
  a permutation moves the token with the maximum.

Each check takes ``head(logits) -> (token, top)`` so planted mistakes can be
run through the same checks.
"""

from __future__ import annotations

import math

import numpy as np


def brute(row):
    best, idx = None, -1
    for i, v in enumerate(row):
        v = float(v)
        if math.isnan(v):
            continue
        if best is None or v > best:
            best, idx = v, i
    if idx < 0 or best == -math.inf:
        return idx, math.nan
    s = 0.0
    for v in row:
        v = float(v)
        if not math.isnan(v):
            s += math.exp(v - best)
    return idx, 1.0 / s


def _close(a, b, tol=1e-12):
    if math.isnan(b):
        return math.isnan(a)
    return abs(a - b) <= tol * abs(b)


def special_rows():
    nan, ninf = np.nan, -np.inf
    rows = [
        [1.0, 3.0, 3.0, 2.0, -1.0, 3.0, 0.5, 0.0],   # ties: first of three
        [nan, 2.0, nan, 2.5, 2.5, nan, 1.0, -3.0],    # NaN beside the maximum
        [nan] * 8,                                     # nothing valid: -1, NaN
        [ninf] * 8,                                    # all masked: 0, NaN
        [nan, ninf, nan, ninf, nan, nan, nan, nan],    # -inf and NaN: 1, NaN
        [ninf, ninf, 4.0, ninf, ninf, 4.0, ninf, 4.0],  # masked but for three ties
        [-1e30, -1e30, -1e30, -1e30, -1e30, -1e30, -1e30, -2e30],
        [0.0, -0.0, 0.0, -0.0, 0.0, 0.0, 0.0, 0.0],   # signed zeros tie
    ]
    return np.array(rows, dtype=np.float32)


def check_brute_force(head):
    rng = np.random.default_rng(31)
    rows = [special_rows()]
    for V in (1, 2, 7, 33, 100):
        x = (rng.standard_normal((3, V)) * 3).astype(np.float32)
        x[0, rng.integers(0, V)] = np.nan
        x[1, rng.integers(0, V)] = -np.inf
        x[2] = np.round(x[2])  # many ties
        rows.append(x)
    for x in rows:
        tok, top = head(x)
        for r in range(x.shape[0]):
            bi, bt = brute(x[r])
            assert int(tok[r]) == bi, f"token {tok[r]} != {bi} for {x[r]}"
            assert _close(float(top[r]), bt), f"top {top[r]} != {bt}"


def check_constant_row(head):
    V = 1000
    x = np.full((2, V), 0.75, dtype=np.float32)
    x[1] = -12.5
    tok, top = head(x)
    assert list(tok) == [0, 0]
    assert _close(float(top[0]), 1.0 / V) and _close(float(top[1]), 1.0 / V)


def check_one_high(head):
    V, gap = 5000, 3.0
    x = np.zeros((1, V), dtype=np.float32)
    x[0, 1234] = gap
    tok, top = head(x)
    assert int(tok[0]) == 1234
    assert _close(float(top[0]), 1.0 / (1.0 + (V - 1) * math.exp(-gap)))


def check_two_levels(head):
    a, b, gap = 7, 993, 1.5
    x = np.full((1, a + b), -2.0, dtype=np.float32)
    x[0, 100:100 + a] = -2.0 + gap
    tok, top = head(x)
    assert int(tok[0]) == 100
    assert _close(float(top[0]), 1.0 / (a + b * math.exp(-gap)))


def check_masks(head):
    V = 64
    x = np.full((1, V), -np.inf, dtype=np.float32)
    x[0, [5, 9, 40, 41]] = 1.25
    tok, top = head(x)
    assert int(tok[0]) == 5 and _close(float(top[0]), 0.25)


def check_special(head):
    tok, top = head(special_rows())
    assert list(tok) == [1, 3, -1, 0, 1, 2, 0, 0]
    assert math.isnan(top[2]) and math.isnan(top[3]) and math.isnan(top[4])
    assert _close(float(top[5]), 1.0 / 3.0)
    assert _close(float(top[7]), 1.0 / 8.0)


def check_shift(head):
    rng = np.random.default_rng(32)
    # multiples of 2^-12 below 64 in magnitude: adding 64 is exact in fp32
    x = (np.round(rng.standard_normal((4, 3000)) * 2 * 4096) / 4096).astype(np.float32)
    t1, p1 = head(x)
    t2, p2 = head(x + np.float32(64.0))
    assert np.array_equal(t1, t2)
    assert np.allclose(p1, p2, rtol=1e-12, atol=0)


def check_permutation(head):
    rng = np.random.default_rng(33)
    x = (rng.standard_normal((3, 2000)) * 2).astype(np.float32)
    perm = rng.permutation(2000)
    t1, p1 = head(x)
    t2, p2 = head(x[:, perm])
    inv = np.argsort(perm)
    assert np.array_equal(inv[t1], t2)
    assert np.allclose(p1, p2, rtol=1e-12, atol=0)


HEAD_CHECKS = [check_brute_force, check_constant_row, check_one_high, check_two_levels,
               check_masks, check_special, check_shift, check_permutation]
