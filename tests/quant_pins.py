"""Pins for the oracle's block-32 int8 quantiser, independent of numpy's float arithmetic.

* ``exact_block``: the quantisation rule re-derived with exact rationals
  (``fractions.Fraction``) and IEEE round-to-nearest-even written from its
  definition (binary format with a p-bit significand, gradual underflow,
  overflow to infinity); it never calls a floating-point divide.
* constructed blocks whose codes follow from the rule by hand: exact .5 ties,
  neighbours one or two ulps from a tie, subnormal and underflowing scales,
  fp16 overflow, zero blocks;
* invariants: |x - scale * code| <= scale / 2 inside the code range, sign
  symmetry, power-of-two scaling of the input.

Neither fp32 divide can round onto a decision boundary it did not reach exactly:
an fp16 midpoint times 127, and (k + 0.5) times an fp16 scale, are fp32 values
with at most 19 significant bits, so any other fp32 numerator is at least one of
its ulps away, which is more than half an ulp of the quotient.  The fp32 steps
therefore give the exactly rounded results, and the exact derivation must agree
with the oracle everywhere, near ties included.

Each check takes ``quant(x) -> (codes, scales)`` so that planted mistakes in
the oracle can be run through the same checks.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

# (significand bits incl. the hidden one, exponent of the smallest normal, largest exponent)
FP32 = (24, -126, 127)
FP16 = (11, -14, 15)
INF = None  # marker for an overflowed rounding


def round_binary(v: Fraction, fmt):
    """IEEE round to nearest, ties to even, of an exact rational into a binary format.

    Returns a Fraction, or INF (with the sign lost: callers only round
    non-negative values to a format that can overflow).
    """
    p, emin, emax = fmt
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)  # below the normal range the quantum stays 2^(emin - p + 1)
    quantum = Fraction(2) ** (e - p + 1)
    n = a / quantum
    k = n.numerator // n.denominator
    rem = n - k
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and k % 2 == 1):
        k += 1
    r = k * quantum
    if r >= Fraction(2) ** (emax + 1):
        return INF
    return sign * r


def exact_block(xs):
    """The rule on one block of 32 exactly representable values: (codes list, scale or INF)."""
    fx = [Fraction(float(x)) for x in xs]
    amax = max(abs(v) for v in fx)
    d32 = round_binary(amax / 127, FP32)
    d16 = round_binary(d32, FP16)
    if d16 is INF:
        return [0] * len(fx), INF  # x / inf = 0 for every finite x
    if d16 == 0:
        return [0] * len(fx), Fraction(0)
    codes = []
    for v in fx:
        y = round_binary(v / d16, FP32)
        c = math.floor(abs(y) + Fraction(1, 2))
        c = min(c, 127)
        codes.append(c if y >= 0 else -c)
    return codes, d16


def _scale_value(s16) -> object:
    f = float(s16)
    return INF if math.isinf(f) else Fraction(f)


def check_against_exact(quant, blocks: np.ndarray):
    """blocks [n][32] fp32 or fp16: every code and scale equals the exact derivation."""
    codes, scales = quant(blocks)
    for i in range(blocks.shape[0]):
        ec, es = exact_block(blocks[i])
        got = [int(c) for c in codes[i]]
        assert got == ec, f"block {i}: codes {got} != {ec}"
        gs = _scale_value(scales[i, 0])
        assert gs == es, f"block {i}: scale {gs} != {es}"


def tie_blocks() -> np.ndarray:
    """Scales that are exact fp16 values and elements at exact .5 multiples of them."""
    out = []
    for d in (2.0 ** -4, 0.75, 3.0 * 2 ** -10, 1.0 + 2 ** -10):
        row = [127 * d] + [(k + 0.5) * d for k in range(-16, 15)]
        out.append(row)
        out.append([-v for v in row])
    return np.array(out, dtype=np.float32)


def near_tie_blocks(seed=11, n=64) -> np.ndarray:
    """Elements one or two fp32 ulps from (k + 0.5) * scale, for random fp16 scales."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        d = float(np.float16(rng.uniform(0.01, 4.0)))
        row = [127 * d]
        while len(row) < 32:
            k = int(rng.integers(-126, 126))
            t = np.float32((k + 0.5) * d)  # exact: <= 20 significant bits
            step = int(rng.choice([-2, -1, 1, 2]))
            v = t
            for _ in range(abs(step)):
                v = np.nextafter(v, np.float32(np.inf if step > 0 else -np.inf), dtype=np.float32)
            row.append(float(v))
        out.append(row)
    return np.array(out, dtype=np.float32)


def edge_blocks() -> np.ndarray:
    """Zero, subnormal-scale, underflowing-scale and fp16-overflow blocks."""
    rows = [
        [0.0] * 32,
        [0.0] * 31 + [-0.0],
        [1e-5 * (i - 16) for i in range(32)],  # scale in fp16's subnormal range
        [5e-6 * (1 if i % 2 else -1) for i in range(32)],  # scale rounds up to 2^-24, the smallest subnormal
        [5e-6 * ((i % 5) - 2) for i in range(32)],  # scale 2^-24 from amax 1e-5: codes clamp at 127
        [2e-9] * 32,  # amax / 127 below half the smallest subnormal: scale 0, codes 0
        [9e6] + [1.0] * 31,  # amax / 127 above 65504: scale +inf, codes 0
        [65504.0 * 127] + [-3.0] * 31,  # exactly the largest fp16 scale
        [3.4e38] + [1e30] * 31,
    ]
    return np.array(rows, dtype=np.float32)


def check_ties(quant):
    check_against_exact(quant, tie_blocks())
    # the hand rule: (k + 0.5) * d -> k + 1 for k >= 0, k for k < 0 (away from zero)
    b = tie_blocks()[:1]
    codes, scales = quant(b)
    assert float(scales[0, 0]) == 2.0 ** -4
    expect = [127] + [(k + 1) if k >= 0 else k for k in range(-16, 15)]
    assert [int(c) for c in codes[0]] == expect


def check_near_ties(quant):
    check_against_exact(quant, near_tie_blocks())


def check_edges(quant):
    b = edge_blocks()
    check_against_exact(quant, b)
    codes, scales = quant(b)
    assert not codes[0].any() and float(scales[0, 0]) == 0.0
    assert not codes[5].any() and float(scales[5, 0]) == 0.0
    assert math.isinf(float(scales[6, 0])) and not codes[6].any()
    assert float(scales[7, 0]) == 65504.0 and int(codes[7, 0]) == 127
    assert int(np.abs(codes[4]).max()) == 127  # clamped


def check_random_exact(quant):
    rng = np.random.default_rng(13)
    b = np.concatenate([
        rng.standard_normal((40, 32)).astype(np.float32),
        (rng.standard_normal((20, 32)) * 10.0 ** rng.integers(-6, 6, (20, 1))).astype(np.float32),
    ])
    check_against_exact(quant, b)
    check_against_exact(quant, rng.standard_normal((30, 32)).astype(np.float16))


def check_error_bound(quant):
    rng = np.random.default_rng(14)
    x = (rng.standard_normal((64, 256)) * 10.0 ** rng.integers(-3, 3, (64, 1))).astype(np.float32)
    codes, scales = quant(x)
    d = np.repeat(scales.astype(np.float64), 32, axis=-1)
    err = np.abs(x.astype(np.float64) - d * codes)
    # |x/d - code| <= 1/2 up to the fp32 quotient's own rounding
    assert np.all(err <= d * (0.5 + 2.0 ** -16))
    assert np.all(np.abs(codes.reshape(64, 8, 32)).max(-1) == 127)


def check_sign_symmetry(quant):
    rng = np.random.default_rng(15)
    x = rng.standard_normal((16, 128)).astype(np.float32)
    c1, s1 = quant(x)
    c2, s2 = quant(-x)
    assert np.array_equal(c1, -c2) and np.array_equal(s1, s2)


def check_pow2_scaling(quant):
    rng = np.random.default_rng(16)
    x = rng.standard_normal((16, 64)).astype(np.float32)
    c1, s1 = quant(x)
    c2, s2 = quant(x * np.float32(8.0))
    assert np.array_equal(c1, c2)
    assert np.array_equal(s1.astype(np.float32) * 8, s2.astype(np.float32))


def check_block_boundaries(quant):
    """One large element per block sets that block's scale only."""
    x = np.ones((1, 128), dtype=np.float32)
    x[0, 40] = 100.0
    codes, scales = quant(x)
    s = scales[0].astype(np.float64)
    assert s[0] == s[2] == s[3] != s[1]
    assert int(codes[0, 40]) == 127 and int(codes[0, 0]) == 127 and int(codes[0, 33]) == 1


QUANT_CHECKS = [check_ties, check_near_ties, check_edges,
                check_random_exact, check_error_bound, check_sign_symmetry, check_pow2_scaling,
                check_block_boundaries]
