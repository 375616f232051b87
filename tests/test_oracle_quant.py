"""The oracle's KV quantiser against its pins, and planted mistakes that the pins must catch."""

import numpy as np
import pytest

import oracle
import oracle.quant as oq
import quant_pins as qp


@pytest.mark.parametrize("check", qp.QUANT_CHECKS, ids=lambda c: c.__name__)
def test_quant_pin(check):
    check(oracle.quantize_q8)


def test_exact_rounding_helper():
    """The rational IEEE rounding against values whose fp32 / fp16 encodings are known."""
    from fractions import Fraction as F

    assert qp.round_binary(F(1, 3), qp.FP32) == F(11184811, 2 ** 25)  # 0x3EAAAAAB
    assert qp.round_binary(F(1, 3), qp.FP16) == F(1365, 2 ** 12)  # 0x3555
    assert qp.round_binary(F(65520), qp.FP16) is qp.INF  # halfway to 2^16 rounds up: overflow
    assert qp.round_binary(F(65519), qp.FP16) == 65504
    assert qp.round_binary(F(1, 2 ** 25), qp.FP16) == 0  # tie with zero goes to even
    assert qp.round_binary(F(3, 2 ** 26), qp.FP16) == F(1, 2 ** 24)
    assert qp.round_binary(F(2049), qp.FP16) == 2048  # tie to even
    assert qp.round_binary(F(2051), qp.FP16) == 2052


def test_kv_append_places_rows():
    rng = np.random.default_rng(3)
    T, H, hd, S, p0 = 5, 3, 64, 20, 7
    x = rng.standard_normal((T, H, hd)).astype(np.float32)
    codes = np.full((H, S, hd), 55, np.int8)
    scales = np.full((H, S, hd // 32), 1.5, np.float16)
    c2, s2 = oracle.kv_append(x, codes, scales, p0)
    for h in range(H):
        for t in range(T):
            cc, ss = oracle.quantize_q8(x[t, h][None])
            assert np.array_equal(c2[h, p0 + t], cc[0]) and np.array_equal(s2[h, p0 + t], ss[0])
    untouched = np.ones(S, bool)
    untouched[p0:p0 + T] = False
    assert (c2[:, untouched] == 55).all() and (s2[:, untouched] == np.float16(1.5)).all()
    with pytest.raises(ValueError):
        oracle.kv_append(x, codes, scales, S - T + 1)


# ---- planted mistakes -------------------------------------------------------------


def _variant(round_fn=None, recip=False, scale16=True, clamp=True, const=127.0, per_row=False):
    def quant(x):
        x = np.asarray(x)
        hd = x.shape[-1]
        b = x.astype(np.float32).reshape(x.shape[:-1] + (hd // 32, 32))
        amax = np.max(np.abs(b), axis=-1)
        if per_row:
            amax = np.repeat(amax.max(-1, keepdims=True), hd // 32, axis=-1)
        with np.errstate(all="ignore"):
            s = (amax / np.float32(const)).astype(np.float16)
            d = s.astype(np.float32) if scale16 else (amax / np.float32(const))
            y = b * (np.float32(1) / d)[..., None] if recip else b / d[..., None]
            yd = y.astype(np.float64)
            r = round_fn(yd) if round_fn else np.sign(yd) * np.floor(np.abs(yd) + 0.5)
            if clamp:
                r = np.clip(r, -127, 127)
            r = np.where(d[..., None] == 0, 0.0, r)
            r = np.nan_to_num(r, nan=0.0, posinf=127, neginf=-127)
            r = np.clip(r, -128, 127)
        return r.astype(np.int8).reshape(x.shape), s

    return quant


QUANT_MUTANTS = {
    "ties_to_even": _variant(round_fn=np.rint),
    "truncate": _variant(round_fn=np.trunc),
    "floor": _variant(round_fn=np.floor),
    "reciprocal_multiply": _variant(recip=True),
    "unrounded_fp32_scale": _variant(scale16=False),
    "no_clamp": _variant(clamp=False),
    "divide_by_128": _variant(const=128.0),
    "row_wide_amax": _variant(per_row=True),
}


@pytest.mark.parametrize("name", sorted(QUANT_MUTANTS))
def test_quant_pins_catch_mutant(name):
    fn = QUANT_MUTANTS[name]
    failures = 0
    for check in qp.QUANT_CHECKS:
        try:
            check(fn)
        except AssertionError:
            failures += 1
    assert failures, f"quantiser mutant {name} passed every pin"


def test_unmutated_variant_passes():
    for check in qp.QUANT_CHECKS:
        check(_variant())


def test_oracle_module_is_the_one_checked():
    assert oq.quantize_q8 is oracle.quantize_q8
