"""Plant plausible mistakes in the oracle (on the CPU) and show the pins catch each.

Every mutant changes one step of the oracle through monkeypatching; the pin
suite must then fail at least once.  This is what makes the pins worth
trusting: a dropped term, a wrong sign, an off-by-one or a transposed index
anywhere in the oracle cannot pass unnoticed.
"""

import math

import numpy as np
import pytest

import oracle
import oracle.core as oa
import pins


def _attn(q, pos, kc, ks, vc, vs, sm_scale=None):
    return oa.attention(q, pos, kc, ks, vc, vs, sm_scale)


def _masked_rows_lt(qrows, pos, khat, vhat, sm_scale, chunk=256):
    # off by one: a row does not see its own position
    out = np.empty((qrows.shape[0], vhat.shape[1]))
    for i in range(qrows.shape[0]):
        T = int(pos[i])
        s = khat[:T] @ qrows[i] * sm_scale
        w = np.exp(s - (s.max() if T else 0.0))
        out[i] = (w @ vhat[:T]) / w.sum() if T else np.nan
    return out


def _masked_rows_no_norm(qrows, pos, khat, vhat, sm_scale, chunk=256):
    out = np.empty((qrows.shape[0], vhat.shape[1]))
    for i in range(qrows.shape[0]):
        T = int(pos[i]) + 1
        s = khat[:T] @ qrows[i] * sm_scale
        w = np.exp(s - s.max())
        out[i] = w @ vhat[:T]
    return out


def _masked_rows_wrong_sign(qrows, pos, khat, vhat, sm_scale, chunk=256):
    out = np.empty((qrows.shape[0], vhat.shape[1]))
    for i in range(qrows.shape[0]):
        T = int(pos[i]) + 1
        s = -(khat[:T] @ qrows[i]) * sm_scale
        w = np.exp(s - s.max())
        out[i] = (w @ vhat[:T]) / w.sum()
    return out


def _masked_rows_transposed_kv(qrows, pos, khat, vhat, sm_scale, chunk=256):
    # K and V swapped
    return oa.__dict__["_orig_masked_rows"](qrows, pos, vhat, khat, sm_scale, chunk)


def _dequant_mod(codes, scales):
    c = np.asarray(codes).astype(np.float64)
    s = np.asarray(scales).astype(np.float64)
    idx = np.arange(c.shape[-1]) % s.shape[-1]  # block index j % nb instead of j // 32
    return c * s[..., idx]


def _dequant_drop_scale(codes, scales):
    return np.asarray(codes).astype(np.float64)


MUTANTS = {
    "visibility_off_by_one": ("_masked_rows", _masked_rows_lt),
    "no_normalisation": ("_masked_rows", _masked_rows_no_norm),
    "wrong_sign_logits": ("_masked_rows", _masked_rows_wrong_sign),
    "k_v_swapped": ("_masked_rows", _masked_rows_transposed_kv),
    "gqa_modulo": ("kv_head_of", lambda h, hq, hkv: h % hkv),
    "gqa_divide_by_hkv": ("kv_head_of", lambda h, hq, hkv: min(h // hkv, hkv - 1)),
    "no_sm_scale": ("default_scale", lambda hd: 1.0),
    "sm_scale_1_over_hd": ("default_scale", lambda hd: 1.0 / hd),
    "block_index_modulo": ("dequantize", _dequant_mod),
    "scale_dropped": ("dequantize", _dequant_drop_scale),
}


def _run_all_checks():
    failures = []
    for check in pins.ATTENTION_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(_attn)
        except (AssertionError, ValueError, IndexError, FloatingPointError) as e:
            failures.append((check.__name__, str(e)[:80]))
    return failures


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setitem(oa.__dict__, "_orig_masked_rows", oa._masked_rows)
    monkeypatch.setattr(oa, attr, fn)
    failures = _run_all_checks()
    assert failures, f"mutant {name} passed every pin"


MERGE_MUTANTS = {
    "natural_exp": lambda m, l, o: _merge_with(m, l, o, np.exp),
    "ignores_l": lambda m, l, o: _merge_ignore_l(m, l, o),
    "min_reference_no_skip": lambda m, l, o: _merge_with(m, l, o, np.exp2, ref=np.min),
}


def _merge_with(m, l, o, ex, ref=np.max):
    M = ref(np.where(l > 0, m, -np.inf) if ref is np.max else m, axis=0)
    w = ex(m - M[None])
    return (w[..., None] * o).sum(0) / (w * l).sum(0)[..., None]


def _merge_ignore_l(m, l, o):
    M = np.max(m, axis=0)
    w = np.exp2(m - M[None])
    return (w[..., None] * o).sum(0) / w.sum(0)[..., None]


@pytest.mark.parametrize("name", sorted(MERGE_MUTANTS))
def test_merge_pins_catch_mutant(name):
    fn = MERGE_MUTANTS[name]
    failures = 0
    for check in (pins.check_merge_single, pins.check_merge_equal_m, pins.check_merge_base2,
                  pins.check_merge_empty):
        try:
            with np.errstate(all="ignore"):
                check(fn)
        except AssertionError:
            failures += 1
    assert failures, f"merge mutant {name} passed every pin"


def test_unmutated_oracle_passes_everything():
    assert _run_all_checks() == []
    assert math.isfinite(1.0)


@pytest.mark.parametrize("shift", [-1, 1])
def test_prompt_f16kv_position_mutants_fail(monkeypatch, shift):
    """prompt_f16kv with its chunk placed one key early or late fails its pins."""
    import test_oracle as T

    def bad(q, k, v, q_pos0, sm_scale=None, rows=None):
        n = np.asarray(q).shape[0]
        return oa.attention_values(q, max(0, q_pos0 + shift) + np.arange(n), oa._fp16(k), oa._fp16(v),
                                   sm_scale, rows)

    monkeypatch.setattr(oracle, "prompt_f16kv", bad)
    failed = 0
    for pin in (T.test_prompt_f16kv_positions_and_brute_force, T.test_prompt_f16kv_closed_forms):
        try:
            pin()
        except (AssertionError, IndexError, ValueError):
            failed += 1
    assert failed >= 1
