"""The oracle against its pins (CPU only)."""

import numpy as np
import pytest

import oracle
import pins


def _attn(q, pos, kc, ks, vc, vs, sm_scale=None):
    return oracle.attention(q, pos, kc, ks, vc, vs, sm_scale)


@pytest.mark.parametrize("check", pins.ATTENTION_CHECKS, ids=lambda f: f.__name__)
def test_attention_pin(check):
    check(_attn)


@pytest.mark.parametrize(
    "check",
    [pins.check_merge_single, pins.check_merge_equal_m, pins.check_merge_base2,
     pins.check_merge_empty],
    ids=lambda f: f.__name__,
)
def test_merge_pin(check):
    check(oracle.merge_partials)


def test_split_invariance():
    pins.check_split_invariance(_attn, oracle.split_partials, oracle.merge_partials)


def test_verify_and_prompt_positions():
    """verify() puts row r at ctx+r; prompt() puts query i at q_pos0+i."""
    q, kc, ks, vc, vs = pins.random_case(40, 3, 4, 2, 64, 20)
    a = oracle.verify(q, kc, ks, vc, vs, ctx_len=10)
    b = oracle.attention(q, [10, 11, 12], kc, ks, vc, vs)
    assert np.array_equal(a, b)
    c = oracle.prompt(q.astype(np.float16), kc, ks, vc, vs, q_pos0=4)
    d = oracle.attention(q.astype(np.float16), [4, 5, 6], kc, ks, vc, vs)
    assert np.array_equal(c, d)


def test_row_subset_matches_full():
    q, kc, ks, vc, vs = pins.random_case(41, 6, 4, 1, 64, 30)
    pos = [24, 25, 26, 27, 28, 29]
    full = oracle.attention(q, pos, kc, ks, vc, vs)
    sub = oracle.attention(q, pos, kc, ks, vc, vs, rows=[1, 4])
    assert np.array_equal(sub, full[[1, 4]])


def test_dequantize_exact():
    r = np.random.default_rng(42)
    codes = r.integers(-127, 128, size=(2, 3, 64)).astype(np.int8)
    scales = r.uniform(1e-4, 10, size=(2, 3, 2)).astype(np.float16)
    got = oracle.dequantize(codes, scales)
    assert np.array_equal(got, pins.deq(codes, scales))


def test_sm_scale_argument():
    """An explicit sm_scale replaces 1/sqrt(hd) (two-key closed form, scale 0.3)."""
    import math

    hd = 32
    q = np.zeros((1, 1, hd), dtype=np.float32)
    q[0, 0, 0] = 2.0
    kc = np.zeros((1, 2, hd), dtype=np.int8)
    kc[0, 1, 0] = 10
    ks = np.full((1, 2, 1), 0.5, dtype=np.float16)
    vc = np.zeros((1, 2, hd), dtype=np.int8)
    vc[0, 1] = 1
    vs = np.ones((1, 2, 1), dtype=np.float16)
    got = oracle.attention(q, [1], kc, ks, vc, vs, sm_scale=0.3)
    D = 2.0 * 10 * 0.5 * 0.3
    assert abs(got[0, 0, 0] - math.exp(D) / (1 + math.exp(D))) < 1e-15


# ---- the fp16-cache entry of the oracle (values given directly) ----------------


def _attn_values(q, pos, kc, ks, vc, vs, sm_scale=None):
    # the pins hand over int8 blocks; the values core receives them dequantised
    # by the pins' own helper
    return oracle.attention_values(q, pos, pins.deq(kc, ks), pins.deq(vc, vs), sm_scale)


@pytest.mark.parametrize("check", pins.ATTENTION_CHECKS, ids=lambda f: f.__name__)
def test_values_core_pin(check):
    check(_attn_values)


def test_values_core_equals_quantised_path_bitwise():
    q, kc, ks, vc, vs = pins.random_case(61, 5, 8, 2, 64, 90)
    pos = np.array([3, 40, 41, 88, 89])
    a = oracle.attention(q, pos, kc, ks, vc, vs)
    b = oracle.attention_values(q, pos, oracle.dequantize(kc, ks), oracle.dequantize(vc, vs))
    assert np.array_equal(a, b)


def test_f16kv_against_brute_force():
    import bruteforce

    rng = np.random.default_rng(62)
    for hq, hkv, hd, T, n in ((4, 2, 32, 9, 3), (3, 1, 64, 20, 2), (2, 2, 32, 1, 1)):
        k = rng.standard_normal((hkv, T, hd)).astype(np.float16)
        v = (rng.standard_normal((hkv, T, hd)) * 4).astype(np.float16)
        q = rng.standard_normal((n, hq, hd)).astype(np.float32)
        ctx = T - n
        got = oracle.verify_f16kv(q, k, v, ctx)
        ones = np.ones((hkv, T, hd // 32))
        ref = np.array(bruteforce.attention(q, ctx + np.arange(n), k, ones, v, ones))
        assert np.max(np.abs(got - ref)) <= 1e-12 * np.abs(ref).max()
        with pytest.raises(TypeError):
            oracle.verify_f16kv(q, k.astype(np.float32), v, ctx)


def test_golden_files_name_their_source():
    import os

    golden = os.path.join(os.path.dirname(__file__), "golden")
    for name in sorted(os.listdir(golden)):
        if name == "README.md" or name.startswith("."):
            continue
        with open(os.path.join(golden, name)) as f:
            head = f.read(2048)
        assert "source:" in head.lower(), f"tests/golden/{name} does not name its source"


def test_prompt_f16kv_positions_and_brute_force():
    """prompt_f16kv puts query i at q_pos0 + i: literal positions through the
    pure-Python brute force on tiny fp16 caches (G in {1, 2, 3}, a chunk that
    starts at key 0 and one that starts mid-cache)."""
    import bruteforce

    rng = np.random.default_rng(63)
    for hq, hkv, hd, T, n, pos0, literal in ((4, 2, 32, 11, 3, 5, (5, 6, 7)),
                                             (3, 1, 64, 9, 2, 0, (0, 1)),
                                             (2, 2, 32, 6, 4, 2, (2, 3, 4, 5))):
        k = rng.standard_normal((hkv, T, hd)).astype(np.float16)
        v = (rng.standard_normal((hkv, T, hd)) * 3).astype(np.float16)
        q = rng.standard_normal((n, hq, hd)).astype(np.float16)
        got = oracle.prompt_f16kv(q, k, v, q_pos0=pos0)
        ones = np.ones((hkv, T, hd // 32))
        ref = np.array(bruteforce.attention(q, list(literal), k, ones, v, ones))
        assert np.max(np.abs(got - ref)) <= 1e-12 * np.abs(ref).max()
        with pytest.raises(TypeError):
            oracle.prompt_f16kv(q, k, v.astype(np.float32), q_pos0=pos0)


def test_prompt_f16kv_closed_forms():
    """A query at position 0 sees only key 0 (output = V[0] exactly); keys
    after a query's position never change it; a row subset equals the rows of
    the whole chunk."""
    rng = np.random.default_rng(64)
    hkv, hq, hd, T = 1, 2, 64, 12
    k = rng.standard_normal((hkv, T, hd)).astype(np.float16)
    v = rng.standard_normal((hkv, T, hd)).astype(np.float16)
    q = rng.standard_normal((4, hq, hd)).astype(np.float16)
    out = oracle.prompt_f16kv(q, k, v, q_pos0=0)
    for h in range(hq):
        assert np.array_equal(out[0, h], v[0, 0].astype(np.float64))
    k2, v2 = k.copy(), v.copy()
    k2[:, 2:] = rng.standard_normal((hkv, T - 2, hd)).astype(np.float16)
    v2[:, 2:] = rng.standard_normal((hkv, T - 2, hd)).astype(np.float16)
    out2 = oracle.prompt_f16kv(q, k2, v2, q_pos0=0)
    assert np.array_equal(out2[:2], out[:2])      # queries at 0 and 1 see keys 0..1 only
    assert not np.array_equal(out2[2:], out[2:])  # the query at 2 sees key 2
    sub = oracle.prompt_f16kv(q, k, v, q_pos0=0, rows=[1, 3])
    assert np.array_equal(sub, out[[1, 3]])
