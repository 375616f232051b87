"""The input recipe: block-32 quantisation and seeded generation (CPU only)."""

import numpy as np

import workloads as W


def test_max_code_is_127_in_nonzero_blocks():
    x = np.random.default_rng(0).standard_normal((3, 50, 128)).astype(np.float32)
    c, d = W.quantize_blocks(x)
    cb = np.abs(c.astype(np.int32)).reshape(3, 50, 4, 32).max(-1)
    assert np.all(cb[d != 0] == 127)


def test_zero_block():
    x = np.zeros((1, 2, 64), dtype=np.float32)
    x[0, 1, 40] = 1.0
    c, d = W.quantize_blocks(x)
    assert d[0, 0, 0] == 0 and d[0, 0, 1] == 0 and d[0, 1, 0] == 0
    assert np.all(c[0, 0] == 0)
    assert c[0, 1, 40] == 127


def test_ties_round_away_from_zero():
    # amax = 127 -> d = 1 exactly; x/d = k + 0.5 rounds away from zero
    x = np.zeros((1, 1, 32), dtype=np.float32)
    x[0, 0, 0] = 127
    x[0, 0, 1:6] = [2.5, -2.5, 0.5, -0.5, 126.5]
    c, d = W.quantize_blocks(x)
    assert d[0, 0, 0] == 1.0
    assert list(c[0, 0, :6]) == [127, 3, -3, 1, -1, 127]


def test_reconstruction_error_bounded():
    x = np.random.default_rng(1).standard_normal((2, 64, 256)).astype(np.float32)
    c, d = W.quantize_blocks(x)
    rec = c.astype(np.float64).reshape(2, 64, 8, 32) * d.astype(np.float64)[..., None]
    err = np.abs(rec.reshape(x.shape) - x)
    bound = np.repeat(d.astype(np.float64), 32, axis=-1) * (0.5 + 1e-3) + 1e-6
    assert np.all(err <= bound)


def test_generation_is_seeded_and_shaped():
    w = W.TINY_VERIFY
    a = W.generate(w)
    b = W.generate(w)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k_codes, b.k_codes)
    assert a.q.shape == (4, 4, 64) and a.q.dtype == np.float32
    assert a.k_codes.shape == (1, 260, 64) and a.k_codes.dtype == np.int8
    assert a.k_scales.shape == (1, 260, 2) and a.k_scales.dtype == np.float16
    p = W.generate(W.with_changes(W.PROMPT_CHUNK, kv_len=128, n_queries=16))
    assert p.q.dtype == np.float16 and p.q.shape == (16, 12, 256)


def test_stride_padding_is_zero():
    w = W.with_changes(W.TINY_VERIFY, kv_stride=300)
    a = W.generate(w)
    assert a.k_codes.shape[1] == 300
    assert np.all(a.k_codes[:, 260:] == 0) and np.all(a.v_scales[:, 260:] == 0)
    b = W.generate(W.TINY_VERIFY)
    assert np.array_equal(a.k_codes[:, :260], b.k_codes)


def test_peaked_tokens():
    w = W.with_changes(W.LONG_VERIFY, ctx_len=2000)
    a = W.generate(w)
    assert a.peaked_tokens.size == round(0.01 * 2004)
    base = W.generate(W.with_changes(w, peaked_frac=0.0))
    # V is untouched by the peaking; K scales at peaked tokens grow about 8x
    assert np.array_equal(a.v_codes, base.v_codes)
    ratio = a.k_scales[:, a.peaked_tokens].astype(np.float64) / base.k_scales[:, a.peaked_tokens]
    assert np.allclose(ratio, 8.0, rtol=2e-3)


def test_byte_and_flop_counts():
    assert W.VERIFY_WINDOW.visible_kv_bytes() == 45_008_384
    assert W.VERIFY_BATCH.unique_kv_bytes() == 17_895_424
    assert W.VERIFY_BATCH.visible_kv_bytes() == 142_919_680
    assert W.LONG_VERIFY.visible_kv_bytes() == 285_221_376
    assert W.PROMPT_CHUNK.algorithmic_flops() == 798_876_499_968
    assert W.TINY_VERIFY.visible_kv_bytes() == 35_360
