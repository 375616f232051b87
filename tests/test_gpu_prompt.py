"""Prompt (chunked causal prefill) attention on the GPU against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from attention_int8_quantized_amd import ops
from gpu_util import assert_parity, note, to_device

pytestmark = pytest.mark.gpu


def run_prompt(w, inp=None):
    inp = inp or W.generate(w)
    dev = to_device(inp)
    out = ops.prompt(*dev, q_pos0=w.pos0, kv_len=w.kv_len)
    torch.cuda.synchronize()
    return inp, out.cpu().numpy(), ops.last_path()


def test_prompt_chunk_whole():
    """The full 32K x 2048-query chunk, every row against the oracle (the accuracy
    figure of "hip: gfx12 (RDNA4) WMMA kernel for the int8-KV QSA prompt
    attention", Measurements, covers the whole chunk)."""
    w = W.PROMPT_CHUNK
    note("prompt chunk 12/1 hd256 kv 32768 x 2048 queries (all rows)")
    inp, got, path = run_prompt(w)
    note(f"  path: {path}")
    ref = oracle.prompt(inp.q, inp.k_codes, inp.k_scales, inp.v_codes, inp.v_scales, w.pos0)
    assert_parity(got, ref, "prompt_chunk (whole chunk)")


SMALL = [
    # hq, hkv, hd, kv_len, n_queries, q_pos0 (None = at the end), stride_pad, q dtype
    (12, 1, 256, 300, 64, None, 0, np.float16),
    (12, 1, 256, 64, 64, 0, 0, np.float16),        # query 0 sees only key 0
    (4, 1, 64, 1, 1, 0, 0, np.float16),
    (4, 2, 64, 37, 17, 5, 3, np.float16),
    (8, 8, 128, 200, 33, None, 0, np.float32),
    (1, 1, 128, 500, 100, 400, 0, np.float16),
    (6, 2, 256, 129, 40, 80, 0, np.float32),
    (16, 1, 64, 2000, 96, None, 0, np.float16),
    (128, 1, 256, 300, 20, None, 0, np.float16),   # 128 vectors per query at head_dim 256
    (128, 2, 64, 150, 9, 3, 0, np.float32),        # 128 vectors per query at head_dim 64
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(str(x) if not isinstance(x, type) else x.__name__ for x in c))
def test_small_shapes(case):
    hq, hkv, hd, kv_len, n, pos0, pad, qd = case
    w = W.PromptWorkload("small", hq, hkv, hd, kv_len, n, seed=kv_len + n, q_pos0=pos0,
                         kv_stride=kv_len + pad)
    note(f"prompt small {case}")
    inp = W.generate(w)
    inp.q = inp.q.astype(qd)
    _, got, path = run_prompt(w, inp)
    note(f"  path: {path}")
    ref = oracle.prompt(inp.q, inp.k_codes, inp.k_scales, inp.v_codes, inp.v_scales, w.pos0)
    assert_parity(got, ref, f"prompt small {case}")


def test_prompt_deterministic_and_causal():
    w = W.PromptWorkload("det", 12, 1, 256, 1000, 128, seed=11)
    note("prompt determinism + causal perturbation")
    inp = W.generate(w)
    dev = list(to_device(inp))
    a = ops.prompt(*dev, q_pos0=w.pos0, kv_len=w.kv_len).cpu().numpy()
    b = ops.prompt(*dev, q_pos0=w.pos0, kv_len=w.kv_len).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    cut = w.pos0 + 50  # queries 0..49 see keys < cut
    dev[1][:, cut:] = -dev[1][:, cut:]
    dev[3][:, cut:] = 100
    c = ops.prompt(*dev, q_pos0=w.pos0, kv_len=w.kv_len).cpu().numpy()
    assert np.array_equal(a[:50].view(np.uint32), c[:50].view(np.uint32))
    assert not np.array_equal(a[50:], c[50:])


def test_prompt_first_query_is_value():
    w = W.PromptWorkload("first", 4, 1, 128, 40, 40, seed=12, q_pos0=0)
    inp, got, _ = run_prompt(w)
    vhat = oracle.dequantize(inp.v_codes[0, 0], inp.v_scales[0, 0])
    for h in range(4):
        assert np.max(np.abs(got[0, h] - vhat)) <= 2.0 ** -21 * np.abs(vhat).max()


OWN = [
    # hq, hkv, hd, kv_len, n_queries, q_pos0 (None = at the end), stride_pad, q dtype: row groups
    # of 81..96 vectors at head_dim 256 (one compute wave per 16 vectors), ragged last groups
    (96, 8, 256, 400, 229, None, 0, np.float16),    # 8 rows x 12 heads; last group 5 rows
    (96, 8, 256, 300, 227, 0, 5, np.float32),       # fp32 q, query 0 at position 0, padded stride
    (32, 2, 256, 800, 700, None, 0, np.float16),    # 6 rows x 16 heads; last group 4 rows
    (11, 1, 256, 1900, 1800, None, 0, np.float32),  # 8 rows x 11 heads = 88 vectors
    (12, 1, 256, 1900, 1795, 17, 0, np.float16),    # last group 3 rows; context past the chunk
    # head_dim 128: eight compute waves for row groups of 65..128 vectors
    (32, 2, 128, 900, 800, None, 0, np.float16),    # 7 rows x 16 heads = 112 vectors
    (64, 1, 128, 700, 600, 0, 3, np.float32),       # 2 rows x 64 heads = 128 vectors, fp32 q
    (16, 1, 128, 1500, 1400, 31, 0, np.float16),    # 6 rows x 16 heads; context past the chunk
]


@pytest.mark.parametrize("case", OWN, ids=lambda c: "-".join(str(x) if not isinstance(x, type) else x.__name__ for x in c))
def test_own_layout_shapes(case):
    hq, hkv, hd, kv_len, n, pos0, pad, qd = case
    w = W.PromptWorkload("own", hq, hkv, hd, kv_len, n, seed=kv_len + 7 * n, q_pos0=pos0,
                         kv_stride=kv_len + pad)
    note(f"prompt own layout {case}")
    inp = W.generate(w)
    inp.q = inp.q.astype(qd)
    _, got, path = run_prompt(w, inp)
    note(f"  path: {path}")
    assert ("tiles6 own" if hd == 256 else "tiles8 own") in path
    # the first and last rows of every row group near the ends, a spread in between
    rows = sorted(set(list(range(0, 18)) + list(range(n - 18, n)) +
                      list(np.random.default_rng(n).integers(0, n, 24))))
    ref = oracle.prompt(inp.q, inp.k_codes, inp.k_scales, inp.v_codes, inp.v_scales, w.pos0,
                        rows=rows)
    assert_parity(got[rows], ref, f"prompt own layout {case}")
