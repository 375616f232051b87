"""Verify and prompt attention over an fp16 K/V cache on the GPU, against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from attention_int8_quantized_amd import ops
from gpu_util import assert_parity, note

pytestmark = pytest.mark.gpu


def _dev(inp):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    return t(inp.q), t(inp.k), t(inp.v)


@pytest.mark.parametrize("name,rg", [("tiny_verify", 0), ("verify_window", 0), ("verify_window", 1),
                                     ("verify_batch", 4), ("verify_batch", 0), ("verify_batch", 32),
                                     ("long_verify", 0)])
def test_verify_f16kv_workloads(name, rg):
    w = W.WORKLOADS[name]
    note(f"verify fp16 cache {name} rows_per_group={rg}")
    inp = W.generate_f16kv(w)
    q, k, v = _dev(inp)
    got = ops.verify_f16kv(q, k, v, ctx_len=w.ctx_len, rows_per_group=rg).cpu().numpy()
    note(f"  path: {ops.last_path()}")
    ref = oracle.verify_f16kv(inp.q, inp.k, inp.v, w.ctx_len)
    assert_parity(got, ref, f"workload {name} over an fp16 cache (full size, rows_per_group {rg})")


SMALL = [
    # hq, hkv, hd, ctx, rows, rows_per_group, splits, qdtype, stride_pad
    (4, 1, 64, 0, 1, 0, 0, np.float32, 0),
    (8, 8, 64, 31, 5, 2, 1, np.float32, 3),
    (6, 2, 128, 33, 7, 3, 2, np.float16, 0),
    (12, 1, 256, 100, 8, 0, 0, np.float32, 17),
    (32, 8, 128, 500, 32, 1, 5, np.float32, 0),
    (16, 2, 64, 1000, 9, 0, 0, np.float16, 0),
    (64, 1, 128, 70, 2, 0, 0, np.float32, 0),   # automatic: one row (64 vectors) per group
    (64, 1, 128, 70, 2, 2, 0, np.float32, 0),   # 128 vectors in one group: the own layout
    (24, 4, 256, 2000, 8, 0, 63, np.float32, 0),
    (48, 1, 256, 300, 2, 2, 0, np.float16, 5),  # 96 vectors: the largest group at hd 256
    (24, 2, 256, 400, 8, 8, 0, np.float32, 0),   # 96 vectors per group: the own layout
    (24, 2, 256, 333, 13, 8, 3, np.float16, 2),  # own layout; groups of 8 and 5 rows
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(str(x) if not isinstance(x, type) else x.__name__ for x in c))
def test_verify_f16kv_small(case):
    hq, hkv, hd, ctx, rows, rg, splits, qd, pad = case
    w = W.VerifyWorkload("small16", hq, hkv, hd, ctx, rows, rg or rows, seed=ctx + rows + 1,
                         kv_stride=ctx + rows + pad)
    note(f"verify fp16 cache small {case}")
    inp = W.generate_f16kv(w)
    inp.q = inp.q.astype(qd)
    q, k, v = _dev(inp)
    ws, S = ops.verify_f16kv_partials(q, k, v, ctx_len=ctx, rows_per_group=rg, n_splits=splits)
    path = ops.last_path()  # the attention kernel's (the reducer records its own)
    got = ops.reduce_partials(ws, rows, hq, hd, S).cpu().numpy()
    note(f"  path: {path}")
    assert path.startswith("verify kvf16")
    assert ("own" in path) == ((hd == 256 and ("tiles6" in path or "tiles3" in path)) or (hd == 128 and "tiles8" in path))
    ref = oracle.verify_f16kv(inp.q, inp.k, inp.v, ctx)
    assert_parity(got, ref, f"small {case}")


def test_prompt_f16kv_chunk():
    w = W.PROMPT_CHUNK
    note("prompt fp16 cache: 12/1 heads, hd 256, 32K x 2,048 (all rows)")
    inp = W.generate_f16kv(w)
    q, k, v = _dev(inp)
    got = ops.prompt_f16kv(q, k, v, q_pos0=w.pos0, kv_len=w.kv_len).cpu().numpy()
    note(f"  path: {ops.last_path()}")
    ref = oracle.prompt_f16kv(inp.q, inp.k, inp.v, w.pos0)
    assert_parity(got, ref, "prompt_chunk over an fp16 cache (whole chunk)")


@pytest.mark.parametrize("hq,hkv,hd,kv_len,n,qd", [
    (12, 1, 256, 700, 64, np.float16), (8, 2, 128, 300, 33, np.float32),
    (4, 4, 64, 129, 129, np.float16), (12, 1, 256, 96, 5, np.float32)])
def test_prompt_f16kv_small(hq, hkv, hd, kv_len, n, qd):
    w = W.PromptWorkload("p16", hq, hkv, hd, kv_len, n, seed=kv_len + n)
    note(f"prompt fp16 cache {hq}/{hkv} hd{hd} kv{kv_len} n{n} {qd.__name__}")
    inp = W.generate_f16kv(w)
    inp.q = inp.q.astype(qd)
    q, k, v = _dev(inp)
    got = ops.prompt_f16kv(q, k, v, q_pos0=w.pos0, kv_len=w.kv_len).cpu().numpy()
    note(f"  path: {ops.last_path()}")
    ref = oracle.prompt_f16kv(inp.q, inp.k, inp.v, w.pos0)
    assert_parity(got, ref, "prompt small")


def test_f16kv_group_limit_at_256():
    w = W.VerifyWorkload("lim", 64, 1, 256, 100, 2, 2)
    inp = W.generate_f16kv(w)
    q, k, v = _dev(inp)
    with pytest.raises(Exception):
        ops.verify_f16kv(q, k, v, ctx_len=100, rows_per_group=2)  # 128 vectors > 96


@pytest.mark.parametrize("hq,hkv,hd,kv_len,n,pos0,qd", [
    (96, 8, 256, 400, 229, None, np.float16),   # 8 rows x 12 heads; last group 5 rows
    (11, 1, 256, 1900, 1800, None, np.float32),  # 8 rows x 11 heads = 88 vectors
    (32, 2, 256, 800, 700, 3, np.float16),       # 6 rows x 16 heads; context past the chunk
    (32, 2, 128, 900, 800, None, np.float16),    # head_dim 128: 7 rows x 16 heads = 112 vectors
    (64, 1, 128, 700, 600, 0, np.float32),       # 2 rows x 64 heads = 128 vectors
])
def test_prompt_f16kv_own_layout(hq, hkv, hd, kv_len, n, pos0, qd):
    """Row groups of six vector tiles at head_dim 256, five to eight at 128, take the own layout."""
    w = W.PromptWorkload("p16own", hq, hkv, hd, kv_len, n, seed=kv_len + 3 * n, q_pos0=pos0)
    note(f"prompt fp16 cache own layout {hq}/{hkv} hd{hd} kv{kv_len} n{n} {qd.__name__}")
    inp = W.generate_f16kv(w)
    inp.q = inp.q.astype(qd)
    q, k, v = _dev(inp)
    got = ops.prompt_f16kv(q, k, v, q_pos0=w.pos0, kv_len=w.kv_len).cpu().numpy()
    path = ops.last_path()
    note(f"  path: {path}")
    assert ("tiles6 own" if hd == 256 else "tiles8 own") in path
    rows = sorted(set(list(range(0, 18)) + list(range(n - 18, n)) +
                      list(np.random.default_rng(n).integers(0, n, 24))))
    ref = oracle.prompt_f16kv(inp.q, inp.k, inp.v, w.pos0, rows=rows)
    assert_parity(got[rows], ref, "prompt fp16 cache own layout")
