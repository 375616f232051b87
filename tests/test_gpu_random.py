"""Seeded random shapes through the C ABI against the oracle.

Each case draws a head_dim, head counts, row or query counts, a context with a
ragged tail, a cache stride with padding, q in fp32 or fp16 and (verify) a row
grouping and split count within the documented limits, so the sweep covers
combinations the hand-picked cases do not.  Sizes stay small enough for the
fp64 oracle (a fraction of a second per case).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from attention_int8_quantized_amd import ops
from gpu_util import assert_parity, note, to_device

pytestmark = pytest.mark.gpu

HDS = (64, 128, 256)
GROUPS = (1, 2, 3, 4, 6, 8, 12, 16)


def _verify_case(i, kv16):
    r = np.random.default_rng(1000 + i + (500 if kv16 else 0))
    hd = int(r.choice(HDS))
    G = int(r.choice(GROUPS))
    hkv = int(r.choice((1, 2, 4)))
    rows = int(r.integers(1, 33))
    while rows * G * hkv > 256 and rows > 1:
        rows //= 2
    ctx = int(r.integers(0, 1200))
    limit = 96 if (kv16 and hd == 256) else 128
    rg = 0
    if r.random() < 0.5:
        rg = int(r.integers(1, rows + 1))
        while rg * G > limit and rg > 1:
            rg -= 1
        if rg * G > limit:
            rg = 0
    if rg == 0 and G > (64 if hd == 256 else 128):
        G = 8
    tiles = (ctx + rows + 31) // 32
    splits = int(r.integers(1, tiles + 1)) if r.random() < 0.4 else 0
    qd = np.float32 if r.random() < 0.7 else np.float16
    pad = int(r.integers(0, 40)) if r.random() < 0.5 else 0
    peaked = 0.02 if r.random() < 0.2 else 0.0
    return dict(hd=hd, hq=G * hkv, hkv=hkv, rows=rows, ctx=ctx, rg=rg, splits=splits, qd=qd, pad=pad,
                peaked=peaked, seed=int(r.integers(0, 1 << 30)))


def _prompt_case(i, kv16):
    r = np.random.default_rng(3000 + i + (500 if kv16 else 0))
    hd = int(r.choice(HDS))
    G = int(r.choice(GROUPS))
    hkv = int(r.choice((1, 2)))
    kv_len = int(r.integers(1, 1200))
    n = int(r.integers(1, min(kv_len, 160) + 1))
    pos0 = int(r.integers(0, kv_len - n + 1)) if r.random() < 0.5 else kv_len - n
    qd = np.float16 if r.random() < 0.7 else np.float32
    pad = int(r.integers(0, 40)) if r.random() < 0.5 else 0
    return dict(hd=hd, hq=G * hkv, hkv=hkv, kv_len=kv_len, n=n, pos0=pos0, qd=qd, pad=pad,
                seed=int(r.integers(0, 1 << 30)))


def _own128_case(i, kv16):
    # head_dim 128 row groups of 65..128 vectors: the own layout's eight compute waves
    r = np.random.default_rng(5000 + i + (500 if kv16 else 0))
    G = int(r.choice((4, 8, 16, 32, 64)))
    hkv = int(r.choice((1, 2)))
    rg = int(r.integers(65 // G + (65 % G > 0), 128 // G + 1))
    rows = int(r.integers(rg, min(32, 3 * rg) + 1))
    ctx = int(r.integers(0, 900))
    tiles = (ctx + rows + 31) // 32
    splits = int(r.integers(1, tiles + 1)) if r.random() < 0.5 else 0
    qd = np.float32 if r.random() < 0.6 else np.float16
    pad = int(r.integers(0, 40)) if r.random() < 0.5 else 0
    peaked = 0.02 if r.random() < 0.3 else 0.0
    return dict(hd=128, hq=G * hkv, hkv=hkv, rows=rows, ctx=ctx, rg=rg, splits=splits, qd=qd, pad=pad,
                peaked=peaked, seed=int(r.integers(0, 1 << 30)))


def _desc(c):
    return " ".join(f"{k}={v.__name__ if isinstance(v, type) else v}" for k, v in c.items())


@pytest.mark.parametrize("i", range(30))
def test_random_verify(i):
    c = _verify_case(i, False)
    note(f"random verify {i}: {_desc(c)}")
    w = W.VerifyWorkload("rand", c["hq"], c["hkv"], c["hd"], c["ctx"], c["rows"], c["rg"] or c["rows"],
                         peaked_frac=c["peaked"], seed=c["seed"], kv_stride=c["ctx"] + c["rows"] + c["pad"])
    inp = W.generate(w)
    inp.q = inp.q.astype(c["qd"])
    out = ops.verify(*to_device(inp), ctx_len=c["ctx"], rows_per_group=c["rg"], n_splits=c["splits"])
    torch.cuda.synchronize()
    note(f"  path: {ops.last_path()}")
    ref = oracle.verify(inp.q, inp.k_codes, inp.k_scales, inp.v_codes, inp.v_scales, c["ctx"])
    assert_parity(out.cpu().numpy(), ref, f"random verify {i}")


@pytest.mark.parametrize("i", range(20))
def test_random_prompt(i):
    c = _prompt_case(i, False)
    note(f"random prompt {i}: {_desc(c)}")
    w = W.PromptWorkload("rand", c["hq"], c["hkv"], c["hd"], c["kv_len"], c["n"], seed=c["seed"],
                         q_pos0=c["pos0"], kv_stride=c["kv_len"] + c["pad"])
    inp = W.generate(w)
    inp.q = inp.q.astype(c["qd"])
    out = ops.prompt(*to_device(inp), q_pos0=c["pos0"], kv_len=c["kv_len"])
    torch.cuda.synchronize()
    note(f"  path: {ops.last_path()}")
    ref = oracle.prompt(inp.q, inp.k_codes, inp.k_scales, inp.v_codes, inp.v_scales, c["pos0"])
    assert_parity(out.cpu().numpy(), ref, f"random prompt {i}")


def _dev16(inp):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    return t(inp.q), t(inp.k), t(inp.v)


@pytest.mark.parametrize("i", range(15))
def test_random_verify_f16kv(i):
    c = _verify_case(i, True)
    note(f"random verify fp16 cache {i}: {_desc(c)}")
    w = W.VerifyWorkload("rand16", c["hq"], c["hkv"], c["hd"], c["ctx"], c["rows"], c["rg"] or c["rows"],
                         peaked_frac=c["peaked"], seed=c["seed"], kv_stride=c["ctx"] + c["rows"] + c["pad"])
    inp = W.generate_f16kv(w)
    inp.q = inp.q.astype(c["qd"])
    out = ops.verify_f16kv(*_dev16(inp), ctx_len=c["ctx"], rows_per_group=c["rg"], n_splits=c["splits"])
    torch.cuda.synchronize()
    note(f"  path: {ops.last_path()}")
    ref = oracle.verify_f16kv(inp.q, inp.k, inp.v, c["ctx"])
    assert_parity(out.cpu().numpy(), ref, f"random verify fp16 cache {i}")


@pytest.mark.parametrize("i", range(10))
def test_random_prompt_f16kv(i):
    c = _prompt_case(i, True)
    note(f"random prompt fp16 cache {i}: {_desc(c)}")
    w = W.PromptWorkload("rand16", c["hq"], c["hkv"], c["hd"], c["kv_len"], c["n"], seed=c["seed"],
                         q_pos0=c["pos0"], kv_stride=c["kv_len"] + c["pad"])
    inp = W.generate_f16kv(w)
    inp.q = inp.q.astype(c["qd"])
    out = ops.prompt_f16kv(*_dev16(inp), q_pos0=c["pos0"], kv_len=c["kv_len"])
    torch.cuda.synchronize()
    note(f"  path: {ops.last_path()}")
    ref = oracle.prompt_f16kv(inp.q, inp.k, inp.v, c["pos0"])
    assert_parity(out.cpu().numpy(), ref, f"random prompt fp16 cache {i}")


@pytest.mark.parametrize("kv16", [False, True], ids=["int8", "fp16"])
@pytest.mark.parametrize("i", range(6))
def test_random_verify_own128(i, kv16):
    c = _own128_case(i, kv16)
    note(f"random verify own layout hd128 {i} {'fp16' if kv16 else 'int8'} cache: {_desc(c)}")
    w = W.VerifyWorkload("rand128", c["hq"], c["hkv"], c["hd"], c["ctx"], c["rows"], c["rg"],
                         peaked_frac=c["peaked"], seed=c["seed"], kv_stride=c["ctx"] + c["rows"] + c["pad"])
    if kv16:
        inp = W.generate_f16kv(w)
        inp.q = inp.q.astype(c["qd"])
        ws, S = ops.verify_f16kv_partials(*_dev16(inp), ctx_len=c["ctx"], rows_per_group=c["rg"],
                                          n_splits=c["splits"])
        ref = oracle.verify_f16kv(inp.q, inp.k, inp.v, c["ctx"])
    else:
        inp = W.generate(w)
        inp.q = inp.q.astype(c["qd"])
        ws, S = ops.verify_partials(*to_device(inp), ctx_len=c["ctx"], rows_per_group=c["rg"],
                                    n_splits=c["splits"])
        ref = oracle.verify(inp.q, inp.k_codes, inp.k_scales, inp.v_codes, inp.v_scales, c["ctx"])
    path = ops.last_path()  # the attention kernel's (the reducer records its own)
    out = ops.reduce_partials(ws, c["rows"], c["hq"], c["hd"], S)
    torch.cuda.synchronize()
    note(f"  path: {path}")
    assert "tiles8 own" in path
    assert_parity(out.cpu().numpy(), ref, f"random verify own layout hd128 {i}")
