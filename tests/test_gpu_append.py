"""KV append quantiser on the GPU through the C ABI, bit for bit against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import quant_pins as qp
import workloads as W
from attention_int8_quantized_amd import ops
from gpu_util import assert_parity, note

pytestmark = pytest.mark.gpu

SENTINEL_CODE = 93
SENTINEL_SCALE = np.float16(-7.5)


def _cache(H, S, hd):
    codes = np.full((H, S, hd), SENTINEL_CODE, np.int8)
    scales = np.full((H, S, hd // 32), SENTINEL_SCALE, np.float16)
    return codes, scales


def _run(k, v, codes_k, scales_k, codes_v, scales_v, pos0):
    dev = torch.device("cuda")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    kc, ks = t(codes_k), t(scales_k)
    args = dict(v=None, v_codes=None, v_scales=None)
    if v is not None:
        vc, vs = t(codes_v), t(scales_v)
        args = dict(v=t(v), v_codes=vc, v_scales=vs)
    ops.kv_append(t(k), kc, ks, pos0, **args)
    torch.cuda.synchronize()
    out = [kc.cpu().numpy(), ks.cpu().numpy()]
    if v is not None:
        out += [args["v_codes"].cpu().numpy(), args["v_scales"].cpu().numpy()]
    return out


def _same(a, b):
    """Bitwise equality (scales compared as fp16 bit patterns)."""
    if a.dtype == np.float16:
        return np.array_equal(a.view(np.uint16), b.view(np.uint16))
    return np.array_equal(a, b)


CASES = [
    # T, H, hd, stride, pos0, dtype
    (8, 4, 256, 40, 20, np.float32),      # a verify window's rows
    (1, 1, 32, 1, 0, np.float32),
    (3, 3, 96, 7, 4, np.float16),         # a head_dim that is a multiple of 32, not of 64
    (32, 8, 128, 64, 32, np.float32),
    (2048, 1, 256, 2048, 0, np.float16),  # a prompt chunk's rows
    (517, 2, 64, 600, 83, np.float32),    # ragged token count
    (5, 2, 4096, 9, 4, np.float32),       # the largest head_dim
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(str(x) if not isinstance(x, type) else x.__name__ for x in c))
def test_append_matches_oracle(case):
    T, H, hd, S, p0, dt = case
    note(f"kv append {case}")
    rng = np.random.default_rng(T * 7 + hd)
    k = rng.standard_normal((T, H, hd)).astype(dt)
    v = (rng.standard_normal((T, H, hd)) * 3).astype(dt)
    kc0, ks0 = _cache(H, S, hd)
    vc0, vs0 = _cache(H, S, hd)
    got = _run(k, v, kc0, ks0, vc0, vs0, p0)
    note(f"  path: {ops.last_path()}")
    ref = list(oracle.kv_append(k, kc0, ks0, p0)) + list(oracle.kv_append(v, vc0, vs0, p0))
    for g, r, name in zip(got, ref, ("k codes", "k scales", "v codes", "v scales")):
        assert _same(g, r), f"{name} differ in {np.count_nonzero(g != r)} places"


def _pin_rows(dtype=np.float32):
    """Every constructed block of the oracle's pins (ties, near ties, edges), as rows."""
    blocks = np.concatenate([qp.tie_blocks(), qp.near_tie_blocks(), qp.edge_blocks()])
    n = -(-blocks.shape[0] // 8) * 8
    pad = np.zeros((n - blocks.shape[0], 32), np.float32)
    return np.concatenate([blocks, pad]).astype(dtype).reshape(n // 8, 1, 256)


def test_append_pinned_blocks():
    note("kv append on the pinned tie / near-tie / edge blocks")
    k = _pin_rows()
    T = k.shape[0]
    kc0, ks0 = _cache(1, T + 3, 256)
    got = _run(k, None, kc0, ks0, None, None, 3)
    ref = oracle.kv_append(k, kc0, ks0, 3)
    assert _same(got[0], ref[0]) and _same(got[1], ref[1])
    # and the same blocks against the exact rational derivation, straight from the GPU
    blocks = k.reshape(-1, 32)
    gc = got[0][0, 3:3 + T].reshape(-1, 32)
    gs = got[1][0, 3:3 + T].reshape(-1)
    for i in range(0, blocks.shape[0], 7):
        ec, es = qp.exact_block(blocks[i])
        assert [int(c) for c in gc[i]] == ec
        assert qp._scale_value(gs[i]) == es


def test_append_fp16_extremes():
    note("kv append fp16 rows at the ends of the fp16 range")
    rng = np.random.default_rng(5)
    k = (rng.standard_normal((16, 2, 128)) * 2.0 ** rng.integers(-24, 15, (16, 2, 1)))
    k = np.clip(k, -65504, 65504).astype(np.float16)
    kc0, ks0 = _cache(2, 16, 128)
    got = _run(k, None, kc0, ks0, None, None, 0)
    ref = oracle.kv_append(k, kc0, ks0, 0)
    assert _same(got[0], ref[0]) and _same(got[1], ref[1])


def test_append_empty_is_a_no_op():
    dev = torch.device("cuda")
    kc = torch.full((2, 8, 64), SENTINEL_CODE, dtype=torch.int8, device=dev)
    ks = torch.full((2, 8, 2), float(SENTINEL_SCALE), dtype=torch.float16, device=dev)
    ops.kv_append(torch.empty((0, 2, 64), device=dev), kc, ks, 8)
    torch.cuda.synchronize()
    assert (kc == SENTINEL_CODE).all() and (ks == float(SENTINEL_SCALE)).all()


def test_append_then_verify_matches_oracle():
    """The GPU-built cache feeds the verify path: parity with the oracle on the recipe's K/V."""
    w = W.with_changes(W.VERIFY_WINDOW, ctx_len=3000)
    note("kv append then verify (24/4 heads, hd 256, ctx 3000, 8 rows)")
    rng = np.random.default_rng(21)
    T = w.ctx_len + w.n_rows
    k = rng.standard_normal((T, w.n_kv_heads, w.head_dim)).astype(np.float32)
    v = rng.standard_normal((T, w.n_kv_heads, w.head_dim)).astype(np.float32)
    q = rng.standard_normal((w.n_rows, w.n_q_heads, w.head_dim)).astype(np.float32)
    dev = torch.device("cuda")
    kc = torch.zeros((w.n_kv_heads, T, w.head_dim), dtype=torch.int8, device=dev)
    vc = torch.zeros_like(kc)
    ks = torch.zeros((w.n_kv_heads, T, w.head_dim // 32), dtype=torch.float16, device=dev)
    vs = torch.zeros_like(ks)
    # the context in two appends, then the rows' own keys, as a decode loop would
    kt, vt = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)
    ops.kv_append(kt[:1000].contiguous(), kc, ks, 0, vt[:1000].contiguous(), vc, vs)
    ops.kv_append(kt[1000:w.ctx_len].contiguous(), kc, ks, 1000, vt[1000:w.ctx_len].contiguous(), vc, vs)
    ops.kv_append(kt[w.ctx_len:].contiguous(), kc, ks, w.ctx_len, vt[w.ctx_len:].contiguous(), vc, vs)
    got = ops.verify(torch.from_numpy(q).to(dev), kc, ks, vc, vs, ctx_len=w.ctx_len).cpu().numpy()
    rkc, rks = oracle.quantize_q8(np.transpose(k, (1, 0, 2)))
    rvc, rvs = oracle.quantize_q8(np.transpose(v, (1, 0, 2)))
    assert _same(kc.cpu().numpy(), rkc) and _same(ks.cpu().numpy(), rks)
    assert _same(vc.cpu().numpy(), rvc) and _same(vs.cpu().numpy(), rvs)
    ref = oracle.verify(q, rkc, rks, rvc, rvs, w.ctx_len)
    assert_parity(got, ref, "append + verify")


def test_append_full_size_long_context():
    """The long-verify cache (131,076 tokens x 4 KV heads x 256) built by one call per tensor."""
    w = W.LONG_VERIFY
    T = w.kv_tokens
    note(f"kv append full size: {T} tokens x {w.n_kv_heads} heads x {w.head_dim}")
    rng = np.random.default_rng(22)
    k = rng.standard_normal((T, w.n_kv_heads, w.head_dim), dtype=np.float32)
    dev = torch.device("cuda")
    kc = torch.empty((w.n_kv_heads, T, w.head_dim), dtype=torch.int8, device=dev)
    ks = torch.empty((w.n_kv_heads, T, w.head_dim // 32), dtype=torch.float16, device=dev)
    ops.kv_append(torch.from_numpy(k).to(dev), kc, ks, 0)
    torch.cuda.synchronize()
    note(f"  path: {ops.last_path()}")
    rc, rs = oracle.quantize_q8(np.transpose(k, (1, 0, 2)))
    assert _same(kc.cpu().numpy(), rc) and _same(ks.cpu().numpy(), rs)


def test_bad_append_arguments_on_gpu():
    dev = torch.device("cuda")
    k = torch.zeros((4, 2, 64), device=dev)
    kc = torch.zeros((2, 8, 64), dtype=torch.int8, device=dev)
    ks = torch.zeros((2, 8, 2), dtype=torch.float16, device=dev)
    with pytest.raises(Exception):
        ops.kv_append(k, kc, ks, 5)  # rows 5..8 run past the cache
    with pytest.raises(Exception):
        ops.kv_append(k, kc, ks, 0, v=k)  # V rows without a V cache
