"""Verify attention on the GPU through the C ABI, element by element against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from attention_int8_quantized_amd import ops
from gpu_util import assert_parity, note, to_device

pytestmark = pytest.mark.gpu


def run_verify(w, rows_per_group=0, n_splits=0, q_dtype=None, inp=None):
    inp = inp or W.generate(w)
    if q_dtype is not None:
        inp.q = inp.q.astype(q_dtype)
    dev = to_device(inp)
    # the attention launch and the reducer separately, so that the returned path
    # is the attention kernel's (the library records the last launch)
    ws, S = ops.verify_partials(*dev, ctx_len=w.ctx_len, rows_per_group=rows_per_group,
                                n_splits=n_splits)
    path = ops.last_path()
    out = ops.reduce_partials(ws, inp.q.shape[0], inp.q.shape[1], inp.q.shape[2], S)
    torch.cuda.synchronize()
    return inp, out.cpu().numpy(), path


def oracle_verify(inp, w):
    return oracle.verify(inp.q, inp.k_codes, inp.k_scales, inp.v_codes, inp.v_scales, w.ctx_len)


def test_i8_to_f16_all_byte_pairs():
    note("selftest_i8_to_f16 over 65,536 byte pairs")
    got = ops.selftest_i8_to_f16().cpu().numpy().view(np.float16).reshape(65536, 2)
    p = np.arange(65536, dtype=np.int64)
    lo = (p & 255).astype(np.uint8).view(np.int8).astype(np.float16)
    hi = (p >> 8).astype(np.uint8).view(np.int8).astype(np.float16)
    assert np.array_equal(got[:, 0].view(np.uint16), lo.view(np.uint16))
    assert np.array_equal(got[:, 1].view(np.uint16), hi.view(np.uint16))


@pytest.mark.parametrize("name,rg", [
    ("tiny_verify", 0),
    ("verify_window", 0),
    ("verify_window", 1),
    ("verify_batch", 4),
    ("verify_batch", 1),
    ("verify_batch", 0),
    ("verify_batch", 32),
    ("long_verify", 0),
])
def test_workload_parity(name, rg):
    w = W.WORKLOADS[name]
    note(f"verify parity {name} rows_per_group={rg}")
    inp, got, path = run_verify(w, rows_per_group=rg)
    note(f"  path: {path}")
    ref = oracle_verify(inp, w)
    assert_parity(got, ref, f"workload {name} (full size, rows_per_group {rg})")


SMALL = [
    # hq, hkv, hd, ctx, rows, rows_per_group, splits, qdtype, stride_pad
    (4, 1, 64, 0, 1, 0, 0, np.float32, 0),
    (4, 1, 64, 1, 4, 0, 0, np.float32, 0),
    (8, 8, 64, 31, 5, 2, 1, np.float32, 3),
    (6, 2, 128, 33, 7, 3, 2, np.float16, 0),
    (12, 1, 256, 100, 8, 0, 0, np.float32, 17),
    (32, 8, 128, 500, 32, 0, 0, np.float32, 0),   # automatic: two groups of 16 rows (64 vectors)
    (32, 8, 128, 500, 32, 32, 0, np.float32, 0),  # one group of 128 vectors: the own layout
    (32, 8, 128, 500, 32, 20, 3, np.float16, 3),  # own layout; groups of 20 and 12 rows (80, 48 vectors)
    (32, 8, 128, 500, 32, 1, 5, np.float32, 0),
    (16, 2, 64, 1000, 9, 0, 0, np.float16, 0),
    (3, 1, 256, 64, 3, 0, 3, np.float32, 0),
    (64, 1, 128, 70, 2, 0, 0, np.float32, 0),   # automatic: one row (64 vectors) per group
    (64, 1, 128, 70, 2, 2, 0, np.float32, 0),   # 128 query vectors in one group: the own layout
    (128, 1, 64, 45, 1, 0, 0, np.float32, 1),   # 8 waves, one row
    (24, 4, 256, 2000, 8, 0, 63, np.float32, 0),  # every split 1 tile
    (24, 4, 256, 777, 32, 0, 0, np.float32, 5),   # 32 rows: groups of 10, 10, 10, 2
    (24, 4, 256, 777, 32, 0, 0, np.float16, 0),
    (24, 2, 256, 900, 8, 8, 0, np.float32, 0),    # 96 vectors per group: the own layout
    (24, 2, 256, 333, 13, 8, 3, np.float16, 2),   # own layout; groups of 8 and 5 rows
    (128, 1, 256, 100, 1, 0, 0, np.float32, 0),   # 128 vectors at head_dim 256: the eight-tile body
    (128, 2, 256, 150, 2, 1, 2, np.float16, 1),   # the same, two KV heads, two groups of one row
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(str(x) if not isinstance(x, type) else x.__name__ for x in c))
def test_small_shapes(case):
    hq, hkv, hd, ctx, rows, rg, splits, qd, pad = case
    w = W.VerifyWorkload("small", hq, hkv, hd, ctx, rows, rg or rows, seed=ctx + rows,
                         kv_stride=ctx + rows + pad)
    note(f"verify small {case}")
    inp = W.generate(w)
    inp.q = inp.q.astype(qd)
    _, got, path = run_verify(w, rows_per_group=rg, n_splits=splits, inp=inp)
    note(f"  path: {path}")
    assert path.startswith("verify kvq8")
    assert ("own" in path) == ((hd == 256 and "tiles6" in path) or (hd == 128 and "tiles8" in path))
    ref = oracle_verify(inp, w)
    assert_parity(got, ref, f"small {case}")


def test_deterministic_repeat():
    w = W.VERIFY_WINDOW
    note("verify determinism (two calls, bitwise)")
    inp = W.generate(w)
    dev = to_device(inp)
    a = ops.verify(*dev, ctx_len=w.ctx_len).cpu().numpy()
    b = ops.verify(*dev, ctx_len=w.ctx_len).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_split_and_grouping_invariance():
    w = W.with_changes(W.VERIFY_BATCH, ctx_len=3000)
    note("verify split / grouping invariance")
    inp = W.generate(w)
    dev = to_device(inp)
    base = ops.verify(*dev, ctx_len=w.ctx_len, rows_per_group=32, n_splits=1).cpu().numpy()
    scale = np.abs(base).max()
    for rg, s in ((4, 0), (32, 0), (8, 7), (1, 94), (16, 3)):
        got = ops.verify(*dev, ctx_len=w.ctx_len, rows_per_group=rg, n_splits=s).cpu().numpy()
        e = np.abs(got - base).max() / scale
        note(f"  rows_per_group={rg} splits={s}: {e:.2e}")
        # Only the fp32 summation order changes: a sum over n ~ 3000 keys carries
        # about sqrt(n) * 2^-24 ~ 3e-6 relative rounding, so two orders agree to
        # a few 1e-6 of the output scale (well inside the 1e-5 oracle bound).
        assert e <= 5e-6


def test_causal_perturbation_leaves_earlier_rows():
    w = W.with_changes(W.VERIFY_WINDOW, ctx_len=4000)
    note("verify causal perturbation")
    inp = W.generate(w)
    dev = list(to_device(inp))
    a = ops.verify(*dev, ctx_len=w.ctx_len, n_splits=16).cpu().numpy()
    # change every key/value after row 3's position
    cut = w.ctx_len + 4
    dev[1][:, cut:] = -dev[1][:, cut:]
    dev[3][:, cut:] = 77
    dev[4][:, cut:] = 2.0
    b = ops.verify(*dev, ctx_len=w.ctx_len, n_splits=16).cpu().numpy()
    assert np.array_equal(a[:4].view(np.uint32), b[:4].view(np.uint32))
    assert not np.array_equal(a[4:], b[4:])


def test_single_visible_key():
    """ctx 0, row 0 sees key 0 only: the output is Vhat[0] (to the hi+lo rounding)."""
    w = W.VerifyWorkload("one_key", 8, 2, 256, 0, 3, 3, seed=5)
    inp = W.generate(w)
    _, got, _ = run_verify(w, inp=inp)
    vhat = oracle.dequantize(inp.v_codes[:, 0], inp.v_scales[:, 0])  # [hkv][hd]
    for h in range(8):
        ref = vhat[h // 4]
        assert np.max(np.abs(got[0, h] - ref)) <= 2.0 ** -21 * np.abs(ref).max()


def test_constant_keys_give_mean():
    w = W.VerifyWorkload("const_k", 8, 2, 128, 700, 4, 4, seed=6)
    inp = W.generate(w)
    inp.k_codes[:] = 11
    inp.k_scales[:] = np.float16(0.02)
    _, got, _ = run_verify(w, inp=inp)
    vhat = oracle.dequantize(inp.v_codes, inp.v_scales)
    for r in range(4):
        for h in range(8):
            mean = vhat[h // 4, : w.ctx_len + r + 1].mean(axis=0)
            assert np.max(np.abs(got[r, h] - mean)) <= 1e-6 * np.abs(mean).max() + 1e-9


def test_reducer_closed_forms():
    note("reducer on hand-built partials")
    S, R, H, D = 3, 2, 4, 64
    rng = np.random.default_rng(9)
    o = rng.standard_normal((S, R, H, D)).astype(np.float32)
    l = rng.uniform(1, 3, size=(S, R, H)).astype(np.float32)
    m = rng.uniform(-5, 5, size=(S, R, H)).astype(np.float32)
    # one empty split per (row 1, head 2)
    o[1, 1, 2] = 0
    l[1, 1, 2] = 0
    m[1, 1, 2] = -np.inf
    ws = np.concatenate([o.ravel(), np.stack([m, l], -1).ravel()]).astype(np.float32)
    wst = torch.from_numpy(ws.view(np.uint8).copy()).cuda()
    got = ops.reduce_partials(wst, R, H, D, S).cpu().numpy()
    ref = oracle.merge_partials(m.astype(np.float64), l.astype(np.float64), o.astype(np.float64))
    assert np.max(np.abs(got - ref)) <= 1e-6 * np.abs(ref).max()
    # a single split gives o / l
    ws1 = np.concatenate([o[:1].ravel(), np.stack([m[:1], l[:1]], -1).ravel()]).astype(np.float32)
    got1 = ops.reduce_partials(torch.from_numpy(ws1.view(np.uint8).copy()).cuda(), R, H, D, 1)
    assert np.allclose(got1.cpu().numpy(), o[0] / l[0][..., None], rtol=1e-6, atol=0)


def test_partials_match_oracle_split():
    """The workspace partials themselves: o/l per split matches the oracle split."""
    w = W.VerifyWorkload("parts", 8, 2, 128, 300, 4, 4, seed=7)
    inp = W.generate(w)
    dev = to_device(inp)
    S = 4
    ws, _ = ops.verify_partials(*dev, ctx_len=w.ctx_len, n_splits=S)
    o, ml = ops.split_views(ws, S, 4, 8, 128)
    o = o.cpu().numpy().astype(np.float64)
    ml = ml.cpu().numpy().astype(np.float64)
    n_tiles = (w.ctx_len + 4 + 31) // 32
    bounds = [(32 * (s * n_tiles // S), min(304, 32 * ((s + 1) * n_tiles // S))) for s in range(S)]
    rm, rl, ro = oracle.split_partials(inp.q, w.ctx_len + np.arange(4), inp.k_codes, inp.k_scales,
                                       inp.v_codes, inp.v_scales, bounds)
    for s in range(S):
        got = o[s] / ml[s, ..., 1:2]
        ref = ro[s] / rl[s][..., None]
        assert_parity(got, ref, f"split {s} o/l")
        # the same partial under the kernel's reference point: l scales by 2^(m_ref - m_kernel)
        ratio = ml[s, ..., 1] / (rl[s] * np.exp2(rm[s] - ml[s, ..., 0]))
        assert np.allclose(ratio, 1.0, rtol=1e-5)


def test_bad_arguments_on_gpu():
    w = W.TINY_VERIFY
    inp = W.generate(w)
    q, kc, ks, vc, vs = to_device(inp)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(Exception):
        ops.verify_partials(q, kc, ks, vc, vs, ctx_len=w.ctx_len, workspace=small)
    with pytest.raises(Exception):
        ops.verify(q, kc, ks, vc, vs, ctx_len=w.ctx_len + 1)  # rows run past the cache


def test_dominant_logit_selects_its_value():
    """One key's logit exceeds the others by 31.75: the output is that key's Vhat
    (the other keys weigh at most 49 e^-31.75 ~ 8e-13 in all, far below the
    kernel's hi+lo rounding, bounded here by 2^-20 of max|Vhat|)."""
    hd, T = 64, 50
    w = W.VerifyWorkload("dominant", 1, 1, hd, T - 1, 1, 1, seed=14)
    inp = W.generate(w)
    rng = np.random.default_rng(14)
    inp.k_codes[:] = 0
    inp.k_scales[:] = np.float16(0.01)
    tstar = 23
    inp.k_codes[0, tstar, 0] = 127
    inp.k_scales[0, tstar, 0] = np.float16(2.0)
    inp.v_codes[:] = rng.integers(-127, 128, size=inp.v_codes.shape).astype(np.int8)
    inp.v_scales[:] = np.float16(0.02)
    inp.q[:] = 0
    inp.q[0, 0, 0] = 1.0
    _, got, _ = run_verify(w, inp=inp)
    vhat = oracle.dequantize(inp.v_codes, inp.v_scales)
    assert np.max(np.abs(got[0, 0] - vhat[0, tstar])) <= 2.0 ** -20 * np.abs(vhat).max()


def test_verify_window_inside_convex_hull():
    """Every output element lies between the smallest and largest Vhat of its
    visible keys (up to fp32 rounding of the weighted mean)."""
    w = W.VERIFY_WINDOW
    note("verify window: convex hull of the visible values")
    inp, got, _ = run_verify(w)
    G = w.n_q_heads // w.n_kv_heads
    for g in range(w.n_kv_heads):
        vhat = oracle.dequantize(inp.v_codes[g, : w.ctx_len + w.n_rows], inp.v_scales[g, : w.ctx_len + w.n_rows])
        tol = 1e-6 * np.abs(vhat).max()
        lo = vhat[: w.ctx_len + 1].min(axis=0)
        hi = vhat[: w.ctx_len + 1].max(axis=0)
        for r in range(w.n_rows):
            if r > 0:
                lo = np.minimum(lo, vhat[w.ctx_len + r])
                hi = np.maximum(hi, vhat[w.ctx_len + r])
            out = got[r, g * G:(g + 1) * G]
            assert np.all(out >= lo - tol) and np.all(out <= hi + tol), f"row {r} KV head {g}"
