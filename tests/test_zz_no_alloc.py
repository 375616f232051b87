"""attn_verify_q8_static (the entry point that allocates nothing) against the
workspace path attn_verify_q8 + attn_reduce_partials, through the C ABI."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from attention_int8_quantized_amd import _lib, ops
from gpu_util import assert_parity, note, to_device

pytestmark = pytest.mark.gpu


def _pair(w, rows_per_group=0):
    inp = W.generate(w)
    dev = to_device(inp)
    n_rows, hq, hd = inp.q.shape
    S = ops.verify_splits(hq, w.n_kv_heads, hd, w.ctx_len, n_rows, rows_per_group)
    ref_dev = ops.verify(*dev, ctx_len=w.ctx_len, rows_per_group=rows_per_group, n_splits=S)
    out = torch.full((n_rows, hq, hd), float("nan"), dtype=torch.float32, device="cuda")
    ops.verify_static(*dev, ctx_len=w.ctx_len, out=out, rows_per_group=rows_per_group)
    torch.cuda.synchronize()
    path = ops.last_path()
    return inp, out.cpu().numpy(), ref_dev.cpu().numpy(), path, S


def test_static_matches_workspace_path_twice():
    """Two calls in a row, the second with a smaller input: each output is
    bitwise the workspace path's (same split count) and within the oracle's
    tolerance (the scratch keeps the first call's larger partials; the second
    call must use only its own)."""
    for w in (W.VERIFY_WINDOW, W.TINY_VERIFY):
        note(f"static verify {w.name}")
        inp, got, ref_ws, path, S = _pair(w)
        note(f"  path: {path}")
        assert path.startswith("static verify") and f"splits{S}" in path
        assert np.array_equal(got.view(np.uint32), ref_ws.view(np.uint32))
        rows = list(range(inp.q.shape[0]))
        ref = oracle.verify(inp.q, inp.k_codes, inp.k_scales, inp.v_codes, inp.v_scales, w.ctx_len, rows=rows)
        assert_parity(got, ref, f"static {w.name}")


def test_static_split_cap_and_limits():
    """A shape whose automatic splits exceed the scratch (one row of 128 Q heads
    over one KV head at head_dim 256: 256 splits of 132 KB) takes the splits
    that fit, and still matches the workspace path at that count; an explicit
    split count beyond the scratch is refused with nothing launched."""
    w = W.VerifyWorkload("static_cap", 128, 1, 256, 16384, 1, 1)
    note("static verify: split cap (128/1 heads, hd 256, ctx 16384, 1 row)")
    inp = W.generate(w)
    dev = to_device(inp)
    n_rows, hq, hd = inp.q.shape
    per = ops.workspace_bytes(n_rows, hq, hd, 1)
    fit = _lib.STATIC_SCRATCH_BYTES // per
    auto = ops.verify_splits(hq, w.n_kv_heads, hd, w.ctx_len, n_rows, 0)
    note(f"  per split {per} B, fits {fit}, automatic {auto}")
    assert auto > fit
    out = torch.full((n_rows, hq, hd), float("nan"), dtype=torch.float32, device="cuda")
    with pytest.raises(_lib.Attnq8Error) as e:
        ops.verify_static(*dev, ctx_len=w.ctx_len, out=out, n_splits=fit + 1)
    assert e.value.status == _lib.EWORKSPACE
    ops.verify_static(*dev, ctx_len=w.ctx_len, out=out)
    torch.cuda.synchronize()
    path = ops.last_path()
    note(f"  path: {path}")
    assert f"splits{fit}" in path
    ref_ws = ops.verify(*dev, ctx_len=w.ctx_len, n_splits=fit).cpu().numpy()
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref_ws.view(np.uint32))
    ref = oracle.verify(inp.q, inp.k_codes, inp.k_scales, inp.v_codes, inp.v_scales, w.ctx_len)
    assert_parity(got, ref, "static split cap")
