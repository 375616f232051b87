"""The C ABI library loads, exports every declared symbol and rejects bad
arguments on the host before any HIP call (CPU only, no GPU needed)."""

import ctypes
import os

import pytest

from attention_int8_quantized_amd import _lib

A = 0x10000  # a 16-byte aligned fake device address; never dereferenced here


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = _lib.header_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib._SIGNATURES)


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4, -5):
        assert _lib.status_string(st)
    assert _lib.status_string(7) == "unknown status"


def test_workspace_bytes(lib):
    f = lib.attn_verify_q8_workspace_bytes
    assert f(8, 24, 256, 64) == 64 * 8 * 24 * 258 * 4
    assert f(0, 24, 256, 64) == 0
    assert f(4, 4, 64, 0) == 0


def test_auto_splits(lib):
    f = lib.attn_verify_q8_splits
    # about one workgroup per CU at head_dim 256 and 128 (two at 64), never
    # fewer than two 32-key tiles per split
    assert f(24, 4, 256, 20676, 8, 0) == 64
    assert f(24, 4, 256, 131072, 4, 0) == 64
    assert f(24, 4, 256, 20676, 32, 0) == 16     # at 256, 10 rows (60 vectors) per group: 4 groups
    assert f(32, 8, 128, 8192, 32, 0) == 16      # two groups of 64 vectors per KV head
    assert f(32, 8, 128, 8192, 32, 32) == 32     # one group of 128 vectors per KV head
    assert f(32, 8, 128, 8192, 32, 4) == 4
    assert f(4, 1, 64, 256, 4, 0) == 4         # 260 keys -> 9 tiles -> at most 4 splits
    assert f(4, 1, 64, 0, 1, 0) == 1
    assert f(4, 3, 64, 10, 4, 0) == _lib.EINVAL
    assert f(4, 1, 96, 10, 4, 0) == _lib.EUNSUPPORTED
    assert f(4, 1, 64, 10, 33, 0) == _lib.EINVAL
    assert f(64, 1, 64, 10, 4, 4) == _lib.EINVAL  # 256 vectors per group > 128
    assert f(8, 1, 64, 10, 4, 1 << 29) == _lib.EINVAL  # the product would wrap to 0 in 32 bits


def _verify(lib, **kw):
    args = dict(q=A, q_dtype=0, kc=A, ks=A, vc=A, vs=A, hq=4, hkv=1, hd=64, stride=300, ctx=256,
                rows=4, rg=0, splits=0, ws=A, ws_bytes=1 << 30, sm=0.0, stream=None)
    args.update(kw)
    return lib.attn_verify_q8(args["q"], args["q_dtype"], args["kc"], args["ks"], args["vc"],
                              args["vs"], args["hq"], args["hkv"], args["hd"], args["stride"],
                              args["ctx"], args["rows"], args["rg"], args["splits"], args["ws"],
                              args["ws_bytes"], args["sm"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), _lib.EINVAL),
    (dict(kc=None), _lib.EINVAL),
    (dict(vs=None), _lib.EINVAL),
    (dict(ws=None), _lib.EINVAL),
    (dict(q_dtype=2), _lib.EINVAL),
    (dict(hkv=3), _lib.EINVAL),
    (dict(hq=0), _lib.EINVAL),
    (dict(hd=96), _lib.EUNSUPPORTED),
    (dict(hd=512), _lib.EUNSUPPORTED),
    (dict(rows=0), _lib.EINVAL),
    (dict(rows=33), _lib.EINVAL),
    (dict(ctx=-1), _lib.EINVAL),
    (dict(ctx=297), _lib.EINVAL),          # ctx + rows > stride
    (dict(rg=-1), _lib.EINVAL),
    (dict(rg=40), _lib.EINVAL),            # 160 vectors per group
    (dict(rg=1 << 29, hq=8, hkv=1), _lib.EINVAL),  # rows_per_group * G wraps to 0 in 32 bits
    (dict(rg=(1 << 31) - 1), _lib.EINVAL),
    (dict(splits=10), _lib.EINVAL),        # more splits than 9 tiles
    (dict(splits=-2), _lib.EINVAL),
    (dict(sm=float("nan")), _lib.EINVAL),
    (dict(sm=-1.0), _lib.EINVAL),
    (dict(sm=float("inf")), _lib.EINVAL),
    (dict(q=A + 8), _lib.EALIGN),
    (dict(kc=A + 4), _lib.EALIGN),
    (dict(ks=A + 2), _lib.EALIGN),
    (dict(ws=A + 4), _lib.EALIGN),
    (dict(ws_bytes=100), _lib.EWORKSPACE),
    (dict(splits=9, ws_bytes=9 * 4 * 4 * 66 * 4 - 1), _lib.EWORKSPACE),
    (dict(hq=65536, hkv=65536), _lib.EINVAL),  # KV heads beyond the launch's third grid dimension
])
def test_verify_rejects_before_launch(lib, kw, status):
    assert _verify(lib, **kw) == status


def _prompt(lib, **kw):
    args = dict(q=A, q_dtype=1, kc=A, ks=A, vc=A, vs=A, hq=12, hkv=1, hd=256, stride=4096,
                kv_len=4096, pos0=2048, n=2048, sm=0.0, out=A, stream=None)
    args.update(kw)
    return lib.attn_prompt_q8(args["q"], args["q_dtype"], args["kc"], args["ks"], args["vc"],
                              args["vs"], args["hq"], args["hkv"], args["hd"], args["stride"],
                              args["kv_len"], args["pos0"], args["n"], args["sm"], args["out"],
                              args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(out=None), _lib.EINVAL),
    (dict(q=None), _lib.EINVAL),
    (dict(n=0), _lib.EINVAL),
    (dict(pos0=-1), _lib.EINVAL),
    (dict(pos0=2049), _lib.EINVAL),        # last query beyond kv_len
    (dict(kv_len=5000), _lib.EINVAL),      # kv_len > stride
    (dict(hq=13, hkv=2), _lib.EINVAL),
    (dict(hd=32), _lib.EUNSUPPORTED),
    (dict(out=A + 4), _lib.EALIGN),
    (dict(vc=A + 1), _lib.EALIGN),
    (dict(sm=float("nan")), _lib.EINVAL),
    (dict(hq=65536, hkv=65536), _lib.EINVAL),  # KV heads beyond the launch's third grid dimension
])
def test_prompt_rejects_before_launch(lib, kw, status):
    assert _prompt(lib, **kw) == status


def test_reduce_rejects_before_launch(lib):
    f = lib.attn_reduce_partials
    assert f(None, 1 << 20, 4, 4, 64, 2, A, None) == _lib.EINVAL
    assert f(A, 1 << 20, 4, 4, 64, 2, None, None) == _lib.EINVAL
    assert f(A, 1 << 20, 0, 4, 64, 2, A, None) == _lib.EINVAL
    assert f(A, 1 << 20, 4, 4, 64, 0, A, None) == _lib.EINVAL
    assert f(A, 1 << 20, 4, 4, 48, 2, A, None) == _lib.EUNSUPPORTED
    assert f(A + 4, 1 << 20, 4, 4, 64, 2, A, None) == _lib.EALIGN
    assert f(A, 100, 4, 4, 64, 2, A, None) == _lib.EWORKSPACE
    # (row, head) pairs past INT_MAX would wrap the grid size
    assert f(A, 1 << 62, 1 << 16, 1 << 15, 64, 1, A, None) == _lib.EINVAL


def _append(lib, **kw):
    args = dict(k=A, v=A, dt=0, T=8, H=4, hd=256, kc=A, ks=A, vc=A, vs=A, stride=20684, pos0=20676,
                stream=None)
    args.update(kw)
    return lib.attn_kv_append_q8(args["k"], args["v"], args["dt"], args["T"], args["H"], args["hd"],
                                 args["kc"], args["ks"], args["vc"], args["vs"], args["stride"],
                                 args["pos0"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(k=None), _lib.EINVAL),
    (dict(kc=None), _lib.EINVAL),
    (dict(vs=None), _lib.EINVAL),            # V given without its scales
    (dict(v=None), _lib.EINVAL),             # V cache given without V rows
    (dict(dt=2), _lib.EINVAL),
    (dict(T=-1), _lib.EINVAL),
    (dict(H=0), _lib.EINVAL),
    (dict(pos0=-1), _lib.EINVAL),
    (dict(pos0=20677), _lib.EINVAL),         # last row beyond the stride
    (dict(hd=48), _lib.EUNSUPPORTED),
    (dict(hd=8192), _lib.EUNSUPPORTED),
    (dict(k=A + 8), _lib.EALIGN),
    (dict(vc=A + 8), _lib.EALIGN),
    (dict(ks=A + 2), _lib.EALIGN),
    (dict(T=0), _lib.OK),                    # nothing to write: no launch, no HIP call
    (dict(T=0, v=None, vc=None, vs=None), _lib.OK),
    (dict(T=0, k=None, v=None), _lib.OK),    # empty rows may come as NULL
    (dict(T=0, kc=None), _lib.EINVAL),
])
def test_kv_append_rejects_before_launch(lib, kw, status):
    assert _append(lib, **kw) == status


def test_head_workspace_bytes(lib):
    f = lib.attn_verify_head_workspace_bytes
    # 4,096 bytes of tickets, then 24 bytes per block state: about 256 blocks
    # over all rows (ceil(256 / rows) per row), sized for 256 + rows states so
    # that the size grows with the row count
    assert f(1, 248320) == 4096 + 257 * 24
    assert f(5, 248320) == 4096 + 261 * 24
    assert f(64, 248320) == 4096 + 320 * 24
    assert f(1, 1) == 4096 + 257 * 24
    assert all(f(n, 248320) <= f(n + 1, 248320) for n in range(1, 1024))
    for n in (1, 3, 5, 7, 64, 100, 255, 257, 1024):  # rows * ceil(256 / rows) states fit
        assert n * -(-256 // n) * 24 <= f(n, 248320) - 4096
    assert f(0, 100) == 0 and f(3, 0) == 0 and f(1025, 100) == 0


def _head(lib, **kw):
    args = dict(x=A, rows=5, V=248320, stride=248320, tok=A, top=A, ws=A, ws_bytes=1 << 20,
                stream=None)
    args.update(kw)
    return lib.attn_verify_head_greedy(args["x"], args["rows"], args["V"], args["stride"],
                                       args["tok"], args["top"], args["ws"], args["ws_bytes"],
                                       args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), _lib.EINVAL),
    (dict(tok=None), _lib.EINVAL),
    (dict(ws=None), _lib.EINVAL),
    (dict(rows=0), _lib.EINVAL),
    (dict(rows=1025), _lib.EINVAL),
    (dict(V=0), _lib.EINVAL),
    (dict(stride=248319), _lib.EINVAL),
    (dict(x=A + 2), _lib.EALIGN),
    (dict(ws=A + 4), _lib.EALIGN),
    (dict(top=A + 1), _lib.EALIGN),
    (dict(ws_bytes=100), _lib.EWORKSPACE),
])
def test_head_rejects_before_launch(lib, kw, status):
    assert _head(lib, **kw) == status


@pytest.mark.parametrize("buf,nbytes,sink,status", [
    (None, 16, A, _lib.EINVAL),
    (A, 16, None, _lib.EINVAL),
    (A + 4, 16, A, _lib.EALIGN),
    (A, 17, A, _lib.EALIGN),
    (A, 16, A + 2, _lib.EALIGN),
])
def test_stream_read_rejects_before_launch(lib, buf, nbytes, sink, status):
    assert lib.attnq8_stream_read(buf, nbytes, sink, None) == status


def test_selftest_rejects_null(lib):
    assert lib.attnq8_selftest_i8_to_f16(None, None) == _lib.EINVAL


def test_library_is_in_tree():
    assert os.path.dirname(_lib.LIB_PATH).endswith("attention_int8_quantized_amd")
    assert isinstance(_lib.load(), ctypes.CDLL)


def _static(lib, **kw):
    args = dict(q=A, q_dtype=0, kc=A, ks=A, vc=A, vs=A, hq=4, hkv=1, hd=64, stride=300, ctx=256,
                rows=4, rg=0, splits=0, sm=0.0, out=A, stream=None)
    args.update(kw)
    return lib.attn_verify_q8_static(args["q"], args["q_dtype"], args["kc"], args["ks"], args["vc"],
                                     args["vs"], args["hq"], args["hkv"], args["hd"], args["stride"],
                                     args["ctx"], args["rows"], args["rg"], args["splits"], args["sm"],
                                     args["out"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(out=None), _lib.EINVAL),
    (dict(out=A + 4), _lib.EALIGN),
    (dict(q=None), _lib.EINVAL),
    (dict(kc=A + 4), _lib.EALIGN),
    (dict(hd=96), _lib.EUNSUPPORTED),
    (dict(rows=33), _lib.EINVAL),
    (dict(splits=-1), _lib.EINVAL),
    (dict(splits=10), _lib.EINVAL),                 # more splits than 9 tiles
    (dict(rg=1 << 29, hq=8), _lib.EINVAL),
    # one row of 128 heads at head_dim 256 holds 132,096 B of partials per split:
    # 254 splits fit the scratch, 255 do not
    (dict(hq=128, hd=256, stride=20000, ctx=16384, rows=1, splits=255), _lib.EWORKSPACE),
    # 32 rows of 1,024 heads: not even one split fits
    (dict(hq=1024, hkv=8, hd=256, stride=20000, ctx=16384, rows=32, splits=1), _lib.EWORKSPACE),
    (dict(hq=1024, hkv=8, hd=256, stride=20000, ctx=16384, rows=32, splits=0), _lib.EWORKSPACE),
])
def test_static_verify_rejects_before_any_hip_call(lib, kw, status):
    assert _static(lib, **kw) == status
