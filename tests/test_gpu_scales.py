"""Attention over int8 caches whose V scales span the whole fp16 range.

The Q8 format carries one fp16 scale per 32-element block, any value up to
65,504 ("[Engine] perf(hip): optimize MTP draft, shared expert, and
verify/sampler head kernels on RDNA4", Problem and result item 2).  Each cache
here is written from finite fp32 rows by the library's own append quantiser
(attn_kv_append_q8, bit-exact against the oracle in test_gpu_append.py), then
read back for the oracle: V drawn at N(0, 1e5) (scales near 3,000), at
N(0, 1e-6) (fp16-subnormal scales), with one element of 65,504 in some
tokens' blocks (scale 516, just past the range the plain fold covers), up to
the largest finite scale, and with token magnitudes spread over eleven
decades; and K at N(0, 1e5), with blocks holding 65,504 and with mixed
magnitudes (q scaled down so that the logits stay of order one), which the
verify kernels' folded K fragments take through their exact per-unit path.
Every verify and prompt kernel instance family is run.
"""

import zlib

import numpy as np
import pytest
import torch

import oracle
from attention_int8_quantized_amd import ops
from gpu_util import assert_parity, note

pytestmark = pytest.mark.gpu


def _v_rows(kind, rng, T, H, hd):
    z = rng.standard_normal((T, H, hd), dtype=np.float32)
    if kind == "v_1e5":
        return z * np.float32(1e5)
    if kind == "v_1e-6":
        return z * np.float32(1e-6)
    if kind == "v_65504":
        # one element of 65,504 in some tokens (all positive: with random signs
        # the large terms cancel to outputs thousands of times smaller than
        # their sum, and fp32 accumulation -- any implementation's -- then
        # carries ~1e-4 of the row's largest output)
        t = rng.choice(T, size=max(1, T // 50), replace=False)
        z[t, :, rng.integers(0, hd)] = np.float32(65504.0)
        return z
    if kind == "v_max":
        # the largest block maxima stay below 127 * 65,504 (a finite scale)
        return np.clip(z * np.float32(1.5e6), -8.3e6, 8.3e6).astype(np.float32)
    if kind == "v_mixed":
        mag = np.float32(10.0) ** rng.uniform(-6, 5, size=(T, 1, 1)).astype(np.float32)
        return z * mag
    return z


def _k_rows(kind, rng, T, H, hd):
    """K at extreme scales; the test scales q down by q_scale(kind) so that the
    logits stay of order one."""
    z = rng.standard_normal((T, H, hd), dtype=np.float32)
    if kind == "k_1e5":
        return z * np.float32(1e5)
    if kind == "k_65504":
        t = rng.choice(T, size=max(1, T // 50), replace=False)
        z[t, :, rng.integers(0, hd)] = np.float32(65504.0) * np.sign(rng.standard_normal(t.size))[:, None]
        return z
    if kind == "k_mixed":
        mag = np.float32(10.0) ** rng.uniform(-6, 5, size=(T, 1, 1)).astype(np.float32)
        return z * mag
    return z


def q_scale(kind):
    return {"k_1e5": 1e-5, "k_65504": 1e-3, "k_mixed": 1e-5}.get(kind, 1.0)


def _cache(kind, seed, H, T, hd, stride):
    rng = np.random.default_rng(seed)
    k = _k_rows(kind, rng, T, H, hd)
    v = _v_rows(kind, rng, T, H, hd)
    dev = torch.device("cuda")
    kc = torch.zeros((H, stride, hd), dtype=torch.int8, device=dev)
    vc = torch.zeros_like(kc)
    ks = torch.zeros((H, stride, hd // 32), dtype=torch.float16, device=dev)
    vs = torch.zeros_like(ks)
    ops.kv_append(torch.from_numpy(k).to(dev), kc, ks, 0, v=torch.from_numpy(v).to(dev), v_codes=vc,
                  v_scales=vs)
    torch.cuda.synchronize()
    host = [t.cpu().numpy() for t in (kc, ks, vc, vs)]
    vmax = float(max(np.abs(host[1].astype(np.float32)).max(), np.abs(host[3].astype(np.float32)).max()))
    return (kc, ks, vc, vs), host, vmax


def _seed(kind, shape):
    return zlib.crc32(repr((kind, shape)).encode())


KINDS = ["v_1e5", "v_1e-6", "v_65504", "v_max", "v_mixed", "k_1e5", "k_65504", "k_mixed"]

VERIFY = [
    # hq, hkv, hd, ctx, rows, rows_per_group
    (24, 4, 256, 3000, 8, 0),    # three vector tiles (the verify window's instance)
    (24, 4, 256, 5000, 4, 0),    # two vector tiles (the long verify's)
    (32, 8, 128, 2000, 32, 0),   # eight vector tiles at head_dim 128
    (32, 8, 128, 2000, 32, 4),   # the pages' R4 grouping
    (4, 1, 64, 256, 4, 0),       # the tiny verify's shape
]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("shape", VERIFY, ids=lambda c: "-".join(map(str, c)))
def test_verify_scale_range(kind, shape):
    hq, hkv, hd, ctx, rows, rg = shape
    note(f"verify scales {kind} {shape}")
    T = ctx + rows
    dev_cache, (kc, ks, vc, vs), vmax = _cache(kind, _seed(kind, shape), hkv, T, hd, T + 5)
    rng = np.random.default_rng(7)
    q = rng.standard_normal((rows, hq, hd), dtype=np.float32) * np.float32(q_scale(kind))
    out = ops.verify(torch.from_numpy(q).cuda(), *dev_cache, ctx_len=ctx, rows_per_group=rg)
    torch.cuda.synchronize()
    note(f"  path: {ops.last_path()}  largest scale {vmax:.4g}")
    ref = oracle.verify(q, kc, ks, vc, vs, ctx)
    assert_parity(out.cpu().numpy(), ref, f"verify {kind} {shape}")


PROMPT = [
    # hq, hkv, hd, kv_len, n_queries
    (12, 1, 256, 1500, 256),     # the own layout (six vector tiles)
    (8, 2, 128, 700, 100),       # eight vector tiles at head_dim 128
    (16, 1, 64, 900, 96),        # eight vector tiles at head_dim 64
]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("shape", PROMPT, ids=lambda c: "-".join(map(str, c)))
def test_prompt_scale_range(kind, shape):
    hq, hkv, hd, kv_len, n = shape
    note(f"prompt scales {kind} {shape}")
    dev_cache, (kc, ks, vc, vs), vmax = _cache(kind, _seed(kind, shape), hkv, kv_len, hd, kv_len)
    rng = np.random.default_rng(8)
    q = (rng.standard_normal((n, hq, hd), dtype=np.float32) * np.float32(q_scale(kind))).astype(np.float16)
    pos0 = kv_len - n
    out = ops.prompt(torch.from_numpy(q).cuda(), *dev_cache, q_pos0=pos0, kv_len=kv_len)
    torch.cuda.synchronize()
    note(f"  path: {ops.last_path()}  largest scale {vmax:.4g}")
    ref = oracle.prompt(q, kc, ks, vc, vs, pos0)
    assert_parity(out.cpu().numpy(), ref, f"prompt {kind} {shape}")
