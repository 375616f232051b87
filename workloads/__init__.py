"""Seeded synthetic workloads for int8-KV GQA attention.

This module is shared by the tests, the benchmark and the oracle harness.  It
holds only the input recipe: the workload shapes, the seeded random draws and
the block-32 int8 quantisation that turns fp32 K/V draws into the cache format
the attention consumes.  It performs none of the attention arithmetic.

Cache format (the pages call it "Q8 KV": "perf(gfx1100): share Q8 KV scans
across verifier rows", Summary; int8 blocks with one scale per block of 32 as in
the Q8_0 format of "[Engine] perf(hip): optimize MTP draft, shared expert, and
verify/sampler head kernels on RDNA4", Approach):

* codes  int8    [n_kv_heads][kv_stride][head_dim]
* scales float16 [n_kv_heads][kv_stride][head_dim // 32]

A block is 32 consecutive head_dim elements of one (KV head, token).  The scale
is the fp16 rounding of amax / 127 (computed in fp32); each code is x / d in
fp32 rounded half away from zero and clamped to [-127, 127]; an all-zero block
has scale 0 and codes 0.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import numpy as np

BLOCK = 32
QMAX = 127


# ----------------------------------------------------------------------------
# workload shapes
# ----------------------------------------------------------------------------


@dataclass(frozen=True)
class VerifyWorkload:
    """Speculative-decode verify: n_rows sequential query rows after ctx_len tokens.

    Row i sits at position ctx_len + i and sees keys 0 .. ctx_len + i.  The KV
    buffers already hold the rows' own keys (ctx_len + n_rows tokens).
    """

    name: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ctx_len: int
    n_rows: int
    rows_per_group: int
    peaked_frac: float = 0.0  # fraction of token positions whose K is multiplied
    peaked_mult: float = 8.0
    seed: int = 0
    kv_stride: Optional[int] = None  # token capacity of the cache (>= ctx_len + n_rows)

    kind: str = field(default="verify", init=False)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def kv_tokens(self) -> int:
        return self.ctx_len + self.n_rows

    @property
    def stride(self) -> int:
        return self.kv_stride if self.kv_stride is not None else self.kv_tokens

    def visible_kv_bytes(self, rows_per_group: Optional[int] = None) -> int:
        """int8 codes + fp16 scales of K and V that one pass per row group reads.

        A row group of rows [r0, r1) reads keys 0 .. ctx_len + r1 - 1.
        """
        rg = rows_per_group or self.rows_per_group
        per_tok = 2 * (self.head_dim + 2 * (self.head_dim // BLOCK))
        total = 0
        for r0 in range(0, self.n_rows, rg):
            r1 = min(self.n_rows, r0 + rg)
            total += (self.ctx_len + r1) * per_tok * self.n_kv_heads
        return total

    def unique_kv_bytes(self) -> int:
        per_tok = 2 * (self.head_dim + 2 * (self.head_dim // BLOCK))
        return self.kv_tokens * per_tok * self.n_kv_heads

    def visible_pairs(self) -> int:
        """Number of visible (row, q head, key) triples."""
        return sum(self.ctx_len + r + 1 for r in range(self.n_rows)) * self.n_q_heads

    def algorithmic_flops(self) -> int:
        """2*hd for q.k plus 2*hd for p.v per visible triple."""
        return 4 * self.head_dim * self.visible_pairs()


@dataclass(frozen=True)
class PromptWorkload:
    """Chunked causal prompt attention: n_queries at positions q_pos0 .. q_pos0+n_queries-1.

    kv_len tokens are in the cache (the chunk's own tokens included); query i
    sees keys 0 .. q_pos0 + i.
    """

    name: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    kv_len: int
    n_queries: int
    seed: int = 0
    q_pos0: Optional[int] = None  # default: the chunk sits at the end of the context
    kv_stride: Optional[int] = None

    kind: str = field(default="prompt", init=False)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def pos0(self) -> int:
        return self.q_pos0 if self.q_pos0 is not None else self.kv_len - self.n_queries

    @property
    def kv_tokens(self) -> int:
        return self.kv_len

    @property
    def stride(self) -> int:
        return self.kv_stride if self.kv_stride is not None else self.kv_len

    def visible_pairs(self) -> int:
        p0 = self.pos0
        n = self.n_queries
        # sum_{i<n} (p0 + i + 1)
        return (n * (p0 + 1) + n * (n - 1) // 2) * self.n_q_heads

    def algorithmic_flops(self) -> int:
        return 4 * self.head_dim * self.visible_pairs()

    def kv_bytes(self) -> int:
        per_tok = 2 * (self.head_dim + 2 * (self.head_dim // BLOCK))
        return self.kv_len * per_tok * self.n_kv_heads


# The five workloads the pages measure (shapes from "perf(gfx1100): share Q8 KV
# scans across verifier rows", Kernel evidence, and "hip: gfx12 (RDNA4) WMMA
# kernel for the int8-KV QSA prompt attention", Measurements).
TINY_VERIFY = VerifyWorkload("tiny_verify", 4, 1, 64, 256, 4, 4)
VERIFY_WINDOW = VerifyWorkload("verify_window", 24, 4, 256, 20676, 8, 8)
VERIFY_BATCH = VerifyWorkload("verify_batch", 32, 8, 128, 8192, 32, 4)
PROMPT_CHUNK = PromptWorkload("prompt_chunk", 12, 1, 256, 32768, 2048)
LONG_VERIFY = VerifyWorkload("long_verify", 24, 4, 256, 131072, 4, 4, peaked_frac=0.01)

WORKLOADS = {
    w.name: w for w in (TINY_VERIFY, VERIFY_WINDOW, VERIFY_BATCH, PROMPT_CHUNK, LONG_VERIFY)
}


def with_changes(w, **kw):
    return replace(w, **kw)


# ----------------------------------------------------------------------------
# block-32 int8 quantisation of the synthetic fp32 draws (input recipe)
# ----------------------------------------------------------------------------


def quantize_blocks(x: np.ndarray):
    """fp32 [..., hd] -> (codes int8 [..., hd], scales float16 [..., hd/32])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    hd = x.shape[-1]
    if hd % BLOCK:
        raise ValueError("head_dim must be a multiple of 32")
    xb = x.reshape(x.shape[:-1] + (hd // BLOCK, BLOCK))
    amax = np.max(np.abs(xb), axis=-1)  # fp32
    d16 = (amax / np.float32(QMAX)).astype(np.float16)  # fp32 divide, RNE to fp16
    d32 = d16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = xb / d32[..., None]  # fp32 divide
    y = y.astype(np.float64)
    r = np.sign(y) * np.floor(np.abs(y) + 0.5)  # half away from zero
    r = np.where(d32[..., None] == 0, 0.0, r)
    r = np.clip(r, -QMAX, QMAX)
    codes = r.astype(np.int8).reshape(x.shape)
    return codes, d16


# ----------------------------------------------------------------------------
# seeded generation
# ----------------------------------------------------------------------------


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    return [np.random.default_rng(s) for s in ss.spawn(4)]


@dataclass
class Inputs:
    """One workload's host arrays, in the layouts the C ABI takes."""

    workload: object
    q: np.ndarray  # verify: fp32 [n_rows][Hq][hd]; prompt: fp16 [n_q][Hq][hd]
    k_codes: np.ndarray  # int8 [Hkv][stride][hd]
    k_scales: np.ndarray  # fp16 [Hkv][stride][hd/32]
    v_codes: np.ndarray
    v_scales: np.ndarray
    peaked_tokens: Optional[np.ndarray] = None


def generate(w) -> Inputs:
    """Draw q, K and V ~ N(0,1) (fp32) from seeded streams and quantise K/V.

    Streams: SeedSequence(seed).spawn(4) -> q, K, V, peaked-token choice.
    Draws are taken in C order of the ABI layouts over the tokens in use; the
    cache's unused tail (stride > tokens) holds zero codes and zero scales.
    For the peaked workload, round(peaked_frac * tokens) distinct token
    positions are drawn and K at those positions (all heads) is multiplied by
    peaked_mult before quantisation; V is untouched.
    """
    rq, rk, rv, rp = _streams(w.seed)
    hd, hkv, hq = w.head_dim, w.n_kv_heads, w.n_q_heads
    T = w.kv_tokens
    S = w.stride
    if S < T:
        raise ValueError("kv_stride smaller than the tokens in use")
    if w.kind == "verify":
        q = rq.standard_normal((w.n_rows, hq, hd), dtype=np.float32)
    else:
        q = rq.standard_normal((w.n_queries, hq, hd), dtype=np.float32).astype(np.float16)
    k = rk.standard_normal((hkv, T, hd), dtype=np.float32)
    v = rv.standard_normal((hkv, T, hd), dtype=np.float32)
    peaked = None
    frac = getattr(w, "peaked_frac", 0.0)
    if frac > 0:
        n = int(round(frac * T))
        peaked = np.sort(rp.choice(T, size=n, replace=False))
        k[:, peaked, :] *= np.float32(w.peaked_mult)
    kc, ks = quantize_blocks(k)
    vc, vs = quantize_blocks(v)
    del k, v
    if S > T:
        pad = ((0, 0), (0, S - T), (0, 0))
        kc = np.pad(kc, pad)
        vc = np.pad(vc, pad)
        ks = np.pad(ks, pad)
        vs = np.pad(vs, pad)
    return Inputs(w, q, kc, ks, vc, vs, peaked)


@dataclass
class Inputs16:
    """A workload's inputs for an fp16 K/V cache (no scales)."""

    workload: object
    q: np.ndarray  # as for Inputs
    k: np.ndarray  # float16 [Hkv][stride][hd]
    v: np.ndarray


def generate_f16kv(w) -> Inputs16:
    """The same seeded draws as generate(), with K and V rounded to fp16 instead of
    quantised to int8 blocks (the peaked-token multiplier applies as there)."""
    rq, rk, rv, rp = _streams(w.seed)
    hd, hkv, hq = w.head_dim, w.n_kv_heads, w.n_q_heads
    T = w.kv_tokens
    S = w.stride
    if S < T:
        raise ValueError("kv_stride smaller than the tokens in use")
    if w.kind == "verify":
        q = rq.standard_normal((w.n_rows, hq, hd), dtype=np.float32)
    else:
        q = rq.standard_normal((w.n_queries, hq, hd), dtype=np.float32).astype(np.float16)
    k = rk.standard_normal((hkv, T, hd), dtype=np.float32)
    v = rv.standard_normal((hkv, T, hd), dtype=np.float32)
    frac = getattr(w, "peaked_frac", 0.0)
    if frac > 0:
        n = int(round(frac * T))
        peaked = np.sort(rp.choice(T, size=n, replace=False))
        k[:, peaked, :] *= np.float32(w.peaked_mult)
    k16 = k.astype(np.float16)
    v16 = v.astype(np.float16)
    del k, v
    if S > T:
        pad = ((0, 0), (0, S - T), (0, 0))
        k16 = np.pad(k16, pad)
        v16 = np.pad(v16, pad)
    return Inputs16(w, q, k16, v16)


def describe(w) -> Dict[str, object]:
    d = {k: getattr(w, k) for k in w.__dataclass_fields__ if k != "kind"}
    d["kind"] = w.kind
    return d
