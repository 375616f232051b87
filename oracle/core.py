"""fp64 CPU oracle for scaled-dot-product GQA attention over an int8 block-32 KV cache.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library and never calls it.

What it computes is the plain definition the pages state:

* "perf(gfx1100): share Q8 KV scans across verifier rows" (Summary, Kernel
  evidence): attention of sequential verifier query rows over a Q8 KV cache,
  with split-context partials merged by a reducer;
* "hip: gfx12 (RDNA4) WMMA kernel for the int8-KV QSA prompt attention" (What,
  How): chunked causal prompt attention over an int8 KV cache; the page's
  hi+lo splits, fixed group order, online softmax and V-scale folding are an
  implementation of this same result, so the oracle does none of them.

Steps, per query row r (position pos_r), Q head h, with G = Hq / Hkv:

1. dequantise: Khat[g,t,j] = scale_K[g,t,j//32] * code_K[g,t,j] (same for V);
2. the row uses KV head g = h // G (heads are grouped consecutively);
3. s_t = sm_scale * sum_j q[r,h,j] * Khat[g,t,j] for the visible keys
   t = 0 .. pos_r (causal: a row sees its own position and everything before);
   sm_scale defaults to 1/sqrt(head_dim);
4. out = sum_t exp(s_t - m) Vhat[g,t,:] / sum_t exp(s_t - m), m = max_t s_t.

Verify rows sit at pos_r = ctx_len + r; prompt query i sits at q_pos0 + i.

Rows are processed a block at a time (each row's result is independent of the
others); within a row nothing is blocked, fused or reordered beyond numpy's own
matrix product and sum.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

BLOCK = 32
_LOG2E = 1.0 / math.log(2.0)


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes int8 [..., hd], scales fp16 [..., hd/32] -> fp64 [..., hd] (exact)."""
    codes = np.asarray(codes)
    scales = np.asarray(scales)
    hd = codes.shape[-1]
    nb = hd // BLOCK
    if scales.shape[-1] != nb or nb * BLOCK != hd:
        raise ValueError("scales must hold one value per 32 codes")
    c = codes.astype(np.float64).reshape(codes.shape[:-1] + (nb, BLOCK))
    d = scales.astype(np.float64)[..., None]
    return (c * d).reshape(codes.shape)


def kv_head_of(h: int, n_q_heads: int, n_kv_heads: int) -> int:
    """Q head h reads KV head h // (Hq / Hkv)."""
    return h // (n_q_heads // n_kv_heads)


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def _masked_rows(qrows: np.ndarray, pos: np.ndarray, khat: np.ndarray,
                 vhat: np.ndarray, sm_scale: float, chunk: int = 256) -> np.ndarray:
    """softmax(sm_scale * q.K^T masked to t <= pos) V for each row of qrows (fp64)."""
    out = np.empty((qrows.shape[0], vhat.shape[1]), dtype=np.float64)
    for a in range(0, qrows.shape[0], chunk):
        b = min(qrows.shape[0], a + chunk)
        p = pos[a:b]
        T = int(p.max()) + 1
        s = (qrows[a:b] @ khat[:T].T) * sm_scale
        visible = np.arange(T)[None, :] <= p[:, None]
        s = np.where(visible, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        out[a:b] = (w @ vhat[:T]) / w.sum(axis=1, keepdims=True)
    return out


def _attend(q: np.ndarray, positions: Sequence[int], values_of, hkv: int,
            sm_scale: Optional[float], rows: Optional[Sequence[int]]) -> np.ndarray:
    """Causal GQA attention; values_of(g, T) gives KV head g's (Khat, Vhat) for keys 0..T-1."""
    q = np.asarray(q)
    n, hq, hd = q.shape
    if hq % hkv:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    pos = np.asarray(positions, dtype=np.int64)
    if pos.shape != (n,):
        raise ValueError("one position per row")
    sel = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    scale = default_scale(hd) if sm_scale is None else float(sm_scale)
    out = np.empty((sel.size, hq, hd), dtype=np.float64)
    T = int(pos[sel].max()) + 1
    for g in range(hkv):
        heads = [h for h in range(hq) if kv_head_of(h, hq, hkv) == g]
        khat, vhat = values_of(g, T)
        for h in heads:
            qrows = q[sel, h, :].astype(np.float64)
            out[:, h, :] = _masked_rows(qrows, pos[sel], khat, vhat, scale)
    return out


def attention(q: np.ndarray, positions: Sequence[int], k_codes, k_scales, v_codes,
              v_scales, sm_scale: Optional[float] = None,
              rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Causal GQA attention of q [n][Hq][hd] rows at the given positions.

    Returns fp64 [n][Hq][hd], or [len(rows)][Hq][hd] when a subset of row
    indices is given.
    """
    return _attend(q, positions,
                   lambda g, T: (dequantize(k_codes[g, :T], k_scales[g, :T]),
                                 dequantize(v_codes[g, :T], v_scales[g, :T])),
                   np.asarray(k_codes).shape[0], sm_scale, rows)


def attention_values(q: np.ndarray, positions: Sequence[int], khat, vhat,
                     sm_scale: Optional[float] = None,
                     rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """The same attention over K/V values given directly: khat, vhat [Hkv][T][hd].

    An fp16 cache ("hip: gfx12 (RDNA4) WMMA kernel for the int8-KV QSA prompt
    attention", What: fp16 KV pools) has Khat = K and Vhat = V; the values are
    widened to fp64 exactly.
    """
    khat = np.asarray(khat)
    vhat = np.asarray(vhat)
    return _attend(q, positions,
                   lambda g, T: (khat[g, :T].astype(np.float64), vhat[g, :T].astype(np.float64)),
                   khat.shape[0], sm_scale, rows)


def verify(q, k_codes, k_scales, v_codes, v_scales, ctx_len: int,
           sm_scale: Optional[float] = None, rows=None) -> np.ndarray:
    """Verify rows: row r sits at ctx_len + r and sees ctx_len + r + 1 keys."""
    n = np.asarray(q).shape[0]
    return attention(q, ctx_len + np.arange(n), k_codes, k_scales, v_codes, v_scales,
                     sm_scale, rows)


def prompt(q, k_codes, k_scales, v_codes, v_scales, q_pos0: int,
           sm_scale: Optional[float] = None, rows=None) -> np.ndarray:
    """Prompt chunk: query i sits at q_pos0 + i and sees q_pos0 + i + 1 keys."""
    n = np.asarray(q).shape[0]
    return attention(q, q_pos0 + np.arange(n), k_codes, k_scales, v_codes, v_scales,
                     sm_scale, rows)


def _fp16(x):
    x = np.asarray(x)
    if x.dtype != np.float16:
        raise TypeError("an fp16 cache holds float16 values")
    return x


def verify_f16kv(q, k, v, ctx_len: int, sm_scale: Optional[float] = None,
                 rows=None) -> np.ndarray:
    """Verify rows over an fp16 cache k, v [Hkv][stride][hd]."""
    n = np.asarray(q).shape[0]
    return attention_values(q, ctx_len + np.arange(n), _fp16(k), _fp16(v), sm_scale, rows)


def prompt_f16kv(q, k, v, q_pos0: int, sm_scale: Optional[float] = None,
                 rows=None) -> np.ndarray:
    """Prompt chunk over an fp16 cache k, v [Hkv][stride][hd]."""
    n = np.asarray(q).shape[0]
    return attention_values(q, q_pos0 + np.arange(n), _fp16(k), _fp16(v), sm_scale, rows)


# ----------------------------------------------------------------------------
# split-context partials and their merge ("partials layout and reducer",
# "perf(gfx1100): share Q8 KV scans across verifier rows", Summary)
#
# Convention (the pages do not print one): logits are carried in base-2 units,
# x_t = s_t * log2(e).  For a split covering keys [a, b):
#   m = max of x_t over the keys of [a, b) the row sees (-inf if none),
#   l = sum 2^(x_t - m),  o = sum 2^(x_t - m) Vhat_t   (0 for an empty split).
# Any m gives the same merge; the kernels may use another reference point.
# ----------------------------------------------------------------------------


def split_partials(q, positions, k_codes, k_scales, v_codes, v_scales, bounds,
                   sm_scale: Optional[float] = None):
    """Partials (m, l, o) for key ranges bounds = [(a0,b0), (a1,b1), ...]."""
    q = np.asarray(q)
    n, hq, hd = q.shape
    hkv = k_codes.shape[0]
    pos = np.asarray(positions, dtype=np.int64)
    scale = default_scale(hd) if sm_scale is None else float(sm_scale)
    S = len(bounds)
    m = np.full((S, n, hq), -np.inf)
    l = np.zeros((S, n, hq))
    o = np.zeros((S, n, hq, hd))
    T = int(pos.max()) + 1
    for g in range(hkv):
        khat = dequantize(k_codes[g, :T], k_scales[g, :T])
        vhat = dequantize(v_codes[g, :T], v_scales[g, :T])
        for h in range(hq):
            if kv_head_of(h, hq, hkv) != g:
                continue
            for r in range(n):
                qv = q[r, h].astype(np.float64)
                for si, (a, b) in enumerate(bounds):
                    hi = min(b, int(pos[r]) + 1)
                    if hi <= a:
                        continue
                    x = (khat[a:hi] @ qv) * scale * _LOG2E
                    mm = x.max()
                    w = np.exp2(x - mm)
                    m[si, r, h] = mm
                    l[si, r, h] = w.sum()
                    o[si, r, h] = w @ vhat[a:hi]
    return m, l, o


def merge_partials(m: np.ndarray, l: np.ndarray, o: np.ndarray) -> np.ndarray:
    """out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, M = max over non-empty s.

    m, l: [S, ...]; o: [S, ..., hd].  Splits with l == 0 contribute nothing.
    """
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    live = l > 0
    M = np.where(live, m, -np.inf).max(axis=0)
    w = np.where(live, np.exp2(np.where(live, m, 0.0) - M[None]), 0.0)
    num = (w[..., None] * o).sum(axis=0)
    den = (w * l).sum(axis=0)
    return num / den[..., None]
