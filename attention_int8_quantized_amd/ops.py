"""torch-facing wrappers over the attnq8 C ABI.

Argument marshalling only: every step of the attention runs in the HIP
kernels of libattnq8.so.  torch supplies device memory and the current HIP
stream; tensors must already live on the GPU in the layouts of
include/attnq8.h.
"""

from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib

_QTYPES = {torch.float32: _lib.F32, torch.float16: _lib.F16}


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def _nbytes(t: torch.Tensor) -> int:
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    return t.numel() * t.element_size()


def _out(t: Optional[torch.Tensor], shape, dtype, device, name: str = "out") -> torch.Tensor:
    """A new output tensor, or the caller's after checking that the kernel's
    writes fit it exactly."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if not t.is_cuda or not t.is_contiguous() or t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous {dtype} GPU tensor of shape {tuple(shape)}")
    return t


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check_cache(q, k_codes, k_scales, v_codes, v_scales):
    for name, t in (("q", q), ("k_codes", k_codes), ("k_scales", k_scales), ("v_codes", v_codes),
                    ("v_scales", v_scales)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dtype not in _QTYPES:
        raise ValueError("q must be float32 or float16")
    if k_codes.dtype != torch.int8 or v_codes.dtype != torch.int8:
        raise ValueError("codes must be int8")
    if k_scales.dtype != torch.float16 or v_scales.dtype != torch.float16:
        raise ValueError("scales must be float16")
    if q.dim() != 3 or k_codes.dim() != 3 or k_scales.dim() != 3:
        raise ValueError("q [rows][Hq][hd], codes [Hkv][stride][hd], scales [Hkv][stride][hd/32]")
    if k_codes.shape != v_codes.shape or k_scales.shape != v_scales.shape:
        raise ValueError("K and V caches must have the same shape")
    hkv, stride, hd = k_codes.shape
    if q.shape[2] != hd or k_scales.shape != (hkv, stride, hd // 32):
        raise ValueError("inconsistent head_dim / scale shapes")
    return q.shape[0], q.shape[1], hkv, hd, stride


def verify_splits(n_q_heads, n_kv_heads, head_dim, ctx_len, n_rows, rows_per_group=0) -> int:
    s = _lib.load().attn_verify_q8_splits(n_q_heads, n_kv_heads, head_dim, ctx_len, n_rows,
                                          rows_per_group)
    if s < 0:
        raise _lib.Attnq8Error("attn_verify_q8_splits", s)
    return s


def workspace_bytes(n_rows, n_q_heads, head_dim, n_splits) -> int:
    return int(_lib.load().attn_verify_q8_workspace_bytes(n_rows, n_q_heads, head_dim, n_splits))


def verify_partials(q, k_codes, k_scales, v_codes, v_scales, ctx_len: int, rows_per_group: int = 0,
                    n_splits: int = 0, sm_scale: float = 0.0,
                    workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, int]:
    """Run attn_verify_q8; returns (workspace uint8 tensor, n_splits)."""
    n_rows, hq, hkv, hd, stride = _check_cache(q, k_codes, k_scales, v_codes, v_scales)
    lib = _lib.load()
    S = n_splits or verify_splits(hq, hkv, hd, ctx_len, n_rows, rows_per_group)
    need = workspace_bytes(n_rows, hq, hd, S)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = lib.attn_verify_q8(_ptr(q), _QTYPES[q.dtype], _ptr(k_codes), _ptr(k_scales),
                            _ptr(v_codes), _ptr(v_scales), hq, hkv, hd, stride, ctx_len, n_rows,
                            rows_per_group, S, _ptr(workspace), _nbytes(workspace),
                            float(sm_scale), _stream())
    _lib.check("attn_verify_q8", st)
    return workspace, S


def split_views(workspace: torch.Tensor, n_splits, n_rows, n_q_heads, head_dim):
    """(o [S][rows][Hq][hd], ml [S][rows][Hq][2]) float32 views of a workspace."""
    n_o = n_splits * n_rows * n_q_heads * head_dim
    f = workspace.view(torch.float32)
    o = f[:n_o].view(n_splits, n_rows, n_q_heads, head_dim)
    ml = f[n_o:n_o + 2 * n_splits * n_rows * n_q_heads].view(n_splits, n_rows, n_q_heads, 2)
    return o, ml


def reduce_partials(workspace: torch.Tensor, n_rows: int, n_q_heads: int, head_dim: int,
                    n_splits: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    out = _out(out, (n_rows, n_q_heads, head_dim), torch.float32, workspace.device)
    st = _lib.load().attn_reduce_partials(_ptr(workspace), _nbytes(workspace), n_rows, n_q_heads,
                                          head_dim, n_splits, _ptr(out), _stream())
    _lib.check("attn_reduce_partials", st)
    return out


def verify(q, k_codes, k_scales, v_codes, v_scales, ctx_len: int, rows_per_group: int = 0,
           n_splits: int = 0, sm_scale: float = 0.0, out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Verify attention: attn_verify_q8 followed by attn_reduce_partials."""
    ws, S = verify_partials(q, k_codes, k_scales, v_codes, v_scales, ctx_len, rows_per_group,
                            n_splits, sm_scale, workspace)
    return reduce_partials(ws, q.shape[0], q.shape[1], q.shape[2], S, out)


def verify_static(q, k_codes, k_scales, v_codes, v_scales, ctx_len: int, out: torch.Tensor,
                  rows_per_group: int = 0, n_splits: int = 0, sm_scale: float = 0.0) -> torch.Tensor:
    """Verify attention through attn_verify_q8_static: the partials live in the
    library's own scratch, so the call takes no workspace and allocates nothing;
    the caller provides `out` [n_rows][Hq][hd] float32."""
    n_rows, hq, hkv, hd, stride = _check_cache(q, k_codes, k_scales, v_codes, v_scales)
    if out.dtype != torch.float32 or tuple(out.shape) != (n_rows, hq, hd) or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError("out must be a contiguous float32 tensor [n_rows][Hq][hd] on q's device")
    st = _lib.load().attn_verify_q8_static(_ptr(q), _QTYPES[q.dtype], _ptr(k_codes), _ptr(k_scales),
                                           _ptr(v_codes), _ptr(v_scales), hq, hkv, hd, stride, ctx_len,
                                           n_rows, rows_per_group, n_splits, float(sm_scale), _ptr(out),
                                           _stream())
    _lib.check("attn_verify_q8_static", st)
    return out


def prompt(q, k_codes, k_scales, v_codes, v_scales, q_pos0: int, kv_len: Optional[int] = None,
           sm_scale: float = 0.0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Causal prompt attention of q [n_queries][Hq][hd] at positions q_pos0 + i."""
    n, hq, hkv, hd, stride = _check_cache(q, k_codes, k_scales, v_codes, v_scales)
    if kv_len is None:
        kv_len = q_pos0 + n
    out = _out(out, (n, hq, hd), torch.float32, q.device)
    st = _lib.load().attn_prompt_q8(_ptr(q), _QTYPES[q.dtype], _ptr(k_codes), _ptr(k_scales),
                                    _ptr(v_codes), _ptr(v_scales), hq, hkv, hd, stride, kv_len,
                                    q_pos0, n, float(sm_scale), _ptr(out), _stream())
    _lib.check("attn_prompt_q8", st)
    return out


def _check_cache16(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if q.dtype not in _QTYPES:
        raise ValueError("q must be float32 or float16")
    if k.dtype != torch.float16 or v.dtype != torch.float16:
        raise ValueError("an fp16 cache holds float16 K and V")
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape:
        raise ValueError("q [rows][Hq][hd], k and v [Hkv][stride][hd]")
    hkv, stride, hd = k.shape
    if q.shape[2] != hd:
        raise ValueError("inconsistent head_dim")
    return q.shape[0], q.shape[1], hkv, hd, stride


def verify_f16kv(q, k, v, ctx_len: int, rows_per_group: int = 0, n_splits: int = 0,
                 sm_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Verify attention over an fp16 cache: attn_verify_f16kv then attn_reduce_partials."""
    n_rows, hq, hkv, hd, stride = _check_cache16(q, k, v)
    lib = _lib.load()
    S = n_splits or verify_splits(hq, hkv, hd, ctx_len, n_rows, rows_per_group)
    need = workspace_bytes(n_rows, hq, hd, S)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = lib.attn_verify_f16kv(_ptr(q), _QTYPES[q.dtype], _ptr(k), _ptr(v), hq, hkv, hd, stride,
                               ctx_len, n_rows, rows_per_group, S, _ptr(workspace),
                               _nbytes(workspace), float(sm_scale), _stream())
    _lib.check("attn_verify_f16kv", st)
    return reduce_partials(workspace, n_rows, hq, hd, S, out)


def verify_f16kv_partials(q, k, v, ctx_len: int, rows_per_group: int = 0, n_splits: int = 0,
                          sm_scale: float = 0.0,
                          workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, int]:
    """attn_verify_f16kv alone; returns (workspace, n_splits)."""
    n_rows, hq, hkv, hd, stride = _check_cache16(q, k, v)
    S = n_splits or verify_splits(hq, hkv, hd, ctx_len, n_rows, rows_per_group)
    if workspace is None:
        workspace = torch.empty(workspace_bytes(n_rows, hq, hd, S), dtype=torch.uint8,
                                device=q.device)
    st = _lib.load().attn_verify_f16kv(_ptr(q), _QTYPES[q.dtype], _ptr(k), _ptr(v), hq, hkv, hd,
                                       stride, ctx_len, n_rows, rows_per_group, S, _ptr(workspace),
                                       _nbytes(workspace), float(sm_scale), _stream())
    _lib.check("attn_verify_f16kv", st)
    return workspace, S


def prompt_f16kv(q, k, v, q_pos0: int, kv_len: Optional[int] = None, sm_scale: float = 0.0,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Causal prompt attention over an fp16 cache."""
    n, hq, hkv, hd, stride = _check_cache16(q, k, v)
    if kv_len is None:
        kv_len = q_pos0 + n
    out = _out(out, (n, hq, hd), torch.float32, q.device)
    st = _lib.load().attn_prompt_f16kv(_ptr(q), _QTYPES[q.dtype], _ptr(k), _ptr(v), hq, hkv, hd,
                                       stride, kv_len, q_pos0, n, float(sm_scale), _ptr(out),
                                       _stream())
    _lib.check("attn_prompt_f16kv", st)
    return out


def kv_append(k: torch.Tensor, k_codes: torch.Tensor, k_scales: torch.Tensor, pos0: int,
              v: Optional[torch.Tensor] = None, v_codes: Optional[torch.Tensor] = None,
              v_scales: Optional[torch.Tensor] = None) -> None:
    """Quantise rows k (and v) [n_tokens][Hkv][hd] into the cache at pos0 (in place)."""
    pairs = [("k", k, k_codes, k_scales)]
    if v is not None or v_codes is not None or v_scales is not None:
        if v is None or v_codes is None or v_scales is None:
            raise ValueError("v, v_codes and v_scales go together")
        pairs.append(("v", v, v_codes, v_scales))
    for name, x, c, s in pairs:
        for n2, t in ((name, x), (name + "_codes", c), (name + "_scales", s)):
            if not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{n2} must be a contiguous GPU tensor")
        if x.dtype not in _QTYPES or c.dtype != torch.int8 or s.dtype != torch.float16:
            raise ValueError(f"{name}: rows float32/float16, codes int8, scales float16")
        if x.dim() != 3 or c.dim() != 3 or s.dim() != 3:
            raise ValueError(f"{name}: rows [T][Hkv][hd], codes [Hkv][stride][hd], scales [Hkv][stride][hd/32]")
        if x.shape[1] != c.shape[0] or x.shape[2] != c.shape[2] or \
                s.shape != (c.shape[0], c.shape[1], c.shape[2] // 32):
            raise ValueError(f"{name}: inconsistent shapes")
    if len(pairs) == 2 and (v.shape != k.shape or v.dtype != k.dtype or v_codes.shape != k_codes.shape):
        raise ValueError("k and v must match")
    T, H, hd = k.shape
    nul = 0
    st = _lib.load().attn_kv_append_q8(
        _ptr(k), _ptr(v) if v is not None else nul, _QTYPES[k.dtype], T, H, hd, _ptr(k_codes),
        _ptr(k_scales), _ptr(v_codes) if v is not None else nul,
        _ptr(v_scales) if v is not None else nul, k_codes.shape[1], pos0, _stream())
    _lib.check("attn_kv_append_q8", st)


def head_workspace_bytes(n_rows: int, vocab: int) -> int:
    return int(_lib.load().attn_verify_head_workspace_bytes(n_rows, vocab))


def verify_head_greedy(logits: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                       token: Optional[torch.Tensor] = None,
                       top_prob: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Greedy token (int32) and its probability (fp32) for each row of fp32 logits.

    A workspace passed in must have been zero-filled before its first use; the
    call leaves it ready for the next call.
    """
    if not logits.is_cuda or logits.dtype != torch.float32 or logits.dim() != 2:
        raise ValueError("logits must be a float32 [rows][vocab] GPU tensor")
    if logits.stride(1) != 1:
        raise ValueError("logits rows must be contiguous")
    rows, vocab = logits.shape
    need = head_workspace_bytes(rows, vocab)
    if workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=logits.device)
    token = _out(token, (rows,), torch.int32, logits.device, "token")
    top_prob = _out(top_prob, (rows,), torch.float32, logits.device, "top_prob")
    st = _lib.load().attn_verify_head_greedy(_ptr(logits), rows, vocab, logits.stride(0),
                                             _ptr(token), _ptr(top_prob), _ptr(workspace),
                                             _nbytes(workspace), _stream())
    _lib.check("attn_verify_head_greedy", st)
    return token, top_prob


def selftest_i8_to_f16(device="cuda") -> torch.Tensor:
    out = torch.empty(2 * 65536, dtype=torch.int16, device=device)
    _lib.check("attnq8_selftest_i8_to_f16",
               _lib.load().attnq8_selftest_i8_to_f16(_ptr(out), _stream()))
    return out


STREAM_SINK_WORDS = 1024


def stream_read(buf: torch.Tensor, sink: torch.Tensor | None = None) -> torch.Tensor:
    """Read every byte of a contiguous device tensor (its size a multiple of 16
    bytes) with the library's plain read kernel; returns the 1,024-word sink
    whose XOR is the XOR of the buffer's 32-bit words."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("stream_read needs a contiguous GPU tensor")
    sink = _out(sink, (STREAM_SINK_WORDS,), torch.int32, buf.device, "sink")
    _lib.check("attnq8_stream_read",
               _lib.load().attnq8_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                              _stream()))
    return sink


def last_path() -> str:
    return _lib.last_path()
