"""ctypes loader for libattnq8.so (the C ABI of include/attnq8.h).

The library must have been built in-tree (``python -m
attention_int8_quantized_amd.build`` or ``__graft_entry__.build()``); loading
fails loudly otherwise -- there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
import re

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libattnq8.so")
HEADER = os.path.join(os.path.dirname(PKG_DIR), "include", "attnq8.h")

OK = 0
EINVAL = -1
EUNSUPPORTED = -2
EALIGN = -3
EWORKSPACE = -4
EHIP = -5

F32 = 0
F16 = 1

STATIC_SCRATCH_BYTES = 32 << 20  # ATTNQ8_STATIC_SCRATCH_BYTES

_c_int = ctypes.c_int
_c_size = ctypes.c_size_t
_c_float = ctypes.c_float
_vp = ctypes.c_void_p

_SIGNATURES = {
    "attn_verify_q8_splits": (_c_int, [_c_int] * 6),
    "attn_verify_q8_workspace_bytes": (_c_size, [_c_int] * 4),
    "attn_verify_q8": (
        _c_int,
        [_vp, _c_int, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
         _c_int, _vp, _c_size, _c_float, _vp],
    ),
    "attn_reduce_partials": (_c_int, [_vp, _c_size, _c_int, _c_int, _c_int, _c_int, _vp, _vp]),
    "attn_verify_q8_static": (
        _c_int,
        [_vp, _c_int, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
         _c_int, _c_float, _vp, _vp],
    ),
    "attn_prompt_q8": (
        _c_int,
        [_vp, _c_int, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
         _c_float, _vp, _vp],
    ),
    "attn_verify_f16kv": (
        _c_int,
        [_vp, _c_int, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
         _vp, _c_size, _c_float, _vp],
    ),
    "attn_prompt_f16kv": (
        _c_int,
        [_vp, _c_int, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float,
         _vp, _vp],
    ),
    "attn_kv_append_q8": (
        _c_int,
        [_vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _c_int, _c_int, _vp],
    ),
    "attn_verify_head_workspace_bytes": (_c_size, [_c_int, _c_int]),
    "attn_verify_head_greedy": (
        _c_int, [_vp, _c_int, _c_int, ctypes.c_longlong, _vp, _vp, _vp, _c_size, _vp]),
    "attnq8_selftest_i8_to_f16": (_c_int, [_vp, _vp]),
    "attnq8_stream_read": (_c_int, [_vp, _c_size, _vp, _vp]),
    "attnq8_status_string": (ctypes.c_char_p, [_c_int]),
    "attnq8_last_path": (ctypes.c_char_p, []),
}

_lib = None


class Attnq8Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")


def header_functions():
    """Names of the functions include/attnq8.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn\w+)\s*\(", text)))


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m attention_int8_quantized_amd.build`"
        )
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().attnq8_status_string(int(status)).decode()


def last_path() -> str:
    return load().attnq8_last_path().decode()


def check(fn: str, status: int) -> None:
    if status != OK:
        raise Attnq8Error(fn, status)
