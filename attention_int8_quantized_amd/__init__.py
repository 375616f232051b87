"""attnq8: int8 block-32 KV-cache GQA attention for AMD Instinct MI355X (gfx950).

The compute path is the HIP library libattnq8.so behind the C ABI in
include/attnq8.h; this package is its thin Python binding (``ops``, which
needs torch) and build step (``build``).
"""

from . import _lib  # noqa: F401
