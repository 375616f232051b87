"""CPU reference for int8-KV GQA attention, the KV append quantiser and the
verify head's greedy token.

TEST INFRASTRUCTURE ONLY: imported by the tests, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the library.
"""

from .core import (  # noqa: F401
    attention,
    attention_values,
    default_scale,
    dequantize,
    kv_head_of,
    merge_partials,
    prompt,
    prompt_f16kv,
    split_partials,
    verify,
    verify_f16kv,
)
from .quant import kv_append, quantize_q8  # noqa: F401
from .head import greedy_head  # noqa: F401
