"""Pure-Python brute-force attention over an int8 block-32 KV cache.

An independent restatement of the definition the oracle follows, written with
scalar loops and ``math.exp`` only, for tiny inputs.  It pins the numpy oracle:
neither calls the other.
"""

from __future__ import annotations

import math


def _value(code, scale_bits_as_float):
    return float(scale_bits_as_float) * float(code)


def attention(q, positions, k_codes, k_scales, v_codes, v_scales, sm_scale=None):
    """q [n][Hq][hd] (any numeric), positions [n]; KV as in the cache layout.

    Returns nested Python lists [n][Hq][hd] of floats.
    """
    n = len(q)
    hq = len(q[0])
    hd = len(q[0][0])
    hkv = len(k_codes)
    group = hq // hkv
    scale = 1.0 / math.sqrt(hd) if sm_scale is None else float(sm_scale)
    out = []
    for r in range(n):
        pos = int(positions[r])
        row_out = []
        for h in range(hq):
            g = h // group
            logits = []
            for t in range(pos + 1):
                acc = 0.0
                for j in range(hd):
                    kval = _value(k_codes[g][t][j], k_scales[g][t][j // 32])
                    acc += float(q[r][h][j]) * kval
                logits.append(acc * scale)
            top = max(logits)
            weights = [math.exp(s - top) for s in logits]
            total = sum(weights)
            vec = []
            for j in range(hd):
                num = 0.0
                for t in range(pos + 1):
                    num += weights[t] * _value(v_codes[g][t][j], v_scales[g][t][j // 32])
                vec.append(num / total)
            row_out.append(vec)
        out.append(row_out)
    return out
