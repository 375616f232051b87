"""The KV-append kernel's rounding step, checked on the host against the oracle.

The kernel does not divide per element: it takes k = floor(|x| * r) with r a
reciprocal of the fp16 scale d accurate to about one ulp, adds 1 when
|x| - (k + 1/2) * d >= 0 (computed exactly: (k + 1/2) * d has at most 19
significant bits), clamps to 127 and applies x's sign; a zero scale is taken as
+inf.  This test restates that recipe in numpy (the difference in fp64, which
holds it exactly) with r the correctly rounded reciprocal and one ulp either
side of it, and requires the oracle's codes and scales bit for bit on ordinary,
tiny, huge and fp16 data and on values within three ulps of every rounding
boundary.  It runs no GPU code.
"""

import numpy as np
import pytest

import oracle.quant as Q


def recipe(x, ulps):
    x = x.astype(np.float32)
    b = x.reshape(x.shape[:-1] + (x.shape[-1] // 32, 32))
    with np.errstate(over="ignore"):
        s16 = (np.max(np.abs(b), axis=-1) / np.float32(127)).astype(np.float16)
    d = s16.astype(np.float32)
    dv = np.where(d == 0, np.float32(np.inf), d).astype(np.float32)
    with np.errstate(divide="ignore"):
        r = (np.float32(1) / dv).astype(np.float32)
    for _ in range(abs(ulps)):
        r = np.nextafter(r, np.float32(np.inf) if ulps > 0 else np.float32(0)).astype(np.float32)
    ax = np.abs(b)
    k = np.floor((ax * r[..., None]).astype(np.float32))
    with np.errstate(invalid="ignore"):
        e = ax.astype(np.float64) - (k.astype(np.float64) + 0.5) * dv[..., None].astype(np.float64)
    k = np.minimum(np.where(e >= 0, k + 1, k), 127)
    return np.where(b < 0, -k, k).astype(np.int8).reshape(x.shape), s16


def near_boundaries(rng, n_blocks):
    out = np.empty((n_blocks, 32), np.float32)
    for i in range(n_blocks):
        amax = np.float32(rng.uniform(0.5, 2.0) * 2.0 ** int(rng.integers(-24, 16)))
        d = np.float64(np.float32(np.float16(amax / np.float32(127))))
        v = ((rng.integers(0, 127, 31) + 0.5) * d).astype(np.float32)
        for j, off in enumerate(rng.integers(-3, 4, 31)):
            for _ in range(abs(int(off))):
                v[j] = np.nextafter(v[j], np.float32(np.inf) if off > 0 else np.float32(0))
        out[i, 0] = amax
        out[i, 1:] = v * np.where(rng.random(31) < 0.5, -1, 1)
    return out.reshape(-1, 256)


@pytest.mark.parametrize("ulps", [0, 1, -1])
def test_reciprocal_rounding_matches_oracle(ulps):
    rng = np.random.default_rng(11)
    cases = [
        rng.standard_normal((512, 256)).astype(np.float32),
        (rng.standard_normal((256, 256)) * 10.0 ** rng.uniform(-30, 30, (256, 1))).astype(np.float32),
        np.clip(rng.standard_normal((256, 256)) * 3e4, -65504, 65504).astype(np.float16),
        near_boundaries(rng, 2048),
        np.zeros((2, 256), np.float32),
    ]
    for x in cases:
        c0, s0 = Q.quantize_q8(x)
        c1, s1 = recipe(x, ulps)
        assert np.array_equal(s0.view(np.uint16), s1.view(np.uint16))
        assert np.array_equal(c0, c1)
