"""CPU reference for the block-32 int8 quantisation of new K/V rows (the KV append).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library and never calls it.

The cache format is the pages' Q8 KV ("perf(gfx1100): share Q8 KV scans across
verifier rows", Summary): int8 codes in blocks of 32 consecutive head_dim
elements with one fp16 scale per block, the Q8_0 block of "[Engine] perf(hip):
optimize MTP draft, shared expert, and verify/sampler head kernels on RDNA4"
(Problem and result, item 2; Summary, item 4).  That page checks its GPU
quantiser bit for bit against a CPU reference on zero blocks, exact .5 ties and
ordinary data (Verification & Parity Evidence), so every rounding step below is
fixed, in this order:

1. a block is 32 consecutive elements of one (token, KV head) row;
2. amax = the largest |x| in the block (exact);
3. the scale is amax / 127 divided in fp32 (IEEE, round to nearest even) and
   then rounded to fp16 (round to nearest even; above the fp16 range it becomes
   +inf);
4. each code is x / scale, divided in fp32 against the stored fp16 scale,
   rounded half away from zero and clamped to [-127, 127];
5. a block whose stored scale is 0 (all zero, or amax / 127 below half the
   smallest fp16 subnormal) has every code 0.

The pages leave the tie rule open; half away from zero is the usual Q8_0 rule
(and round(x) in C).  Inputs are fp32 or fp16 values (fp16 widens to fp32
exactly).

Parity pins (tests/test_oracle_quant.py): an exact rational re-derivation of
steps 2-5 with IEEE rounding written from its definition, hand-built tie,
near-tie, double-rounding, subnormal and overflow blocks, and the invariants
|x - scale * code| <= scale / 2, sign symmetry and power-of-two scaling.
"""

from __future__ import annotations

import numpy as np

BLOCK = 32
QMAX = 127


def quantize_q8(x: np.ndarray):
    """fp32 / fp16 [..., hd] -> (codes int8 [..., hd], scales float16 [..., hd/32])."""
    x = np.asarray(x)
    if x.dtype not in (np.float32, np.float16):
        raise TypeError("quantize_q8 takes float32 or float16 values")
    hd = x.shape[-1]
    if hd % BLOCK or hd == 0:
        raise ValueError("the last axis must be a positive multiple of 32")
    nb = hd // BLOCK
    # step 1: blocks of 32 along the last axis
    blocks = x.astype(np.float32).reshape(x.shape[:-1] + (nb, BLOCK))
    # step 2: amax per block
    amax = np.max(np.abs(blocks), axis=-1)
    with np.errstate(over="ignore"):
        # step 3: fp32 divide, then fp16 (round to nearest even, overflow to inf)
        scale = (amax / np.float32(QMAX)).astype(np.float16)
    d = scale.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        # step 4: fp32 divide against the stored scale ...
        y = blocks / d[..., None]
    # ... rounded half away from zero (exact in fp64), then clamped
    yd = y.astype(np.float64)
    r = np.sign(yd) * np.floor(np.abs(yd) + 0.5)
    r = np.clip(r, -QMAX, QMAX)
    # step 5: a zero scale gives zero codes
    r = np.where(d[..., None] == 0, 0.0, r)
    codes = r.astype(np.int8).reshape(x.shape)
    return codes, scale


def kv_append(x: np.ndarray, codes: np.ndarray, scales: np.ndarray, pos0: int):
    """Quantise rows x [T][Hkv][hd] into copies of the cache at positions pos0 .. pos0+T-1.

    codes int8 [Hkv][stride][hd] and scales float16 [Hkv][stride][hd/32] are
    the cache planes; returns new (codes, scales) with only those T positions of
    every KV head replaced.
    """
    x = np.asarray(x)
    T, H, hd = x.shape
    if codes.shape[0] != H or codes.shape[2] != hd or pos0 < 0 or pos0 + T > codes.shape[1]:
        raise ValueError("rows do not fit the cache")
    c, s = quantize_q8(x)  # [T][H][hd], [T][H][hd/32]
    codes = codes.copy()
    scales = scales.copy()
    codes[:, pos0:pos0 + T, :] = np.transpose(c, (1, 0, 2))
    scales[:, pos0:pos0 + T, :] = np.transpose(s, (1, 0, 2))
    return codes, scales
