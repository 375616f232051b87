"""Verify head (greedy token, top probability) on the GPU through the C ABI against the oracle.

Tokens must match exactly.  The top probability is 1 / S with S a sum of
exp(x - max) terms in fp32: each term carries the rounding of x - max times
log2(e) (at most |x - max| * 2^-24 * 1.44 relative for the terms that matter,
|x - max| < 40) and of exp2 (about 2 ulp); the sum of positive terms keeps the
largest relative term error plus one rounding per merge level (< 20 levels).
That is below 4e-6 of S, so 1e-5 relative is the bound used here.
"""

import math

import numpy as np
import pytest
import torch

import head_pins as hp
import oracle
from attention_int8_quantized_amd import ops
from gpu_util import note

pytestmark = pytest.mark.gpu

TOP_RTOL = 1e-5


def _check(x, tok, top, what):
    rt, rp = oracle.greedy_head(x)
    assert np.array_equal(tok.astype(np.int64), rt), f"{what}: tokens {tok} != {rt}"
    for r in range(x.shape[0]):
        if math.isnan(rp[r]):
            assert math.isnan(top[r]), f"{what}: row {r} top {top[r]} != NaN"
        else:
            assert abs(float(top[r]) - rp[r]) <= TOP_RTOL * rp[r], f"{what}: row {r} top {top[r]} vs {rp[r]}"


def _run(x, ws=None):
    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    tok, top = ops.verify_head_greedy(t, workspace=ws)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), top.cpu().numpy()


@pytest.mark.parametrize("rows,vocab", [(1, 248320), (4, 248320), (5, 248320), (8, 248320),
                                        (3, 106299), (2, 1), (3, 7), (1, 2049), (64, 4096),
                                        (257, 1000), (1024, 3000)])  # one block per row
def test_head_matches_oracle(rows, vocab):
    note(f"verify head rows={rows} vocab={vocab}")
    rng = np.random.default_rng(rows * 1000 + vocab % 997)
    x = (rng.standard_normal((rows, vocab)) * 3).astype(np.float32)
    tok, top = _run(x)
    note(f"  path: {ops.last_path()}")
    _check(x, tok, top, f"rows={rows} vocab={vocab}")


def test_head_special_rows():
    """Ties across blocks, NaN beside the maximum, -inf masks, rows with nothing valid."""
    V = 248320
    rng = np.random.default_rng(41)
    x = (rng.standard_normal((8, V)) * 2).astype(np.float32)
    x[0, [200000, 5000, 123456]] = 50.0            # tie across blocks: 5000 wins
    x[1, :] = -np.inf
    x[1, [70000, 9]] = 1.0                          # masked row, two survivors
    x[2, :] = np.nan                                # nothing valid: -1, NaN
    x[3, :] = -np.inf                               # all masked: 0, NaN
    x[4, ::3] = np.nan
    x[4, 3000] = 40.0
    x[4, 2999] = np.nan                             # NaN beside the maximum
    x[5, :] = np.where(rng.random(V) < 0.5, np.nan, -np.inf).astype(np.float32)
    x[6, :] = 7.25                                  # constant: 0, 1/V
    x[7, V - 1] = 30.0                              # maximum in the ragged last chunk
    tok, top = _run(x)
    _check(x, tok, top, "special rows")
    assert list(tok[:4]) == [5000, 9, -1, 0] and tok[7] == V - 1
    # and the pins' own special rows, scattered over a long row
    sp = hp.special_rows()
    y = np.full((sp.shape[0], 50000), -np.inf, dtype=np.float32)
    y[:, 41000:41008] = sp
    y[:, 3:11] = sp                                 # the same values earlier: earlier indices win
    tok2, top2 = _run(y)
    _check(y, tok2, top2, "scattered pin rows")


def test_head_workspace_reuse_and_determinism():
    note("verify head: one zeroed workspace across calls of 8, 1, 5 rows; bitwise repeat")
    V = 248320
    ws = torch.zeros(ops.head_workspace_bytes(64, V), dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(43)
    first = None
    for rows in (8, 1, 5, 8):
        x = (rng.standard_normal((rows, V)) * 3).astype(np.float32) if rows != 8 or first is None else first[0]
        tok, top = _run(x, ws)
        _check(x, tok, top, f"reuse rows={rows}")
        if rows == 8:
            if first is None:
                first = (x, tok, top)
            else:
                assert np.array_equal(tok, first[1])
                assert np.array_equal(top.view(np.uint32), first[2].view(np.uint32))


@pytest.mark.parametrize("V,S", [(10000, 10240), (10001, 10003), (248320, 248321)])
def test_head_row_stride(V, S):
    """Rows at a stride (16-byte aligned rows and rows that are not: the
    kernel's vector and scalar loads), padding beyond each row ignored."""
    rng = np.random.default_rng(44 + V)
    buf = (rng.standard_normal((3, S)) * 2).astype(np.float32)
    buf[:, V:] = 1e9  # padding beyond the row must be ignored
    t = torch.from_numpy(buf).cuda()[:, :V]
    tok, top = ops.verify_head_greedy(t)
    torch.cuda.synchronize()
    _check(buf[:, :V].copy(), tok.cpu().numpy(), top.cpu().numpy(), "strided rows")
