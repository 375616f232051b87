"""Checks that pin the attention oracle to facts outside itself.

Each ``check_*`` takes the functions under test (so that the same checks can be
run against deliberately broken copies of the oracle) and raises
AssertionError on failure.  The facts come from the definition of attention
over a block-32 int8 cache and from closed forms, never from the oracle's own
code:

* brute force (pure-Python loops) on tiny inputs;
* torch's CPU fp64 scaled_dot_product_attention with an explicit mask;
* closed forms: equal logits give the mean of the visible values; a single
  visible key returns its value; two keys give a logistic mix whose logit
  difference is computed by hand; a dominant logit selects one value;
* invariants: convex hull, power-of-two scaling, causality, GQA grouping;
* per-block scale indexing through values chosen per block.
"""

from __future__ import annotations

import math

import numpy as np

import bruteforce

BLOCK = 32


def _rng(seed):
    return np.random.default_rng(seed)


def random_case(seed, n, hq, hkv, hd, T, qdtype=np.float32):
    """Small random cache + queries (codes uniform in [-127,127], scales ~ U(0.005,0.05))."""
    r = _rng(seed)
    q = r.standard_normal((n, hq, hd)).astype(qdtype)
    kc = r.integers(-127, 128, size=(hkv, T, hd), dtype=np.int64).astype(np.int8)
    vc = r.integers(-127, 128, size=(hkv, T, hd), dtype=np.int64).astype(np.int8)
    ks = r.uniform(0.005, 0.05, size=(hkv, T, hd // BLOCK)).astype(np.float16)
    vs = r.uniform(0.005, 0.05, size=(hkv, T, hd // BLOCK)).astype(np.float16)
    return q, kc, ks, vc, vs


def deq(codes, scales):
    """Test-side dequantisation written with explicit Python arithmetic."""
    codes = np.asarray(codes)
    out = np.zeros(codes.shape, dtype=np.float64)
    it = np.ndindex(codes.shape[:-1])
    for idx in it:
        for j in range(codes.shape[-1]):
            out[idx + (j,)] = float(scales[idx + (j // BLOCK,)]) * float(codes[idx + (j,)])
    return out


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ----------------------------------------------------------------------------
# brute force and library cross-checks
# ----------------------------------------------------------------------------

SMALL_CASES = [
    # (seed, n, hq, hkv, hd, T, positions)
    (1, 3, 2, 1, 32, 9, [5, 6, 8]),
    (2, 2, 4, 2, 64, 7, [0, 6]),
    (3, 4, 4, 1, 32, 12, [8, 9, 10, 11]),
    (4, 1, 8, 2, 64, 40, [39]),
    (5, 2, 3, 3, 32, 5, [2, 4]),
]


def check_bruteforce(attn, tol=1e-12):
    for seed, n, hq, hkv, hd, T, pos in SMALL_CASES:
        q, kc, ks, vc, vs = random_case(seed, n, hq, hkv, hd, T)
        got = attn(q, pos, kc, ks, vc, vs)
        ref = bruteforce.attention(q.tolist(), pos, kc.tolist(), ks.astype(np.float64).tolist(),
                                   vc.tolist(), vs.astype(np.float64).tolist())
        e = rel_err(got, ref)
        assert e <= tol, f"brute force mismatch seed={seed}: {e}"


def check_torch_sdpa(attn, tol=1e-12):
    import torch
    import torch.nn.functional as F

    for seed, n, hq, hkv, hd, T, pos in SMALL_CASES + [(6, 5, 6, 2, 128, 70, [60, 61, 62, 63, 64])]:
        q, kc, ks, vc, vs = random_case(seed, n, hq, hkv, hd, T)
        got = attn(q, pos, kc, ks, vc, vs)
        kh = torch.from_numpy(deq(kc, ks))  # [hkv][T][hd]
        vh = torch.from_numpy(deq(vc, vs))
        g = hq // hkv
        kh = kh.repeat_interleave(g, dim=0)  # [hq][T][hd]
        vh = vh.repeat_interleave(g, dim=0)
        qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2).contiguous()  # [hq][n][hd]
        mask = torch.arange(T)[None, :] <= torch.tensor(pos)[:, None]  # [n][T]
        ref = F.scaled_dot_product_attention(qt, kh, vh, attn_mask=mask[None])
        ref = ref.permute(1, 0, 2).numpy()
        e = rel_err(got, ref)
        assert e <= tol, f"sdpa mismatch seed={seed}: {e}"


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------


def check_constant_keys(attn):
    """All keys equal -> equal logits -> the plain mean of the visible values."""
    q, kc, ks, vc, vs = random_case(11, 3, 4, 2, 64, 20)
    kc[:] = 17
    ks[:] = np.float16(0.03)
    pos = [4, 11, 19]
    got = attn(q, pos, kc, ks, vc, vs)
    vh = deq(vc, vs)
    for r, p in enumerate(pos):
        for h in range(4):
            expect = vh[h // 2, : p + 1].mean(axis=0)
            assert rel_err(got[r, h], expect) <= 1e-13, "constant keys"


def check_single_key(attn):
    """A row at position 0 sees one key and returns its value exactly."""
    q, kc, ks, vc, vs = random_case(12, 1, 4, 2, 64, 3)
    got = attn(q, [0], kc, ks, vc, vs)
    vh = deq(vc, vs)
    for h in range(4):
        assert np.array_equal(got[0, h], vh[h // 2, 0]), "single visible key"


def check_visible_count(attn):
    """Equal logits and V_t = t*d give pos*d/2: pins that row p sees p+1 keys."""
    hd, T = 32, 100
    kc = np.full((1, T, hd), 3, dtype=np.int8)
    ks = np.full((1, T, 1), 0.5, dtype=np.float16)
    vc = np.repeat(np.arange(T, dtype=np.int8)[None, :, None], hd, axis=2)
    d = 0.25
    vs = np.full((1, T, 1), d, dtype=np.float16)
    pos = [0, 1, 2, 37, 98, 99]
    q = _rng(13).standard_normal((len(pos), 2, hd)).astype(np.float32)
    got = attn(q, pos, kc, ks, vc, vs)
    for r, p in enumerate(pos):
        assert np.allclose(got[r], p * d / 2.0, rtol=0, atol=1e-12), f"visible count at {p}"


def check_two_key_logistic(attn):
    """Two keys: out = (V0 + e^D V1)/(1 + e^D) with D computed by hand.

    hd = 64, q = 1.5 e_5, key 0 all zero, key 1 has code 40 at dim 5 with
    scale 0.125: D = 1.5 * 40 * 0.125 / sqrt(64) = 0.9375.
    """
    hd = 64
    q = np.zeros((1, 1, hd), dtype=np.float32)
    q[0, 0, 5] = 1.5
    kc = np.zeros((1, 2, hd), dtype=np.int8)
    kc[0, 1, 5] = 40
    ks = np.full((1, 2, 2), 0.125, dtype=np.float16)
    vc = np.zeros((1, 2, hd), dtype=np.int8)
    vc[0, 0, :] = 10
    vc[0, 1, :] = -20
    vs = np.full((1, 2, 2), 0.5, dtype=np.float16)
    got = attn(q, [1], kc, ks, vc, vs)
    D = 1.5 * 40 * 0.125 / 8.0
    expect = (5.0 + math.exp(D) * -10.0) / (1.0 + math.exp(D))
    assert abs(got[0, 0, 0] - expect) <= 1e-14, "two-key logistic"
    assert np.allclose(got[0, 0], expect, rtol=0, atol=1e-14)


def check_block_scale_index(attn):
    """Per-block scales are indexed by j // 32, for both K and V.

    V: one visible key with codes 1 and block scale 2^-b returns 2^-b at dim j
    of block b.  K: key 1 has code 1 at dim j only, block scales 2^b; q = e_j,
    key 0 zero, V0 = 0, V1 = 1, so out = sigmoid(2^(j//32) / sqrt(hd)).
    """
    hd = 128
    q = np.ones((1, 1, hd), dtype=np.float32)
    kc = np.zeros((1, 1, hd), dtype=np.int8)
    ks = np.zeros((1, 1, 4), dtype=np.float16)
    vc = np.ones((1, 1, hd), dtype=np.int8)
    vs = np.array([[[1.0, 0.5, 0.25, 0.125]]], dtype=np.float16)
    got = attn(q, [0], kc, ks, vc, vs)
    for j in range(hd):
        assert got[0, 0, j] == 2.0 ** -(j // 32), "V block scale index"
    for j in (0, 31, 32, 70, 127):
        q = np.zeros((1, 1, hd), dtype=np.float32)
        q[0, 0, j] = 1.0
        kc = np.zeros((1, 2, hd), dtype=np.int8)
        kc[0, 1, j] = 1
        ks = np.array([[[0.0] * 4, [1.0, 2.0, 4.0, 8.0]]], dtype=np.float16)
        vc = np.zeros((1, 2, hd), dtype=np.int8)
        vc[0, 1, :] = 1
        vs = np.ones((1, 2, 4), dtype=np.float16)
        got = attn(q, [1], kc, ks, vc, vs)
        D = 2.0 ** (j // 32) / math.sqrt(hd)
        expect = math.exp(D) / (1.0 + math.exp(D))
        assert abs(got[0, 0, 0] - expect) <= 1e-14, f"K block scale index at {j}"


def check_one_hot(attn):
    """A dominant logit selects its value to within (n-1) e^-Delta max|V|."""
    hd, T = 64, 50
    r = _rng(14)
    kc = np.zeros((1, T, hd), dtype=np.int8)
    ks = np.full((1, T, 2), 0.01, dtype=np.float16)
    tstar = 23
    kc[0, tstar, 0] = 127
    ks[0, tstar, 0] = np.float16(2.0)
    vc = r.integers(-127, 128, size=(1, T, hd)).astype(np.int8)
    vs = np.full((1, T, 2), 0.02, dtype=np.float16)
    q = np.zeros((1, 1, hd), dtype=np.float32)
    q[0, 0, 0] = 1.0
    got = attn(q, [T - 1], kc, ks, vc, vs)
    vh = deq(vc, vs)
    delta = 127 * 2.0 / 8.0
    bound = (T - 1) * math.exp(-delta) * np.abs(vh).max() * 2
    assert np.max(np.abs(got[0, 0] - vh[0, tstar])) <= bound, "one-hot"


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------


def check_convex_hull(attn):
    q, kc, ks, vc, vs = random_case(15, 4, 4, 2, 64, 30)
    pos = [3, 10, 20, 29]
    got = attn(q, pos, kc, ks, vc, vs)
    vh = deq(vc, vs)
    for r, p in enumerate(pos):
        for h in range(4):
            lo = vh[h // 2, : p + 1].min(axis=0)
            hi = vh[h // 2, : p + 1].max(axis=0)
            assert np.all(got[r, h] >= lo - 1e-12) and np.all(got[r, h] <= hi + 1e-12), "hull"


def check_all_v_equal(attn):
    q, kc, ks, vc, vs = random_case(16, 2, 2, 1, 64, 25)
    vc[:] = -77
    vs[:] = np.float16(0.0625)
    got = attn(q, [10, 24], kc, ks, vc, vs)
    assert np.allclose(got, -77 * 0.0625, rtol=0, atol=1e-13), "all V equal"


def check_pow2_v_scaling(attn):
    q, kc, ks, vc, vs = random_case(17, 3, 4, 1, 64, 20)
    pos = [5, 12, 19]
    a = attn(q, pos, kc, ks, vc, vs)
    b = attn(q, pos, kc, ks, vc, (vs.astype(np.float32) * 2).astype(np.float16))
    assert np.array_equal(b, 2 * a), "power-of-two V scaling"


def check_causality(attn):
    q, kc, ks, vc, vs = random_case(18, 3, 4, 2, 64, 30)
    pos = [7, 15, 29]
    a = attn(q, pos, kc, ks, vc, vs)
    kc2, vc2, ks2 = kc.copy(), vc.copy(), ks.copy()
    kc2[:, 8:] = -kc2[:, 8:]
    vc2[:, 8:] = 99
    ks2[:, 8:] = np.float16(3.0)
    b = attn(q, pos, kc2, ks2, vc2, vs)
    assert np.array_equal(a[0], b[0]), "future keys changed an earlier row"
    assert not np.array_equal(a[1], b[1])


def check_gqa_grouping(attn):
    """Q head h reads KV head h // (Hq/Hkv): KV head g carries values g+1."""
    hq, hkv, hd, T = 8, 4, 32, 6
    q = _rng(19).standard_normal((2, hq, hd)).astype(np.float32)
    kc = _rng(20).integers(-127, 128, size=(hkv, T, hd)).astype(np.int8)
    ks = np.full((hkv, T, 1), 0.01, dtype=np.float16)
    vc = np.zeros((hkv, T, hd), dtype=np.int8)
    for g in range(hkv):
        vc[g] = g + 1
    vs = np.ones((hkv, T, 1), dtype=np.float16)
    got = attn(q, [2, 5], kc, ks, vc, vs)
    for h in range(hq):
        assert np.allclose(got[:, h], h // (hq // hkv) + 1, rtol=0, atol=1e-13), f"head {h}"
    # heads of one group with identical q give identical outputs
    q2 = q.copy()
    q2[:, 1] = q2[:, 0]
    got = attn(q2, [2, 5], kc, ks, _rng(21).integers(-9, 9, size=(hkv, T, hd)).astype(np.int8), vs)
    assert np.array_equal(got[:, 0], got[:, 1])


ATTENTION_CHECKS = [
    check_bruteforce,
    check_torch_sdpa,
    check_constant_keys,
    check_single_key,
    check_visible_count,
    check_two_key_logistic,
    check_block_scale_index,
    check_one_hot,
    check_convex_hull,
    check_all_v_equal,
    check_pow2_v_scaling,
    check_causality,
    check_gqa_grouping,
]


# ----------------------------------------------------------------------------
# reducer (split partials and their merge)
# ----------------------------------------------------------------------------


def check_merge_single(merge):
    r = _rng(30)
    o = r.standard_normal((1, 3, 16))
    l = r.uniform(1, 5, size=(1, 3))
    m = r.standard_normal((1, 3))
    assert np.allclose(merge(m, l, o), o[0] / l[0][:, None], rtol=1e-15, atol=0)


def check_merge_equal_m(merge):
    r = _rng(31)
    o = r.standard_normal((2, 4, 8))
    l = r.uniform(1, 5, size=(2, 4))
    m = np.full((2, 4), 0.75)
    expect = (o[0] + o[1]) / (l[0] + l[1])[:, None]
    assert np.allclose(merge(m, l, o), expect, rtol=1e-14, atol=0)


def check_merge_base2(merge):
    """m differing by 1 weighs the second split by 2 (base-2 convention)."""
    o = np.array([[[1.0, 2.0]], [[3.0, -1.0]]])
    l = np.array([[2.0], [1.0]])
    m = np.array([[0.0], [1.0]])
    expect = (o[0, 0] + 2 * o[1, 0]) / (l[0, 0] + 2 * l[1, 0])
    assert np.allclose(merge(m, l, o)[0], expect, rtol=1e-15, atol=0)


def check_merge_empty(merge):
    r = _rng(32)
    o = r.standard_normal((3, 2, 8))
    l = r.uniform(1, 5, size=(3, 2))
    m = r.standard_normal((3, 2))
    o[1] = 0
    l[1] = 0
    m[1] = -np.inf
    keep = [0, 2]
    assert np.allclose(merge(m, l, o), merge(m[keep], l[keep], o[keep]), rtol=1e-15, atol=0)


def check_split_invariance(attn, split, merge):
    q, kc, ks, vc, vs = random_case(33, 4, 4, 2, 64, 40)
    pos = [30, 33, 36, 39]
    whole = attn(q, pos, kc, ks, vc, vs)
    for bounds in ([(0, 40)], [(0, 13), (13, 31), (31, 40)], [(0, 5), (5, 32), (32, 35), (35, 40)]):
        m, l, o = split(q, pos, kc, ks, vc, vs, bounds)
        got = merge(m, l, o)
        assert rel_err(got, whole) <= 1e-13, f"split invariance {bounds}"
