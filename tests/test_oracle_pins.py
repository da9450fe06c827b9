"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, never against a retyped copy of the oracle's own formulas.

Each test names the mistake it is there to catch.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import csa2_inputs as ci

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")


def pages():
    with open(GOLDEN) as f:
        return json.load(f)


def e4m3_table_torch():
    """Independent E4M3 (OCP FN) decode: PyTorch's float8_e4m3fn."""
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


# E2M1 magnitudes as the OCP microscaling spec lists them, codes 0..7.
E2M1_SPEC = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


# ------------------------------------------------------------------ formats
def test_e2m1_table_matches_spec():
    got = [oracle.e2m1_value(c) for c in range(16)]
    assert got[:8] == E2M1_SPEC
    assert got[8:] == [-v for v in E2M1_SPEC]
    assert math.copysign(1.0, got[8]) == -1.0  # code 8 is -0


def test_e4m3_table_matches_torch():
    ref = e4m3_table_torch()
    for c in range(256):
        v = oracle.e4m3_value(c)
        if math.isnan(ref[c]):
            assert math.isnan(v), c
        else:
            assert v == ref[c], (c, v, ref[c])
    # spot values of the format
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0x38) == 1.0


def test_mxfp4_range_is_pages_number():
    g = pages()["mxfp4_range"]
    top = oracle.e2m1_value(7) * oracle.e4m3_value(0x7E)
    assert top == g["value"] == g["factors"][0] * g["factors"][1]
    # the encoder saturates there: a block far above the range decodes to +-2688
    x = np.zeros((1, 16), np.float32)
    x[0, 0], x[0, 1] = 1e6, -1e6
    c, s = oracle.mxfp4_encode(x)
    d = oracle.mxfp4_decode(c, s)
    assert d[0, 0] == 2688.0 and d[0, 1] == -2688.0 and s[0, 0] == 0x7E


# -------------------------------------------------- MXFP4 encode by brute force
E4_VALS = None


def _nearest_even(target: Fraction, grid):
    """Brute-force round-to-nearest over an ascending grid of (code, value);
    ties go to the even code; above the top value: saturate."""
    best = None
    for code, val in grid:
        d = abs(Fraction(val) - target)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return best[1]


def _brute_encode_block(x16):
    global E4_VALS
    if E4_VALS is None:
        t = e4m3_table_torch()
        E4_VALS = [(c, float(t[c])) for c in range(127)]  # non-negative finite codes
    amax = max(abs(Fraction(float(v))) for v in x16)
    sc = _nearest_even(amax / 6, E4_VALS)
    s = Fraction(E4_VALS[sc][1])
    nibs = []
    for v in x16:
        if s == 0:
            nibs.append(0)
            continue
        mag = _nearest_even(abs(Fraction(float(v))) / s, list(enumerate(E2M1_SPEC)))
        nibs.append(mag | (8 if (v < 0 and mag != 0) else 0))
    return sc, nibs


def _unpack(codes_row):
    out = []
    for b in codes_row:
        out.append(int(b) & 15)
        out.append(int(b) >> 4)
    return out


@pytest.mark.parametrize("scale", [1.0, 1e-3, 0.37, 22.6, 300.0])
def test_mxfp4_encode_equals_bruteforce_nearest(scale):
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((24, 64)) * scale).astype(np.float32)
    # plant exact ties and grid points
    x[0, :16] = np.float32(1.0) * np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, 6,
                                            -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5, -6],
                                           np.float32)
    x[1, :16] = 0.0
    x[1, 3] = -0.0
    codes, scales = oracle.mxfp4_encode(x)
    for r in range(x.shape[0]):
        nib = _unpack(codes[r])
        for b in range(x.shape[1] // 16):
            sc, ref = _brute_encode_block(x[r, 16 * b:16 * b + 16])
            assert scales[r, b] == sc, (r, b)
            assert nib[16 * b:16 * b + 16] == ref, (r, b)


def test_mxfp4_scale_ties_to_even():
    # amax / 6 exactly halfway between two E4M3 values -> even code.
    # 1.0625 is halfway between 1.0 (0x38) and 1.125 (0x39): picks 0x38.
    # 1.1875 is halfway between 1.125 (0x39) and 1.25 (0x3A): picks 0x3A.
    for mid, want in [(1.0625, 0x38), (1.1875, 0x3A)]:
        x = np.zeros((1, 16), np.float32)
        x[0, 0] = 6 * mid
        _, s = oracle.mxfp4_encode(x)
        assert s[0, 0] == want


def test_mxfp4_nibble_order_worked_example():
    # amax 6 -> scale 1.0 (0x38).  6 -> 0x7, -6 -> 0xF, 0.5 -> 0x1, 3 -> 0x5.
    # Channel 2j sits in the low nibble of byte j.
    x = np.zeros((1, 16), np.float32)
    x[0, :4] = [6.0, -6.0, 0.5, 3.0]
    c, s = oracle.mxfp4_encode(x)
    assert s[0, 0] == 0x38
    assert c[0, 0] == 0xF7 and c[0, 1] == 0x51
    assert all(v == 0 for v in c[0, 2:])


def test_mxfp4_canonical_roundtrip_is_exact():
    rng = np.random.default_rng(3)
    t = e4m3_table_torch()
    rows = []
    for _ in range(200):
        sc = int(rng.integers(1, 127))
        mags = rng.integers(0, 8, 16)
        mags[rng.integers(0, 16)] = 7  # largest |code| is 6 -> the block is canonical
        sign = rng.integers(0, 2, 16)
        vals = [(-1.0 if sg and m else 1.0) * E2M1_SPEC[m] * t[sc] for m, sg in zip(mags, sign)]
        rows.append(vals)
    x = np.array(rows, np.float64).astype(np.float32)
    assert np.array_equal(x.astype(np.float64), np.array(rows))  # exactly representable
    c, s = oracle.mxfp4_encode(x)
    d = oracle.mxfp4_decode(c, s)
    assert np.array_equal(d, x.astype(np.float64))
    c2, s2 = oracle.mxfp4_encode(d.astype(np.float32))
    assert np.array_equal(c, c2) and np.array_equal(s, s2)


def test_mxfp4_norm_bound_cases():
    g = pages()["norm_bound"]
    bound = math.sqrt(g["channels"])
    assert round(bound, 1) == g["value"]
    D = g["channels"]
    # one-hot at the bound: scale RNE(22.627/6 = 3.771) = 3.75, code 6 -> 22.5
    x = np.zeros((1, D), np.float32)
    x[0, 100] = np.float32(bound)
    c, s = oracle.mxfp4_encode(x)
    assert oracle.e4m3_value(int(s[0, 100 // 16])) == 3.75
    d = oracle.mxfp4_decode(c, s)
    assert d[0, 100] == 22.5
    assert abs(d[0, 100] - bound) < 0.13
    # a flat +-1 vector: scale RNE(1/6) = 0.171875, every element -> code 6 -> 1.03125
    x = np.where(np.arange(D) % 3 == 0, -1.0, 1.0).astype(np.float32)[None]
    c, s = oracle.mxfp4_encode(x)
    assert all(oracle.e4m3_value(int(v)) == 0.171875 for v in s[0])
    d = oracle.mxfp4_decode(c, s)
    assert np.array_equal(np.abs(d), np.full((1, D), 1.03125))
    assert np.array_equal(np.sign(d), np.sign(x))
    # the largest scale any |v| <= bound can need is far inside the format (headroom)
    worst = max(oracle.e4m3_value(int(v)) for v in s[0])
    _, s_one = oracle.mxfp4_encode(np.full((1, 16), bound, np.float32))
    assert oracle.e4m3_value(int(s_one[0, 0])) <= 3.75 < 448 / 100


def test_mxfp4_zero_block_and_negative_zero():
    x = np.zeros((2, 32), np.float32)
    x[1, :] = -0.0
    x[1, 20] = -1e-30  # scale underflows to 0 -> whole block zero
    c, s = oracle.mxfp4_encode(x)
    assert not c.any() and not s.any()


# ------------------------------------------------------------------ score
def test_score_one_head_one_channel():
    # w * max(q*k, 0)
    assert oracle.score_one([[2.0]], [0.5], [3.0]) == np.float32(3.0)
    assert oracle.score_one([[2.0]], [0.5], [-3.0]) == np.float32(0.0)
    assert oracle.score_one([[-2.0]], [0.25], [-3.0]) == np.float32(1.5)


def test_score_exactly_summable_regime():
    # q, k multiples of 2^-3 in [-4, 4]; w multiples of 2^-4 in [0, 1):
    # every partial sum is exact in float32, so the chain equals the exact value.
    rng = np.random.default_rng(11)
    H_I, d_I, n = 8, 128, 300
    q = np.clip(np.round(rng.standard_normal((H_I, d_I)) * 8) / 8, -4, 4).astype(np.float32)
    k = np.clip(np.round(rng.standard_normal((n, d_I)) * 8) / 8, -4, 4).astype(np.float32)
    w = (rng.integers(0, 16, H_I) / 16).astype(np.float32)
    exact = np.maximum(k.astype(np.float64) @ q.astype(np.float64).T, 0.0) @ w.astype(np.float64)
    got = oracle.full_scores(q, w, k, n, n)
    assert np.array_equal(got.astype(np.float64), exact)


def test_score_chain_runs_forward_over_channels():
    # k = [2^24, 1, -2^24], q = 1: forward chain gives 2^24 + 1 -> 2^24 (tie to
    # even), then 0, so the score is 0; a reversed or pairwise sum would give 1.
    q = np.ones((1, 3), np.float32)
    k = np.array([2.0 ** 24, 1.0, -(2.0 ** 24)], np.float32)
    assert oracle.score_one(q, [1.0], k) == np.float32(0.0)
    assert oracle.score_one(q, [1.0], k[::-1].copy()) == np.float32(1.0)


def test_score_uses_fused_multiply_add():
    # a = 1 + 2^-12: a*a = 1 + 2^-11 + 2^-24 needs 25 bits, so RN(a*a) = 1 + 2^-11
    # (tie to even).  A fused step keeps the 2^-24 that a separate multiply loses.
    a = np.float32(1 + 2.0 ** -12)
    # d-chain: d = RN(-a*a) = -(1 + 2^-11); d = fma(a, a, d) = +2^-24 (mul+add: 0)
    q = np.array([[-a, a]], np.float32)
    k = np.array([a, a], np.float32)
    assert oracle.score_one(q, [1.0], k) == np.float32(2.0 ** -24)
    # w-chain: r = [a, a]; s = RN(a*a); s = fma(-a, a, s) = -2^-24 (mul+add: 0)
    q2 = np.array([[1.0], [1.0]], np.float32)
    k2 = np.array([a], np.float32)
    w2 = np.array([a, -a], np.float32)
    assert oracle.score_one(q2, w2, k2) == np.float32(-(2.0 ** -24))
    # heads are summed in order h = 0, 1: swapping w gives RN(-a*a) then +a*a
    assert oracle.score_one(q2, w2[::-1].copy(), k2) == np.float32(2.0 ** -24)


def test_score_transposition_and_head_weights():
    # non-square shapes catch q[h][c] vs q[c][h] and w indexing mistakes
    rng = np.random.default_rng(5)
    q = np.round(rng.standard_normal((3, 5)) * 4).astype(np.float32) / 4
    w = np.array([0.25, 0.5, 1.0], np.float32)
    k = np.round(rng.standard_normal((7, 5)) * 4).astype(np.float32) / 4
    ref = np.maximum(k.astype(np.float64) @ q.T.astype(np.float64), 0) @ w.astype(np.float64)
    got = oracle.full_scores(q, w, k, 7, 9)
    assert np.array_equal(got[:7].astype(np.float64), ref)
    assert np.all(np.isneginf(got[7:]))


# ------------------------------------------------------------------ top-k
def _brute_topk(vals, k):
    items = [(-float(v), i) for i, v in enumerate(vals) if not np.isneginf(v)]
    items.sort()
    sel = sorted(i for _, i in items[:k])
    return sel + [-1] * (k - len(sel))


def test_topk_exhaustive_tiny():
    for n in range(0, 7):
        for pattern in itertools.product([0.0, 1.0, 2.0, -np.inf], repeat=n):
            vals = np.array(pattern, np.float32)
            for k in range(1, n + 2):
                assert list(oracle.topk(vals, k)) == _brute_topk(vals, k), (pattern, k)


def test_topk_random_and_special_cases():
    rng = np.random.default_rng(1)
    for n, k in [(100, 10), (1000, 64), (5000, 2048), (333, 333), (50, 80)]:
        vals = rng.integers(0, 20, n).astype(np.float32)  # heavy ties
        assert list(oracle.topk(vals, k)) == _brute_topk(vals, k)
    vals = np.full(100, 3.0, np.float32)
    assert list(oracle.topk(vals, 10)) == list(range(10))  # all equal -> lowest positions
    vals = np.array([1, 5, 2, 5, 0], np.float32)
    assert list(oracle.topk(vals, 1)) == [1]  # argmax, lowest index
    assert list(oracle.topk(vals, 9)) == [0, 1, 2, 3, 4, -1, -1, -1, -1]  # k >= n: everything
    z = np.array([-0.0, 0.0, -0.0], np.float32)
    assert list(oracle.topk(z, 2)) == [0, 1]  # -0 ties with +0


# ------------------------------------------------------------------ pool
def test_block_max_and_pool_small_context_is_everything():
    g = pages()["candidate_pool"]
    assert g["blocks"] * g["block_positions"] == g["positions"]
    assert abs(g["positions"] / 2 ** 20 - g["fraction_of_1M"]) < 0.0005
    rng = np.random.default_rng(2)
    vis = 1000  # 125 blocks < 2048: the pool is every visible position
    s = rng.standard_normal(1024).astype(np.float32)
    bm = oracle.block_max(np.where(np.arange(1024) < vis, s, -np.inf).astype(np.float32), vis, 128)
    assert np.all(np.isneginf(bm[125:]))
    assert bm[3] == s[24:32].max()
    pool = oracle.candidate_pool(bm, g["blocks"])
    assert list(pool[:125]) == list(range(125)) and np.all(pool[125:] == -1)


def test_block_max_partial_last_block():
    s = np.arange(20, dtype=np.float32)
    bm = oracle.block_max(s, 19, 3)  # block 2 holds positions 16..18 only
    assert list(bm) == [7.0, 15.0, 18.0]


def _make_tie_heavy(rng, n, d_I=4, H_I=2):
    q = rng.integers(-1, 2, (H_I, d_I)).astype(np.float32)
    k = rng.integers(-1, 2, (n, d_I)).astype(np.float32)
    w = np.array([0.5, 0.25][:H_I], np.float32)
    return q, w, k


def test_full_topk_is_inside_pool_and_reindex_reproduces_it():
    rng = np.random.default_rng(9)
    for trial in range(40):
        n = int(rng.integers(40, 400))
        vis = int(rng.integers(1, n + 1))
        P_b = int(rng.integers(1, 12))
        k = int(rng.integers(1, P_b + 1))  # k <= pool blocks
        q, w, kc = _make_tie_heavy(rng, n)
        s = oracle.full_scores(q, w, kc, vis, n)
        nb = (n + 7) // 8
        bm = oracle.block_max(s, vis, nb)
        pool = oracle.candidate_pool(bm, P_b)
        full_idx = oracle.topk(s, k)
        pool_pos = {8 * b + j for b in pool if b >= 0 for j in range(8) if 8 * b + j < vis}
        assert all(i in pool_pos for i in full_idx if i >= 0)
        ps = oracle.pool_scores(q, w, kc, vis, pool)
        re_idx = oracle.pool_topk(ps, pool, k)
        assert list(re_idx) == list(full_idx), trial


def test_pool_scores_match_full_scores_at_pool_positions():
    rng = np.random.default_rng(4)
    n, vis = 200, 181
    q = rng.standard_normal((3, 16)).astype(np.float32)
    w = rng.random(3).astype(np.float32)
    kc = rng.standard_normal((n, 16)).astype(np.float32)
    s = oracle.full_scores(q, w, kc, vis, n)
    pool = np.array([2, 7, 22, -1], np.int32)  # block 22 holds 176..183: 181.. invisible
    ps = oracle.pool_scores(q, w, kc, vis, pool)
    for slot in range(32):
        b = pool[slot // 8]
        pos = 8 * b + slot % 8
        if b < 0 or pos >= vis:
            assert np.isneginf(ps[slot])
        else:
            assert ps[slot] == s[pos]


# ------------------------------------------------------------------ attention
def _dense_attention(q, rows, scale):
    z = scale * (q.astype(np.float64) @ rows.T)
    z -= z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    return p @ rows


def _canonical_kv(rng, n, D):
    """Rows whose MXFP4 encoding is exact (every 16-block has a max code 6)."""
    t = e4m3_table_torch()
    out = np.zeros((n, D))
    for r in range(n):
        for b in range(D // 16):
            sc = int(rng.integers(40, 70))
            mags = rng.integers(0, 8, 16)
            mags[0] = 7
            sg = rng.integers(0, 2, 16)
            out[r, 16 * b:16 * b + 16] = [(-1 if s and m else 1) * E2M1_SPEC[m] * t[sc]
                                          for m, s in zip(mags, sg)]
    return out.astype(np.float32)


def test_attention_topk_everything_equals_dense():
    rng = np.random.default_rng(12)
    n, D, H, W = 40, 64, 4, 5
    kv = _canonical_kv(rng, n, D)
    codes, scales = oracle.mxfp4_encode(kv)
    swa = rng.standard_normal((W, D)).astype(np.float32)
    q = rng.standard_normal((H, D)).astype(np.float32)
    idx = np.arange(n, dtype=np.int32)[::-1].copy()  # order must not matter
    idx = np.concatenate([idx, -np.ones(3, np.int32)])
    got = oracle.attn_decode(q, codes, scales, idx, swa, W, 1 / 8)
    ref = _dense_attention(q, np.concatenate([kv, swa]).astype(np.float64), 1 / 8)
    assert np.max(np.abs(got - ref)) < 1e-6


def test_attention_special_cases():
    rng = np.random.default_rng(13)
    n, D, H = 30, 32, 2
    kv = _canonical_kv(rng, n, D)
    codes, scales = oracle.mxfp4_encode(kv)
    swa = rng.standard_normal((4, D)).astype(np.float32)
    idx = np.arange(n, dtype=np.int32)
    # q = 0 -> uniform weights -> mean of the set
    out = oracle.attn_decode(np.zeros((H, D), np.float32), codes, scales, idx, swa, 4, 0.1)
    mean = np.concatenate([kv, swa]).astype(np.float64).mean(0)
    assert np.max(np.abs(out - mean)) < 1e-6
    # a single row -> that row exactly
    one = np.array([7] + [-1] * 5, np.int32)
    out = oracle.attn_decode(rng.standard_normal((H, D)).astype(np.float32), codes, scales, one,
                             swa, 0, 0.1)
    assert np.array_equal(out, np.broadcast_to(kv[7], (H, D)))
    # permutation of idx does not change the result
    qq = rng.standard_normal((H, D)).astype(np.float32)
    a = oracle.attn_decode(qq, codes, scales, idx, swa, 4, 0.2)
    b = oracle.attn_decode(qq, codes, scales, rng.permutation(idx).astype(np.int32), swa, 4, 0.2)
    assert np.max(np.abs(a - b)) < 1e-6
    # empty set -> zeros
    z = oracle.attn_decode(qq, codes, scales, -np.ones(4, np.int32), swa, 0, 0.2)
    assert not z.any()


# ------------------------------------------------------------------ prefill
def test_prefill_visibility_closed_form():
    w = ci.PREFILL_CHUNK
    p0, T, m = w.prior_tokens, w.T, w.m
    total = sum(oracle.prefill_vis(p0 + t, w.N, m) for t in range(T))
    # floor((p0 + t + 1) / 2) over t = 0..T-1 with p0 even: pairs (a, a) for a = p0/2 ... ;
    # T/2 pairs of equal values starting at p0/2 (t=0 gives (p0+1)//2 = p0/2),
    # plus the final +1 shift: sum = 2 * sum_{a=p0/2}^{p0/2+T/2-1} a + T/2.
    a0 = p0 // 2
    closed = 2 * (T // 2) * (2 * a0 + T // 2 - 1) // 2 + T // 2
    assert total == closed == 1_090_519_040
    assert oracle.prefill_vis(0, 10, 2) == 0 and oracle.prefill_vis(1, 10, 2) == 1
    assert oracle.prefill_vis(100, 10, 1) == 10  # capped by the cache length


def test_prefill_window_and_replay_start():
    rng = np.random.default_rng(21)
    T, H, D, W = 6, 2, 32, 4
    kv = _canonical_kv(rng, 8, D)
    codes, scales = oracle.mxfp4_encode(kv)
    swa = rng.standard_normal((T + W - 1, D)).astype(np.float32)
    q = rng.standard_normal((T, H, D)).astype(np.float32)
    idx = -np.ones((T, 2), np.int32)
    idx[:, 0] = 3
    q_pos0 = 1  # token positions 1..6; window rows cover positions -2..6
    out = oracle.attn_prefill(q, codes, scales, idx, swa, W, q_pos0, 0, 0.125)
    for t in range(T):
        i = q_pos0 + t
        lo = max(0, i - W + 1)
        rows = [kv[3]] + [swa[p - (q_pos0 - (W - 1))] for p in range(lo, i + 1)]
        ref = _dense_attention(q[t], np.array(rows, np.float64), 0.125)
        assert np.max(np.abs(out[t] - ref)) < 1e-6
    # replay start s = 4: window [max(4, i-3), i]
    out = oracle.attn_prefill(q, codes, scales, idx, swa, W, q_pos0, 4, 0.125)
    for t in range(T):
        i = q_pos0 + t
        lo = max(4, i - W + 1)
        rows = [kv[3]] + [swa[p - (q_pos0 - (W - 1))] for p in range(lo, i + 1)]
        ref = _dense_attention(q[t], np.array(rows, np.float64), 0.125)
        assert np.max(np.abs(out[t] - ref)) < 1e-6


# ------------------------------------------------------------------ modes
def test_reuse_layers_emit_identical_indices_and_reindex_differs():
    """Schedule F R R R X R R R: Reuse layers keep their source's idx bitwise;
    Reindex with its own query makes a new selection inside the pool."""
    rng = np.random.default_rng(31)
    n, d_I, H_I, k, P_b = 512, 16, 2, 16, 8
    kc = rng.standard_normal((n, d_I)).astype(np.float32)
    qs = [rng.standard_normal((H_I, d_I)).astype(np.float32) for _ in range(2)]
    ws = [rng.random(H_I).astype(np.float32) for _ in range(2)]
    s = oracle.full_scores(qs[0], ws[0], kc, n, n)
    pool = oracle.candidate_pool(oracle.block_max(s, n, n // 8), P_b)
    idx_full = oracle.topk(s, k)
    idx_re = oracle.pool_topk(oracle.pool_scores(qs[1], ws[1], kc, n, pool), pool, k)
    per_layer = []
    cur = None
    for mode in "FRRRXRRR":
        if mode == "F":
            cur = idx_full
        elif mode == "X":
            cur = idx_re
        per_layer.append(cur.copy())
    for l in (1, 2, 3):
        assert np.array_equal(per_layer[l], per_layer[0])
    for l in (5, 6, 7):
        assert np.array_equal(per_layer[l], per_layer[4])
    assert not np.array_equal(per_layer[4], per_layer[0])
    pool_pos = {8 * b + j for b in pool if b >= 0 for j in range(8)}
    assert all(i in pool_pos for i in idx_re)


# ------------------------------------------------------------------ generator
def test_generator_is_deterministic_and_row_addressable():
    a = ci.gaussian(5, ci.TID_KV, (10, 64))
    b = ci.gaussian_rows(5, ci.TID_KV, torch.tensor([3, 7]), 64)
    assert torch.equal(a[[3, 7]], b)
    u = ci.uniform(5, ci.TID_W, (1000,))
    assert float(u.min()) >= 0.0 and float(u.max()) < 1.0
    g = ci.gaussian(1, 2, (200000,))
    assert abs(float(g.mean())) < 0.02 and abs(float(g.std()) - 1) < 0.02


def test_attention_large_logits_stay_finite():
    # logits near 1e3 overflow exp() unless the softmax subtracts its maximum;
    # the answer is then the row with the largest logit.
    rng = np.random.default_rng(14)
    n, D, H = 12, 32, 2
    kv = _canonical_kv(rng, n, D)
    codes, scales = oracle.mxfp4_encode(kv)
    dec = oracle.mxfp4_decode(codes, scales)
    q = np.broadcast_to(dec[5].astype(np.float32), (H, D)).copy()
    z = dec @ q[0].astype(np.float64)
    top = np.sort(z)
    j = int(np.argmax(z))
    scale = 1000.0 / top[-1]
    assert scale * (top[-1] - top[-2]) > 40  # the top row wins by e^40
    out = oracle.attn_decode(q, codes, scales, np.arange(n, dtype=np.int32), kv[:0], 0, scale)
    assert np.all(np.isfinite(out))
    assert np.max(np.abs(out - dec[j])) < 1e-6


def test_full_topk_equals_topk_inside_pool_and_pool_through_superblocks():
    """Two identities the GPU path relies on, checked by brute force on the
    oracle: (1) with k <= P_b the Full top-k is the top-k among the pool's
    positions; (2) the P_b best blocks are the P_b best among the blocks of
    the P_b best 8-block super-blocks."""
    rng = np.random.default_rng(17)
    for trial in range(600):
        n = int(rng.integers(8, 2500)); vis = int(rng.integers(1, n + 1))
        P_b = int(rng.integers(1, 30)); k = int(rng.integers(1, P_b + 1))
        if trial % 3 == 0:
            s = rng.integers(0, 4, n).astype(np.float32)
        elif trial % 3 == 1:
            s = rng.standard_normal(n).astype(np.float32)
        else:
            s = np.round(rng.standard_normal(n) * 3).astype(np.float32)
        s[vis:] = -np.inf
        nb = (n + 7) // 8
        bm = oracle.block_max(s, vis, nb)
        pool = oracle.candidate_pool(bm, P_b)
        slots = np.full(8 * P_b, -np.inf, np.float32)
        for i, b in enumerate(pool):
            for j in range(8):
                if b >= 0 and 8 * b + j < n:
                    slots[8 * i + j] = s[8 * b + j]
        assert np.array_equal(oracle.pool_topk(slots, pool, k), oracle.topk(s, k)), trial
        nsb = (nb + 7) // 8
        sbm = np.array([bm[8 * i:8 * i + 8].max() for i in range(nsb)], np.float32)
        sb = oracle.topk(sbm, P_b)
        cand = np.full(8 * P_b, -np.inf, np.float32)
        for i, x in enumerate(sb):
            for j in range(8):
                if x >= 0 and 8 * x + j < nb:
                    cand[8 * i + j] = bm[8 * x + j]
        sel = oracle.topk(cand, P_b)
        pool2 = np.array([8 * sb[t // 8] + t % 8 if t >= 0 else -1 for t in sel], np.int32)
        assert np.array_equal(pool2, pool), trial


# ---------------------------------------------------------------------------
# Indexer-K projection (a Full layer projects indexer K from its main KV):
# fp32 fma chain over the latent channels, then the nearest bfloat16.

def _bf16_bits_torch(v: np.ndarray) -> np.ndarray:
    # torch's float32 -> bfloat16 conversion (round to nearest, ties to even)
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_nearest_matches_library_conversion_and_ties():
    g = np.random.default_rng(7)
    vals = np.concatenate([g.standard_normal(4000).astype(np.float32) * 10.0 ** g.integers(-30, 30, 4000),
                           np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40, -1e-40], np.float32)])
    got = np.array([oracle.bf16_nearest(v) for v in vals], np.uint16)
    assert np.array_equal(got, _bf16_bits_torch(vals))
    # exact ties: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> the even one (1);
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6 -> the even one (1 + 2^-6)
    assert oracle.bf16_nearest(1.0 + 2.0 ** -8) == 0x3F80
    assert oracle.bf16_nearest(1.0 + 3 * 2.0 ** -8) == 0x3F82
    assert oracle.bf16_nearest(-(1.0 + 2.0 ** -8)) == 0xBF80


def test_projection_one_hot_and_permutation_copy_the_latent():
    g = np.random.default_rng(11)
    D, d_I, n = 512, 128, 5
    x = torch.from_numpy(g.standard_normal((n, D)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    W = np.zeros((D, d_I), np.float32)
    W[np.arange(d_I), np.arange(d_I)] = 1.0
    assert np.array_equal(oracle.project_kidx(x, W), _bf16_bits_torch(x[:, :d_I]))
    perm = g.permutation(D)[:d_I]
    W = np.zeros((D, d_I), np.float32)
    W[perm, np.arange(d_I)] = 1.0
    assert np.array_equal(oracle.project_kidx(x, W), _bf16_bits_torch(x[:, perm]))
    # a scaled column: k[j] = 2^-3 * x[perm[j]] exactly
    W *= 0.125
    assert np.array_equal(oracle.project_kidx(x, W), _bf16_bits_torch(x[:, perm] * 0.125))


def test_projection_exactly_summable_equals_float64_matmul():
    # x and W on a 2^-3 grid within +-4: every partial sum is a multiple of
    # 2^-6 below 2^13, exact in float32 in any order, so the chain equals the
    # float64 matrix product, and the rounding is the library's conversion
    g = np.random.default_rng(13)
    D, d_I, n = 512, 128, 7
    x = np.clip(np.round(g.standard_normal((n, D)) * 8) / 8, -4, 4).astype(np.float32)
    W = np.clip(np.round(g.standard_normal((D, d_I)) * 8) / 8, -4, 4).astype(np.float32)
    exact = x.astype(np.float64) @ W.astype(np.float64)
    assert np.array_equal(exact.astype(np.float32).astype(np.float64), exact)
    assert np.array_equal(oracle.project_kidx(x, W), _bf16_bits_torch(exact.astype(np.float32)))


def test_projection_chain_is_fused_and_forward():
    D, d_I = 16, 8
    # fused: channel 0 puts -(1 + 2^-22) in the accumulator, channel 1 adds
    # (1 + 2^-23)^2 = 1 + 2^-22 + 2^-46; one rounding leaves exactly 2^-46
    # (bfloat16 0x2880), a rounded product first would leave 0
    x = np.zeros((1, D), np.float32)
    W = np.zeros((D, d_I), np.float32)
    x[0, 0], W[0, 0] = 1.0, -(1.0 + 2.0 ** -22)
    x[0, 1] = W[1, 0] = 1.0 + 2.0 ** -23
    out = oracle.project_kidx(x, W)
    assert out[0, 0] == 0x2880 and np.all(out[0, 1:] == 0)
    # forward order: 2^30 + 1 rounds to 2^30 in float32, then -2^30 cancels
    # to +0; a chain run from the last channel would give exactly 1 (0x3F80)
    x = np.zeros((1, D), np.float32)
    W = np.zeros((D, d_I), np.float32)
    x[0, 0], W[0, 0] = 2.0 ** 30, 1.0
    x[0, 1], W[1, 0] = 1.0, 1.0
    x[0, 2], W[2, 0] = 2.0 ** 30, -1.0
    assert oracle.project_kidx(x, W)[0, 0] == 0


# ---------------------------------------------------------- prefill scores
@pytest.mark.parametrize("m", [1, 2])
def test_prefill_scores_equal_masked_float64_product(m):
    """Per-row scores of a prefill chunk ("...KV Cache Compression" notes,
    section 2: the encoder compresses m tokens per entry; section 3: a Full
    layer scores every causally visible entry).

    On an exactly-summable grid (q, k multiples of 2^-3 in [-4, 4], w multiples
    of 2^-4) every partial sum is exact in float32, so the oracle's rows must
    equal a float64 product masked by the closed-form visibility
    vis(t) = min(ctx_len, floor((q_pos[t] + 1) / m)).  Non-square H_I x d_I,
    per-row w and q, and ld > ctx_len catch a stride slip (row t reading row
    t-1's q or w, or writing at t * ctx_len) and a visibility taken from the
    wrong row (all rows see different counts here)."""
    rng = np.random.default_rng(40 + m)
    T, H_I, d_I, ctx, ld = 9, 3, 5, 37, 45
    q = np.clip(np.round(rng.standard_normal((T, H_I, d_I)) * 8) / 8, -4, 4).astype(np.float32)
    k = np.clip(np.round(rng.standard_normal((ctx, d_I)) * 8) / 8, -4, 4).astype(np.float32)
    w = (rng.integers(1, 16, (T, H_I)) / 16).astype(np.float32)
    # positions out of order and spread so every row has its own vis; the last
    # row's count is capped by ctx_len
    q_pos = np.array([0, 5, 2, 19, 11, 30, 33, 7, 200], np.int64)
    got = oracle.prefill_scores(q, w, k, q_pos, ctx, m, ld)
    assert got.shape == (T, ld)
    seen = set()
    for t in range(T):
        vis = min(ctx, (int(q_pos[t]) + 1) // m)
        seen.add(vis)
        d = k.astype(np.float64) @ q[t].astype(np.float64).T        # [ctx][H_I]
        ref = np.maximum(d, 0.0) @ w[t].astype(np.float64)           # [ctx]
        assert np.array_equal(got[t, :vis].astype(np.float64), ref[:vis]), t
        assert np.all(np.isneginf(got[t, vis:])), t
    assert len(seen) == T          # every row has a different visible count
    assert min(ctx, (200 + 1) // m) == ctx


def test_prefill_scores_rows_are_independent_full_scores():
    """Swapping two rows' (q, w, q_pos) swaps their output rows, and a row
    equals the decode-form score of the same query over its visible entries:
    a prefill row is a Full-layer score with its own visibility."""
    rng = np.random.default_rng(77)
    T, H_I, d_I, ctx = 4, 2, 7, 50
    q = rng.standard_normal((T, H_I, d_I)).astype(np.float32)
    k = rng.standard_normal((ctx, d_I)).astype(np.float32)
    w = rng.random((T, H_I)).astype(np.float32)
    q_pos = np.array([3, 60, 21, 98], np.int64)
    a = oracle.prefill_scores(q, w, k, q_pos, ctx, 2, ctx)
    perm = [2, 0, 3, 1]
    b = oracle.prefill_scores(q[perm].copy(), w[perm].copy(), k, q_pos[perm].copy(), ctx, 2, ctx)
    assert np.array_equal(a[perm].view(np.uint32), b.view(np.uint32))
    for t in range(T):
        vis = min(ctx, (int(q_pos[t]) + 1) // 2)
        one = np.array([oracle.score_one(q[t], w[t], k[j]) for j in range(vis)], np.float32)
        assert np.array_equal(a[t, :vis].view(np.uint32), one.view(np.uint32))
