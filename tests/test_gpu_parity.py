"""GPU (HIP, through the C ABI) versus the CPU oracle on the same seeded inputs.

Bar: bit-exact for MXFP4 bytes, scores, block maxima, pool ids and top-k
indices; attention outputs within 2e-3 max abs of the float64 oracle.
Every expected value comes from oracle/ on inputs from csa2_inputs; nothing
the GPU computed is fed to the oracle.
"""
import math

import numpy as np
import pytest
import torch

import csa2_inputs as ci
import oracle

pytestmark = pytest.mark.gpu

ATOL = 2e-3


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.fail("gpu tests need a GPU")
    import compressed_sparse_attention_05_amd as K
    K.lib()
    print("libcsa2:", K.version(), flush=True)
    return K


def dev(x):
    return torch.as_tensor(x).cuda()


def bf16_bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ MXFP4
def _special_rows(D):
    rows = []
    base = np.zeros(D, np.float32)
    for s in [1.0, 0.171875, 3.75, 448.0, 2.0 ** -9, 2.0 ** -6]:
        r = base.copy()
        pts = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, 6, -0.25, -0.75, -1.25, -1.75,
                        -2.5, -3.5, -5, -6], np.float32) * np.float32(s)
        r[:16] = pts
        rows.append(r)
    r = base.copy(); r[5] = math.sqrt(512); rows.append(r)
    r = base.copy(); r[:] = -0.0; rows.append(r)
    r = base.copy(); r[0], r[1] = 1e6, -1e6; rows.append(r)
    r = base.copy(); r[17] = 1e-30; rows.append(r)
    r = base.copy(); r[:16] = 6 * 1.0625; rows.append(r)
    r = base.copy(); r[:16] = 6 * 1.1875; rows.append(r)
    return np.stack(rows)


@pytest.mark.parametrize("D,dtype", [(64, torch.float32), (512, torch.bfloat16), (512, torch.float32)])
def test_kv_write_bitexact(K, D, dtype):
    n = 300
    x = ci.gaussian(11, ci.TID_KV, (n, D), dtype=torch.float32, clip=ci.NORM_BOUND)
    x = torch.cat([x, torch.from_numpy(_special_rows(D))]).to(dtype)
    n = x.shape[0]
    cap_rows = n + 37
    dst = torch.randperm(cap_rows, generator=torch.Generator().manual_seed(3))[:n].to(torch.int64)
    dst[5] = -1                 # skipped
    dst[6] = cap_rows + 4       # out of range: skipped
    codes = dev(torch.full((cap_rows, D // 2), 0xAB, dtype=torch.uint8))
    scales = dev(torch.full((cap_rows, D // 16), 0xCD, dtype=torch.uint8))
    K.mxfp4_kv_write(dev(x), dev(dst), codes, scales)
    torch.cuda.synchronize()
    want_c, want_s = oracle.mxfp4_encode(x.float() if dtype == torch.float32 else x)
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    for i in range(n):
        d = int(dst[i])
        if 0 <= d < cap_rows:
            assert np.array_equal(got_c[d], want_c[i]), i
            assert np.array_equal(got_s[d], want_s[i]), i
    untouched = set(range(cap_rows)) - {int(d) for d in dst if 0 <= int(d) < cap_rows}
    for d in untouched:
        assert (got_c[d] == 0xAB).all() and (got_s[d] == 0xCD).all()


def test_kv_write_copies_indexer_rows(K):
    n, D, d_I, cap = 10, 512, 128, 128
    x = ci.gaussian(12, ci.TID_KV, (n, D), dtype=torch.bfloat16)
    kr = ci.gaussian(12, ci.TID_K_IDX, (n, d_I), dtype=torch.bfloat16)
    dst = torch.arange(n, dtype=torch.int64) + 3
    codes = dev(torch.zeros((cap, D // 2), dtype=torch.uint8))
    scales = dev(torch.zeros((cap, D // 16), dtype=torch.uint8))
    kc = dev(torch.zeros((cap, d_I), dtype=torch.bfloat16))
    K.mxfp4_kv_write(dev(x), dev(dst), codes, scales, dev(kr), kc)
    torch.cuda.synchronize()
    rows = K.untile_indexer_cache(kc.view(1, cap, d_I))[0].cpu()
    assert torch.equal(rows[3:13], kr)
    assert (rows[:3].view(torch.int16) == 0).all() and (rows[13:].view(torch.int16) == 0).all()


# ------------------------------------------------------------------ dequant through attention
def test_dequant_every_code_and_scale_exact(K):
    """A single selected row attended by any query returns that row exactly:
    checks E2M1 x E4M3 decoding, nibble order and the V operand path."""
    D, H = 512, 64
    scs = list(range(1, 127, 3)) + [126]
    n = len(scs)
    codes = np.zeros((n, D // 2), np.uint8)
    scales = np.zeros((n, D // 16), np.uint8)
    for r, sc in enumerate(scs):
        nib = (np.arange(D) + r) % 16
        codes[r] = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)
        scales[r] = sc
        scales[r, 3] = (sc + 40) % 127
    want = oracle.mxfp4_decode(codes, scales)
    B = n
    q = ci.gaussian(13, ci.TID_Q, (B, H, D), dtype=torch.bfloat16)
    idx = torch.full((B, 4), -1, dtype=torch.int32)
    idx[:, 1] = torch.arange(B, dtype=torch.int32)
    codes_b = np.broadcast_to(codes, (B, n, D // 2)).copy()
    scales_b = np.broadcast_to(scales, (B, n, D // 16)).copy()
    swa = torch.zeros((B, 1, D), dtype=torch.bfloat16)
    out = K.csa2_sparse_attn_decode(dev(q), dev(torch.from_numpy(codes_b)), dev(torch.from_numpy(scales_b)),
                                    dev(idx), dev(swa), dev(torch.zeros(B, dtype=torch.int32)))
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    for b in range(B):
        assert np.array_equal(o[b], np.broadcast_to(want[b], (H, D))), b


# ------------------------------------------------------------------ scores
def _score_case(K, seed, B, N, H_I, d_I, dtype, cap=None, ctx=None, ld=None):
    cap = cap or N
    ld = ld or cap
    q = ci.gaussian(seed, ci.TID_Q_IDX, (B, 1, H_I, d_I), dtype=dtype)
    w = ci.uniform(seed, ci.TID_W, (B, 1, H_I))
    kc = ci.gaussian(seed, ci.TID_K_IDX, (B, cap, d_I), dtype=dtype)
    ctx = ctx if ctx is not None else [N] * B
    ctx_t = torch.tensor(ctx, dtype=torch.int32)
    s, bm = K.csa2_index_score(dev(q), dev(w), K.tile_indexer_cache(dev(kc)), dev(ctx_t), ld=ld,
                               want_block_max=True)
    torch.cuda.synchronize()
    s, bm = s.cpu().numpy(), bm.cpu().numpy()
    for b in range(B):
        vis = min(ctx[b], cap)
        want = oracle.full_scores(q[b, 0], w[b, 0], kc[b], vis, ld)
        assert np.array_equal(s[b, 0].view(np.uint32), want.view(np.uint32)), b
        wbm = oracle.block_max(want, vis, (ld + 7) // 8)
        assert np.array_equal(bm[b, 0].view(np.uint32), wbm.view(np.uint32)), b
    return q, w, kc, s, bm


def test_score_full_tiny_fp32(K):
    _score_case(K, 101, B=1, N=1024, H_I=2, d_I=32, dtype=torch.float32)


def test_score_full_bf16_ragged(K):
    # ragged visible lengths, a tail that is not a multiple of 8 or of the tile
    _score_case(K, 102, B=3, N=5000, H_I=8, d_I=128, dtype=torch.bfloat16, cap=5056,
                ctx=[5003, 4099, 1], ld=5005)


def test_score_4x64(K):
    _score_case(K, 103, B=2, N=777, H_I=4, d_I=64, dtype=torch.bfloat16, cap=832, ctx=[777, 700])


def test_score_exactly_summable_grid(K):
    # multiples of 2^-3 in [-4, 4]: every order gives the exact value; heavy ties
    B, N, H_I, d_I = 2, 3008, 8, 128
    g = torch.Generator().manual_seed(5)
    q = (torch.randint(-32, 33, (B, 1, H_I, d_I), generator=g) / 8.0).to(torch.bfloat16)
    kc = (torch.randint(-32, 33, (B, N, d_I), generator=g) / 8.0).to(torch.bfloat16)
    w = (torch.randint(0, 16, (B, 1, H_I), generator=g) / 16.0).float()
    ctx = torch.tensor([N, N - 13], dtype=torch.int32)
    s, _ = K.csa2_index_score(dev(q), dev(w), K.tile_indexer_cache(dev(kc)), dev(ctx))
    s = s.cpu().numpy()
    for b in range(B):
        exact = np.maximum(kc[b].double().numpy() @ q[b, 0].double().numpy().T, 0) @ w[b, 0].double().numpy()
        vis = int(ctx[b])
        assert np.array_equal(s[b, 0, :vis].astype(np.float64), exact[:vis])
        assert np.all(np.isneginf(s[b, 0, vis:]))


# ------------------------------------------------------------------ top-k and pool
def _topk_check(K, vals, k, pool=None):
    vals = np.ascontiguousarray(vals, np.float32)
    got = K.csa2_topk(dev(torch.from_numpy(vals)), k,
                      pool_blocks=None if pool is None else dev(torch.from_numpy(pool))).cpu().numpy()
    for r in range(vals.shape[0]):
        want = oracle.topk(vals[r], k) if pool is None else oracle.pool_topk(vals[r], pool[r], k)
        assert np.array_equal(got[r], want), r



@pytest.mark.parametrize("n", [16384, 32768])
def test_topk_threshold_in_a_small_tied_bin(K, n):
    # The k-th key falls in a radix bin that holds only a cluster of 40 keys
    # near 50 (no other key lies in [40, 60)): the selection finishes such a
    # bin in one wave.  Rows 0-1: cluster values 2^-16 apart, some repeated;
    # rows 2-3: steps of 2^-20, which round to four float32 values (the ulp
    # at 50 is 2^-18), so the k-th key is tied many times over.
    rng = np.random.default_rng(21)
    rows = 4
    v = np.empty((rows, n), np.float32)
    for r in range(rows):
        hi = rng.uniform(60, 100, 2000)
        lo = rng.uniform(0, 40, n - 2040)
        steps = np.sort(rng.integers(0, 30 if r < 2 else 12, 40))
        cluster = 50.0 + steps * 2.0 ** (-16 if r < 2 else -20)
        row = np.concatenate([hi, cluster, lo]).astype(np.float32)
        v[r] = row[rng.permutation(n)]
    for k in (2001, 2020, 2039, 2040):
        _topk_check(K, v, k)

def test_topk_random_and_ties(K):
    rng = np.random.default_rng(7)
    v = rng.standard_normal((6, 20000)).astype(np.float32)
    v[1] = rng.integers(0, 5, 20000)           # heavy ties
    v[2] = 0.0                                  # all equal
    v[3, ::2] = -np.inf                         # half invalid
    v[4, :] = -np.inf; v[4, 17] = 3.0           # one valid
    v[5, 100:] = -0.0; v[5, :100] = 0.0         # signed zeros tie
    for k in (1, 64, 2048, 20000, 25000):
        _topk_check(K, v, k)


def test_topk_long_rows_fast_path_and_fallbacks(K):
    rng = np.random.default_rng(9)
    n = 100003
    v = rng.standard_normal((6, n)).astype(np.float32)
    v[1] = np.abs(v[1])                                   # scores >= 0 as in the method
    v[2] = rng.integers(0, 5, n)                          # ~20K ties per value: tie list overflows
    v[3] = 7.0                                            # everything equal
    v[4, :] = -np.inf; v[4, 50000:50010] = 1.0            # 10 valid slots
    v[5, ::3] = -np.inf
    for k in (1, 2048, 4096, 5000):                       # 5000 > the in-LDS sort: fallback
        _topk_check(K, v, k)
    # the full-scan shape: 1M slots, k = 2048
    big = np.abs(rng.standard_normal((2, 1 << 20))).astype(np.float32) * 10
    big[1, :] = np.round(big[1, :])                       # ties across the threshold
    _topk_check(K, big, 2048)


def test_topk_from_pool_equals_full_topk(K):
    rng = np.random.default_rng(10)
    rows, n, P_b = 5, 70000, 2048
    v = np.abs(rng.standard_normal((rows, n))).astype(np.float32) * 10
    v[1] = np.round(v[1])                       # ties everywhere
    v[2, 60001:] = -np.inf                      # invisible tail
    v[3] = 1.0                                  # all equal
    v[4, :] = -np.inf; v[4, 5:900:7] = 2.0      # fewer visible blocks than the pool
    nb = (n + 7) // 8
    bm = np.stack([oracle.block_max(v[r], int(np.sum(np.isfinite(v[r]))) if r in (2,) else n, nb)
                   for r in range(rows)])
    # block_max from the oracle for rows with an invisible tail uses vis; -inf entries
    # elsewhere are simply never chosen
    bm_t = dev(torch.from_numpy(bm))
    pool = K.csa2_build_candidate_pool(bm_t, P_b)
    for k in (1, 64, 2048):
        got = K.csa2_topk_from_pool(dev(torch.from_numpy(v)), pool, k).cpu().numpy()
        for r in range(rows):
            assert np.array_equal(got[r], oracle.topk(v[r], k)), (r, k)


@pytest.mark.parametrize("nb,ld", [(131075, 131075), (131069, 131069), (100003, 100003),
                                   (131072, 131072), (131069, 131072)])
def test_pool_through_superblocks(K, nb, ld):
    # > 32,768 blocks.  131,075 takes 32 super-blocks per thread.  The others
    # take 16: with odd strides (131,069 and 100,003 per row) rows are not
    # 16-byte aligned and each thread reads its own run; a stride that is a
    # multiple of 4 reads the rows coalesced, 131,069 of 131,072 with a
    # partial last float4
    rng = np.random.default_rng(11)
    rows, P_b = 3, 2048
    full = np.abs(rng.standard_normal((rows, ld))).astype(np.float32) * 20
    full[1] = np.round(full[1] / 4)             # heavy ties
    full[2, nb - 31075:] = -np.inf
    full[:, nb:] = 1e30                         # past n_blocks: must be ignored
    got = K.csa2_build_candidate_pool(dev(torch.from_numpy(full)), P_b, n_blocks=nb).cpu().numpy()
    for r in range(rows):
        assert np.array_equal(got[r], oracle.candidate_pool(full[r, :nb], P_b)), r


@pytest.mark.parametrize("n", [70000, 262144])
def test_pool_topk_fused_equals_two_calls(K, n):
    # csa2_pool_topk = pool and the Full top-k inside it, in one launch:
    # 70,000 positions (16 block maxima per thread) and 262,144 (32 per
    # thread, the largest row the fused path takes)
    rng = np.random.default_rng(12)
    rows, P_b = 4, 2048
    v = np.abs(rng.standard_normal((rows, n))).astype(np.float32) * 10
    v[1] = np.round(v[1])                       # ties everywhere
    v[2, n - 9999:] = -np.inf                   # invisible tail
    v[3, :] = -np.inf; v[3, 5:900:7] = 2.0      # fewer visible blocks than the pool
    vis = [n, n, n - 9999, n]
    nb = (n + 7) // 8
    bm = np.stack([oracle.block_max(v[r], vis[r], nb) for r in range(rows)])
    for k in (1, 64, 2048):
        pool, idx = K.csa2_pool_topk(dev(torch.from_numpy(bm)), dev(torch.from_numpy(v)), P_b, k)
        pool, idx = pool.cpu().numpy(), idx.cpu().numpy()
        for r in range(rows):
            assert np.array_equal(pool[r], oracle.candidate_pool(bm[r], P_b)), (r, k)
            assert np.array_equal(idx[r], oracle.topk(v[r], k)), (r, k)



@pytest.mark.parametrize("n", [70000, 262144])
def test_pool_topk_many_tied_block_maxima(K, n):
    # The top-k workgroup of csa2_pool_topk takes every block whose maximum
    # reaches the lower edge of the radix bin holding the P_b-th largest
    # maximum; with more than 3,072 such blocks it selects the exact pool
    # itself.  Rows 0-2 reach that (all maxima equal, a few values tied by
    # thousands, 2,047 distinct maxima above a plateau); row 3 stays on the
    # bracket with somewhat more than P_b blocks.
    rng = np.random.default_rng(13)
    P_b = 2048
    v = np.abs(rng.standard_normal((4, n))).astype(np.float32)
    v[0] = 1.5
    v[1] = np.round(v[1] * 2)
    v[2] = 0.25
    v[2, 64:64 + 8 * 2047:8] = 5 + np.arange(2047, dtype=np.float32)
    v[3] = np.round(v[3] * 64) / 64 + 3
    nb = (n + 7) // 8
    bm = np.stack([oracle.block_max(v[r], n, nb) for r in range(4)])
    for k in (1, 2047, 2048):
        pool, idx = K.csa2_pool_topk(dev(torch.from_numpy(bm)), dev(torch.from_numpy(v)), P_b, k)
        pool, idx = pool.cpu().numpy(), idx.cpu().numpy()
        for r in range(4):
            assert np.array_equal(pool[r], oracle.candidate_pool(bm[r], P_b)), (r, k)
            assert np.array_equal(idx[r], oracle.topk(v[r], k)), (r, k)

def test_topk_small_rows_exhaustive(K):
    rng = np.random.default_rng(8)
    rows = rng.integers(0, 3, (500, 9)).astype(np.float32)
    rows[rng.random((500, 9)) < 0.2] = -np.inf
    for k in (1, 3, 9, 12):
        _topk_check(K, rows, k)


def test_pool_and_reindex_bitexact(K):
    B, N, H_I, d_I, P_b, k = 2, 70016, 8, 128, 2048, 2048
    q, w, kc, s, bm = _score_case(K, 104, B=B, N=N, H_I=H_I, d_I=d_I, dtype=torch.bfloat16,
                                  ctx=[N, N - 4001])
    pool = K.csa2_build_candidate_pool(dev(torch.from_numpy(bm)), P_b).cpu().numpy()
    pools = []
    for b in range(B):
        vis = [N, N - 4001][b]
        ws = oracle.full_scores(q[b, 0], w[b, 0], kc[b], vis, N)
        wpool = oracle.candidate_pool(oracle.block_max(ws, vis, (N + 7) // 8), P_b)
        assert np.array_equal(pool[b, 0], wpool), b
        pools.append(wpool)
    # Reindex with a new indexer query over the pool
    q2 = ci.gaussian(105, ci.TID_Q_IDX, (B, 1, H_I, d_I), dtype=torch.bfloat16)
    w2 = ci.uniform(105, ci.TID_W, (B, 1, H_I))
    pool_t = dev(torch.from_numpy(np.stack(pools)[:, None]))
    ctx = torch.tensor([N, N - 4001], dtype=torch.int32)
    ps, _ = K.csa2_index_score(dev(q2), dev(w2), K.tile_indexer_cache(dev(kc)), dev(ctx), pool_blocks=pool_t)
    idx = K.csa2_topk(ps, k, pool_blocks=pool_t).cpu().numpy()
    ps = ps.cpu().numpy()
    for b in range(B):
        vis = [N, N - 4001][b]
        wps = oracle.pool_scores(q2[b, 0], w2[b, 0], kc[b], vis, pools[b])
        assert np.array_equal(ps[b, 0].view(np.uint32), wps.view(np.uint32)), b
        assert np.array_equal(idx[b, 0], oracle.pool_topk(wps, pools[b], k)), b


# ------------------------------------------------------------------ attention
def _attn_case(K, seed, B, N, D, H, k, W, swa_lens, dtype=torch.bfloat16, sm=None, dup=False):
    kv = ci.gaussian(seed, ci.TID_KV, (B, N, D), dtype=torch.float32, clip=ci.NORM_BOUND)
    codes = np.zeros((B, N, D // 2), np.uint8)
    scales = np.zeros((B, N, D // 16), np.uint8)
    for b in range(B):
        codes[b], scales[b] = oracle.mxfp4_encode(kv[b])
    g = torch.Generator().manual_seed(seed)
    idx = torch.stack([torch.randperm(N, generator=g)[:k] for _ in range(B)]).to(torch.int32)
    idx, _ = torch.sort(idx, dim=1)
    idx[0, -5:] = -1
    if dup:
        idx[-1, :k // 2] = idx[-1, 0]
    q = ci.gaussian(seed, ci.TID_Q, (B, H, D), dtype=dtype)
    swa = ci.gaussian(seed, ci.TID_SWA, (B, W, D), dtype=dtype)
    sl = torch.tensor(swa_lens, dtype=torch.int32)
    sm = sm if sm is not None else 1 / math.sqrt(D)
    out = K.csa2_sparse_attn_decode(dev(q), dev(torch.from_numpy(codes)), dev(torch.from_numpy(scales)),
                                    dev(idx), dev(swa), dev(sl), sm_scale=sm).cpu().numpy()
    errs = []
    for b in range(B):
        want = oracle.attn_decode(q[b], codes[b], scales[b], idx[b].numpy(), swa[b], min(swa_lens[b], W), sm)
        errs.append(np.max(np.abs(out[b] - want)))
    print("max abs err per unit:", ["%.2e" % e for e in errs], flush=True)
    assert max(errs) < ATOL
    return max(errs)


def test_attention_tiny_config(K):
    w = ci.TINY
    _attn_case(K, w.seed, B=1, N=w.N, D=w.D, H=w.H, k=w.k, W=w.W, swa_lens=[w.W], dtype=torch.float32,
               sm=1 / 8)


def test_attention_d512_ragged(K):
    # k not a multiple of the key tile, partial windows, duplicates, -1 entries
    _attn_case(K, 201, B=3, N=5000, D=512, H=64, k=333, W=128, swa_lens=[128, 7, 0], dup=True)


def test_attention_d512_k2048_split(K):
    _attn_case(K, 202, B=2, N=40000, D=512, H=128, k=2048, W=128, swa_lens=[128, 128])


def test_attention_many_units_warp_specialised(K):
    # 16 or more query units take the warp-specialised kernel: a tile that
    # straddles the main/window boundary (k = 333), ragged windows, -1
    # entries and duplicates, in bf16 and float32, one and two head blocks
    lens = [(7 * b) % 129 for b in range(64)]
    _attn_case(K, 203, B=64, N=3000, D=512, H=64, k=333, W=128, swa_lens=lens, dup=True)
    _attn_case(K, 204, B=64, N=2000, D=512, H=128, k=256, W=128, swa_lens=[128] * 64, dtype=torch.float32)
    # the smallest batch on this kernel, with several key splits per unit
    _attn_case(K, 205, B=16, N=4000, D=512, H=64, k=1500, W=128, swa_lens=[(11 * b) % 129 for b in range(16)])


def test_attention_empty_set_is_zero(K):
    B, N, D, H = 2, 64, 512, 64
    codes = dev(torch.zeros((B, N, D // 2), dtype=torch.uint8))
    scales = dev(torch.zeros((B, N, D // 16), dtype=torch.uint8))
    idx = dev(torch.full((B, 40), -1, dtype=torch.int32))
    q = dev(ci.gaussian(3, ci.TID_Q, (B, H, D), dtype=torch.bfloat16))
    swa = dev(torch.zeros((B, 8, D), dtype=torch.bfloat16))
    out = K.csa2_sparse_attn_decode(q, codes, scales, idx, swa, dev(torch.zeros(B, dtype=torch.int32)))
    assert not out.cpu().any()


def test_attention_prefill_window(K):
    T, N, D, H, k, W = 40, 3000, 512, 64, 256, 128
    seed = 301
    kv = ci.gaussian(seed, ci.TID_KV, (N, D), dtype=torch.float32)
    codes, scales = oracle.mxfp4_encode(kv)
    g = torch.Generator().manual_seed(seed)
    idx = torch.stack([torch.sort(torch.randperm(N, generator=g)[:k])[0] for _ in range(T)]).to(torch.int32)
    q = ci.gaussian(seed, ci.TID_Q, (T, H, D), dtype=torch.bfloat16)
    swa = ci.gaussian(seed, ci.TID_SWA, (T + W - 1, D), dtype=torch.bfloat16)
    for q_pos0, s0 in [(5, 0), (1000, 0), (1000, 1030)]:
        out = K.csa2_sparse_attn_prefill(dev(q), dev(torch.from_numpy(codes)), dev(torch.from_numpy(scales)),
                                         dev(idx), dev(swa), W, q_pos0, swa_start=s0).cpu().numpy()
        want = oracle.attn_prefill(q, codes, scales, idx.numpy(), swa, W, q_pos0, s0, 1 / math.sqrt(D))
        err = np.max(np.abs(out - want))
        print("prefill", q_pos0, s0, "err %.2e" % err, flush=True)
        assert err < ATOL


@pytest.mark.parametrize("T,k", [(520, 2048), (1024, 2048), (1024, 2000)])
def test_attention_prefill_long_split_sampled(K, T, k):
    """Many query units on the warp-specialised kernel: 520 units take two
    key splits per query; 1,024 units take one, so each workgroup walks all
    34 key tiles of its query (index list restaged in windows) and writes
    the output directly.  These long splits dequantise the next tile inside
    P.V; with k = 2,000 the split starts with three generic tiles, the first
    of them 16 main entries and 48 window rows.  Sampled queries vs the
    oracle."""
    N, D, H, W = 40000, 512, 64, 128
    seed = 302
    kv = ci.gaussian(seed, ci.TID_KV, (N, D), dtype=torch.float32)
    codes, scales = oracle.mxfp4_encode(kv)
    g = torch.Generator().manual_seed(seed)
    idx = torch.stack([torch.sort(torch.randperm(N, generator=g)[:k])[0] for _ in range(T)]).to(torch.int32)
    idx[7, 100:300] = -1
    q = ci.gaussian(seed, ci.TID_Q, (T, H, D), dtype=torch.bfloat16)
    swa = ci.gaussian(seed, ci.TID_SWA, (T + W - 1, D), dtype=torch.bfloat16)
    q_pos0 = 30000
    out = K.csa2_sparse_attn_prefill(dev(q), dev(torch.from_numpy(codes)), dev(torch.from_numpy(scales)),
                                     dev(idx), dev(swa), W, q_pos0).cpu().numpy()
    errs = []
    for t in (0, 7, 100, 333, T - 1):
        want = oracle.attn_prefill(q[t:t + 1], codes, scales, idx[t:t + 1].numpy(), swa[t:t + W], W,
                                   q_pos0 + t, 0, 1 / math.sqrt(D))
        errs.append(np.max(np.abs(out[t] - want[0])))
    print("sampled errs", ["%.2e" % e for e in errs], flush=True)
    assert max(errs) < ATOL
