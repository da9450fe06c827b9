"""The decode token's cache write fused into the step's first scan
(csa2_write_and_score) against the same two calls made one after the other,
and against the oracle: MXFP4 bytes, indexer cache, scores and block maxima
bit-exact.  Inputs come from csa2_inputs; expected values from oracle/ only.
"""
import numpy as np
import pytest
import torch

import csa2_inputs as ci
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.fail("gpu tests need a GPU")
    import compressed_sparse_attention_05_amd as K
    K.lib()
    return K


def _case(seed, B, cap, D, d_I, xdt):
    codes = torch.randint(0, 256, (B, cap, D // 2), dtype=torch.uint8, generator=torch.Generator().manual_seed(seed))
    scales = torch.randint(0x30, 0x40, (B, cap, D // 16), dtype=torch.uint8,
                           generator=torch.Generator().manual_seed(seed + 1))
    kc = ci.gaussian(seed, ci.TID_K_IDX, (B, cap, d_I), dtype=torch.bfloat16)
    x = ci.gaussian(seed + 7, ci.TID_KV, (B, D), dtype=torch.float32, clip=ci.NORM_BOUND).to(xdt)
    knew = ci.gaussian(seed + 7, ci.TID_K_IDX, (B, d_I), dtype=torch.bfloat16)
    q = ci.gaussian(seed, ci.TID_Q_IDX, (B, 1, 8, d_I), dtype=torch.bfloat16)
    w = ci.uniform(seed, ci.TID_W, (B, 1, 8))
    return codes, scales, kc, x, knew, q, w


@pytest.mark.parametrize("mode,xdt", [("full", torch.bfloat16), ("full", torch.float32), ("pool", torch.bfloat16)])
def test_write_and_score_equals_write_then_score(K, mode, xdt):
    B, cap, D, d_I, P_b = 5, 4096, 512, 128, 64
    ctx = [4096, 1003, 2500, 64, 777]
    codes, scales, kc, x, knew, q, w = _case(41, B, cap, D, d_I, xdt)
    dst = [b * cap + ctx[b] - 1 for b in range(B)]
    dst[3] = -1                      # no write for sequence 3
    dst[4] = 0 * cap + 17            # a row of sequence 0: the fused call skips it
    dst_sep = list(dst)
    dst_sep[4] = -1                  # so the reference writes skip it too
    ctx_t = torch.tensor(ctx, dtype=torch.int32).cuda()
    pool = None
    if mode == "pool":
        pool = torch.full((B, 1, P_b), -1, dtype=torch.int32)
        for b in range(B):
            blocks = sorted({(ctx[b] - 1) // 8, 0, 2, (ctx[b] - 1) // 16} | {(ctx[b] // 8 * j) // 40 for j in range(40)})
            pool[b, 0, :len(blocks)] = torch.tensor(blocks[:P_b], dtype=torch.int32)
        pool = pool.cuda()
    outs = []
    for fused in (True, False):
        c, s, k = codes.clone().cuda(), scales.clone().cuda(), K.tile_indexer_cache(kc.cuda())
        if fused:
            sc, bm = K.csa2_write_and_score(x.cuda(), torch.tensor(dst).cuda(), c, s, knew.cuda(), q.cuda(), w.cuda(),
                                            k, ctx_t, pool_blocks=pool, want_block_max=mode == "full")
        else:
            K.mxfp4_kv_write(x.cuda(), torch.tensor(dst_sep).cuda(), c.view(B * cap, D // 2),
                             s.view(B * cap, D // 16), knew.cuda(), k.view(B * cap, d_I))
            sc, bm = K.csa2_index_score(q.cuda(), w.cuda(), k, ctx_t, pool_blocks=pool,
                                        want_block_max=mode == "full")
        torch.cuda.synchronize()
        outs.append((c.cpu(), s.cpu(), K.untile_indexer_cache(k).cpu(), sc.cpu(), None if bm is None else bm.cpu()))
    (c1, s1, k1, sc1, bm1), (c2, s2, k2, sc2, bm2) = outs
    assert torch.equal(c1, c2) and torch.equal(s1, s2)
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16))
    assert torch.equal(sc1.view(torch.int32), sc2.view(torch.int32))
    if bm1 is not None:
        assert torch.equal(bm1.view(torch.int32), bm2.view(torch.int32))
    # the oracle on the caches as the write leaves them
    want_c, want_s = oracle.mxfp4_encode(x.float() if xdt == torch.float32 else x)
    kc_after = kc.clone()
    for b in range(B):
        d = dst_sep[b]
        if d >= 0:
            assert np.array_equal(c1.view(B * cap, D // 2)[d].numpy(), want_c[b]), b
            assert np.array_equal(s1.view(B * cap, D // 16)[d].numpy(), want_s[b]), b
            kc_after[d // cap, d % cap] = knew[b]
    assert torch.equal(k1.view(torch.int16), kc_after.view(torch.int16))
    for b in range(B):
        if mode == "full":
            want = oracle.full_scores(q[b, 0], w[b, 0], kc_after[b], ctx[b], cap)
            assert np.array_equal(sc1[b, 0].numpy().view(np.uint32), want.view(np.uint32)), b
            wbm = oracle.block_max(want, ctx[b], cap // 8)
            assert np.array_equal(bm1[b, 0].numpy().view(np.uint32), wbm.view(np.uint32)), b
        else:
            want = oracle.pool_scores(q[b, 0], w[b, 0], kc_after[b], ctx[b], pool[b, 0].cpu().numpy())
            assert np.array_equal(sc1[b, 0].numpy().view(np.uint32), want.view(np.uint32)), b
