"""The decode composition (compressed_sparse_attention_05_amd.decode) against
the oracle: one token for two sequences through a Full, a Reindex and a
Reuse layer over one shared cache, with the token's own entry written first.
Pool and index lists bit-exact; each layer's attention within 2e-3."""
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
    return K


@pytest.mark.parametrize("k,P_b,mfma,project,fuse", [(256, 512, False, False, True), (600, 512, False, False, True),
                                                     (256, 512, True, False, True), (256, 512, False, True, True),
                                                     (256, 512, False, False, False)])
def test_decode_step_full_reindex_reuse(K, k, P_b, mfma, project, fuse):
    # k <= P_b: the Full layer's pool and top-k run as one launch (or, with
    # mfma, the matrix-core scan and the band-exact selection);
    # k > P_b: pool, then the Full top-k over the whole row.  With project,
    # the token's indexer key is projected from its latent row by the write.
    # fuse: the write shares the Full scan's launch (csa2_write_and_score)
    # when the step allows it; off, it is a launch of its own.
    from compressed_sparse_attention_05_amd.decode import DecodeCache, DecodeStep, LayerInputs
    dev = torch.device("cuda:0")
    B, cap, D, H, d_I, H_I, W = 2, 20032, 512, 64, 128, 8, 128
    ctx = [20000, 15001]
    swa_len = [128, 50]
    seed = 401
    kv = ci.gaussian(seed, ci.TID_KV, (B, cap, D), clip=ci.NORM_BOUND)
    kidx = ci.gaussian(seed, ci.TID_K_IDX, (B, cap, d_I), dtype=torch.bfloat16)
    codes = torch.zeros((B, cap, D // 2), dtype=torch.uint8, device=dev)
    scales = torch.zeros((B, cap, D // 16), dtype=torch.uint8, device=dev)
    # every entry but the token's own (written by the step)
    rows = torch.cat([torch.arange(b * cap, b * cap + ctx[b] - 1) for b in range(B)]).to(dev)
    flat_kv = kv.reshape(B * cap, D).to(dev)
    K.mxfp4_kv_write(flat_kv[rows], rows, codes, scales)
    kc_rows = kidx.clone()
    for b in range(B):
        kc_rows[b, ctx[b] - 1:] = 0
    kcache = K.tile_indexer_cache(kc_rows.to(dev))
    new_rows = torch.tensor([b * cap + ctx[b] - 1 for b in range(B)], dtype=torch.int64)
    cache = DecodeCache(codes=codes, scales=scales, k_idx=kcache,
                        ctx_len=torch.tensor(ctx, dtype=torch.int32, device=dev),
                        swa_len=torch.tensor(swa_len, dtype=torch.int32, device=dev))
    w_ik = None
    if project:
        w_ik = ci.gaussian(seed, ci.TID_W_IK, (D, d_I)) * np.float32(1.0 / math.sqrt(D))
        for b in range(B):
            bits = oracle.project_kidx(kv[b, ctx[b] - 1:ctx[b]], w_ik)
            kidx[b, ctx[b] - 1] = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16)[0]
    layers = []
    for li in range(3):
        q = ci.gaussian(seed + li, ci.TID_Q, (B, H, D), dtype=torch.bfloat16)
        swa = ci.gaussian(seed + li, ci.TID_SWA, (B, W, D), dtype=torch.bfloat16)
        qi = ci.gaussian(seed + li, ci.TID_Q_IDX, (B, 1, H_I, d_I), dtype=torch.bfloat16)
        wi = ci.uniform(seed + li, ci.TID_W, (B, 1, H_I))
        layers.append((q, swa, qi, wi))
    lin = [LayerInputs(q=q.to(dev), swa=swa.to(dev), q_idx=qi.to(dev), w=wi.to(dev)) for q, swa, qi, wi in layers]
    step = DecodeStep("FXR", cache, lin, k=k, P_b=P_b,
                      new_kv=flat_kv[new_rows.to(dev)].contiguous(),
                      new_kidx=None if project else kidx.reshape(B * cap, d_I)[new_rows].contiguous().to(dev),
                      dst_row=new_rows.to(dev), mfma_select=mfma,
                      w_ik=w_ik.to(dev) if project else None, fuse_write=fuse)
    names = [c[1].__name__ for c in step.calls]
    assert ("csa2_write_and_score" in names) == (fuse and not mfma and not project), names
    step.run()
    torch.cuda.synchronize()
    sm = 1.0 / math.sqrt(D)
    pool = step.pool.cpu().numpy()
    idx_f = step.idx_bufs[0].cpu().numpy()
    idx_x = step.idx_bufs[1].cpu().numpy()
    for b in range(B):
        oc, osc = oracle.mxfp4_encode(kv[b, :ctx[b]])
        q0, s0, qi0, wi0 = layers[0]
        sc = oracle.full_scores(qi0[b, 0], wi0[b, 0], kidx[b], ctx[b], cap)
        opool = oracle.candidate_pool(oracle.block_max(sc, ctx[b], (cap + 7) // 8), P_b)
        assert np.array_equal(pool[b, 0], opool), b
        of = oracle.topk(sc, k)
        assert np.array_equal(idx_f[b, 0], of), b
        q1, s1, qi1, wi1 = layers[1]
        ps = oracle.pool_scores(qi1[b, 0], wi1[b, 0], kidx[b], ctx[b], opool)
        ox = oracle.pool_topk(ps, opool, k)
        assert np.array_equal(idx_x[b, 0], ox), b
        for li, oidx in ((0, of), (1, ox), (2, ox)):
            q, swa = layers[li][0], layers[li][1]
            want = oracle.attn_decode(q[b], oc, osc, oidx, swa[b], swa_len[b], sm)
            err = float(np.max(np.abs(step.outs[li][b].cpu().numpy() - want)))
            assert err < ATOL, (b, li, err)


def test_decode_step_encoder_full_m2(K):
    # schedule F R E R: a decoder Full layer and its Reuse, then an encoder
    # Full layer over its own KV set at m = 2 and a Reuse of it.  Sequence 0's
    # token (position 19,999) completes encoder entry 9,999, written by the
    # step; sequence 1's token (position 15,000) completes none, and its
    # encoder set holds entries past floor((i + 1) / 2) = 7,500 that must stay
    # invisible.
    from compressed_sparse_attention_05_amd.decode import DecodeCache, DecodeStep, LayerInputs
    dev = torch.device("cuda:0")
    B, cap, cap_e, D, H, d_I, H_I, W, k, P_b = 2, 20032, 10048, 512, 64, 128, 8, 128, 256, 512
    ctx = [20000, 15001]
    pos = [19999, 15000]
    ctx_e = [10000, 8000]
    vis_e = [oracle.prefill_vis(pos[b], ctx_e[b], 2) for b in range(B)]
    assert vis_e == [10000, 7500]
    swa_len = [128, 90]
    seed = 433
    kv = ci.gaussian(seed, ci.TID_KV, (B, cap, D), clip=ci.NORM_BOUND)
    kidx = ci.gaussian(seed, ci.TID_K_IDX, (B, cap, d_I), dtype=torch.bfloat16)
    kv_e = ci.gaussian(seed + 50, ci.TID_KV, (B, cap_e, D), clip=ci.NORM_BOUND)
    kidx_e = ci.gaussian(seed + 50, ci.TID_K_IDX, (B, cap_e, d_I), dtype=torch.bfloat16)

    def make_cache(kv_, kidx_, cap_, n_rows, skip):
        codes = torch.zeros((B, cap_, D // 2), dtype=torch.uint8, device=dev)
        scales = torch.zeros((B, cap_, D // 16), dtype=torch.uint8, device=dev)
        rows = torch.cat([torch.tensor([b * cap_ + r for r in range(n_rows[b]) if (b, r) not in skip],
                                       dtype=torch.int64) for b in range(B)]).to(dev)
        flat = kv_.reshape(B * cap_, D).to(dev)
        K.mxfp4_kv_write(flat[rows], rows, codes, scales)
        krows = kidx_.clone()
        for b in range(B):
            krows[b, n_rows[b]:] = 0
        for (b, r) in skip:
            krows[b, r] = 0
        return codes, scales, K.tile_indexer_cache(krows.to(dev)), flat

    dec_new = [(0, ctx[0] - 1), (1, ctx[1] - 1)]
    enc_new = [(0, ctx_e[0] - 1)]
    codes, scales, kcache, flat_kv = make_cache(kv, kidx, cap, ctx, set(dec_new))
    codes_e, scales_e, kcache_e, flat_kv_e = make_cache(kv_e, kidx_e, cap_e, ctx_e, set(enc_new))
    sl = torch.tensor(swa_len, dtype=torch.int32, device=dev)
    cache = DecodeCache(codes=codes, scales=scales, k_idx=kcache,
                        ctx_len=torch.tensor(ctx, dtype=torch.int32, device=dev), swa_len=sl)
    ecache = DecodeCache(codes=codes_e, scales=scales_e, k_idx=kcache_e,
                         ctx_len=torch.tensor(ctx_e, dtype=torch.int32, device=dev), swa_len=sl)
    layers = []
    for li in range(4):
        q = ci.gaussian(seed + li, ci.TID_Q, (B, H, D), dtype=torch.bfloat16)
        swa = ci.gaussian(seed + li, ci.TID_SWA, (B, W, D), dtype=torch.bfloat16)
        qi = ci.gaussian(seed + li, ci.TID_Q_IDX, (B, 1, H_I, d_I), dtype=torch.bfloat16)
        wi = ci.uniform(seed + li, ci.TID_W, (B, 1, H_I))
        layers.append((q, swa, qi, wi))
    lin = [LayerInputs(q=q.to(dev), swa=swa.to(dev), q_idx=qi.to(dev), w=wi.to(dev)) for q, swa, qi, wi in layers]
    d_rows = torch.tensor([b * cap + r for b, r in dec_new], dtype=torch.int64)
    e_rows = torch.tensor([b * cap_e + r for b, r in enc_new], dtype=torch.int64)
    step = DecodeStep("FRER", cache, lin, k=k, P_b=P_b,
                      new_kv=flat_kv[d_rows.to(dev)].contiguous(),
                      new_kidx=kidx.reshape(B * cap, d_I)[d_rows].contiguous().to(dev), dst_row=d_rows.to(dev),
                      enc_caches=[ecache], enc_q_pos=torch.tensor(pos, dtype=torch.int64, device=dev),
                      enc_writes=[(flat_kv_e[e_rows.to(dev)].contiguous(),
                                   kidx_e.reshape(B * cap_e, d_I)[e_rows].contiguous().to(dev), e_rows.to(dev))])
    step.run()
    torch.cuda.synchronize()
    sm = 1.0 / math.sqrt(D)
    idx_f = step.idx_bufs[0].cpu().numpy()
    idx_e = step.idx_bufs[1].cpu().numpy()
    for b in range(B):
        q0, s0, qi0, wi0 = layers[0]
        sc = oracle.full_scores(qi0[b, 0], wi0[b, 0], kidx[b], ctx[b], cap)
        of = oracle.topk(sc, k)
        assert np.array_equal(idx_f[b, 0], of), b
        q2, s2, qi2, wi2 = layers[2]
        sce = oracle.full_scores(qi2[b, 0], wi2[b, 0], kidx_e[b], vis_e[b], cap_e)
        oe = oracle.topk(sce, k)
        assert np.array_equal(idx_e[b, 0], oe), b
        assert oe.max() < vis_e[b]
        oc, osc = oracle.mxfp4_encode(kv[b, :ctx[b]])
        oce, osce = oracle.mxfp4_encode(kv_e[b, :vis_e[b]])
        for li, oidx, (c_, s_) in ((0, of, (oc, osc)), (1, of, (oc, osc)), (2, oe, (oce, osce)), (3, oe, (oce, osce))):
            q, swa = layers[li][0], layers[li][1]
            want = oracle.attn_decode(q[b], c_, s_, oidx, swa[b], swa_len[b], sm)
            err = float(np.max(np.abs(step.outs[li][b].cpu().numpy() - want)))
            assert err < ATOL, (b, li, err)


@pytest.mark.parametrize("schedule,pass_pool", [("FRFX", False), ("FR", True)])
def test_later_full_layer_selects_over_whole_context(K, schedule, pass_pool):
    # A Full layer scores every visible entry ("...KV Cache Compression"
    # notes, section 2); only its own block maxima bound where its top-k can
    # lie.  FRFX: the second F must select over the whole context, and X
    # rescores the pool of the first F.  FR with a pool passed in: that pool
    # says nothing about this layer's scores, so F selects over the whole
    # context too.  The per-sequence pool passed in is a block range that
    # misses most of the true top-k, so a pool-restricted top-k would fail.
    from compressed_sparse_attention_05_amd.decode import DecodeCache, DecodeStep, LayerInputs
    dev = torch.device("cuda:0")
    B, cap, D, H, d_I, H_I, W, k, P_b = 2, 12032, 512, 64, 128, 8, 128, 256, 512
    ctx = [12000, 9001]
    swa_len = [128, 77]
    seed = 471
    kv = ci.gaussian(seed, ci.TID_KV, (B, cap, D), clip=ci.NORM_BOUND)
    kidx = ci.gaussian(seed, ci.TID_K_IDX, (B, cap, d_I), dtype=torch.bfloat16)
    for b in range(B):
        kidx[b, ctx[b]:] = 0
    codes = torch.zeros((B, cap, D // 2), dtype=torch.uint8, device=dev)
    scales = torch.zeros((B, cap, D // 16), dtype=torch.uint8, device=dev)
    rows = torch.cat([torch.arange(b * cap, b * cap + ctx[b]) for b in range(B)]).to(dev)
    K.mxfp4_kv_write(kv.reshape(B * cap, D).to(dev)[rows], rows, codes, scales)
    cache = DecodeCache(codes=codes, scales=scales, k_idx=K.tile_indexer_cache(kidx.to(dev)),
                        ctx_len=torch.tensor(ctx, dtype=torch.int32, device=dev),
                        swa_len=torch.tensor(swa_len, dtype=torch.int32, device=dev))
    layers = []
    for li in range(len(schedule)):
        q = ci.gaussian(seed + li, ci.TID_Q, (B, H, D), dtype=torch.bfloat16)
        swa = ci.gaussian(seed + li, ci.TID_SWA, (B, W, D), dtype=torch.bfloat16)
        qi = ci.gaussian(seed + li, ci.TID_Q_IDX, (B, 1, H_I, d_I), dtype=torch.bfloat16)
        wi = ci.uniform(seed + li, ci.TID_W, (B, 1, H_I))
        layers.append((q, swa, qi, wi))
    lin = [LayerInputs(q=q.to(dev), swa=swa.to(dev), q_idx=qi.to(dev), w=wi.to(dev)) for q, swa, qi, wi in layers]
    given = None
    if pass_pool:
        given = torch.arange(P_b, dtype=torch.int32).repeat(B, 1).reshape(B, 1, P_b).contiguous()
    step = DecodeStep(schedule, cache, lin, k=k, P_b=P_b,
                      pool=given.to(dev) if given is not None else None)
    step.run()
    torch.cuda.synchronize()
    sm = 1.0 / math.sqrt(D)
    for b in range(B):
        oc, osc = oracle.mxfp4_encode(kv[b, :ctx[b]])
        want_idx = []
        pool = None
        for li, mode in enumerate(schedule):
            q, swa, qi, wi = layers[li]
            if mode == "F":
                sc = oracle.full_scores(qi[b, 0], wi[b, 0], kidx[b], ctx[b], cap)
                if pool is None and not pass_pool:
                    pool = oracle.candidate_pool(oracle.block_max(sc, ctx[b], (cap + 7) // 8), P_b)
                cur = oracle.topk(sc, k)
                want_idx.append(cur)
                if pass_pool:
                    # the passed pool really does miss part of this top-k
                    assert (cur >= 8 * P_b).any()
            elif mode == "X":
                ps = oracle.pool_scores(qi[b, 0], wi[b, 0], kidx[b], ctx[b], pool)
                cur = oracle.pool_topk(ps, pool, k)
                want_idx.append(cur)
            want = oracle.attn_decode(q[b], oc, osc, cur, swa[b], swa_len[b], sm)
            err = float(np.max(np.abs(step.outs[li][b].cpu().numpy() - want)))
            assert err < ATOL, (b, li, err)
        for i, wi_ in enumerate(want_idx):
            assert np.array_equal(step.idx_bufs[i][b, 0].cpu().numpy(), wi_), (b, i)
        if not pass_pool:
            assert np.array_equal(step.pool[b, 0].cpu().numpy(), pool), b


def test_reindex_over_padded_pool_and_full_identity(K):
    # Short contexts, where the pool is nearly the whole sequence ("...KV Cache
    # Compression" notes, section 3) and holds fewer than P_b blocks, so its
    # tail is -1 ("up to 16,384 positions", summary page, Methodology item 3).
    # Sequence 0: 4,096 entries = 512 whole blocks.  Sequence 1: 1,003 entries,
    # whose last block holds 3 visible positions.  Schedule F X X R: the first
    # X reuses the Full layer's own (q, w), so it must return the Full top-k
    # (the Full top-k lies inside the pool); the second X has its own query.
    from compressed_sparse_attention_05_amd.decode import DecodeCache, DecodeStep, LayerInputs
    dev = torch.device("cuda:0")
    B, cap, D, H, d_I, H_I, W, k, P_b = 2, 4096, 512, 64, 128, 8, 128, 2048, 2048
    ctx = [4096, 1003]
    swa_len = [128, 128]
    seed = 487
    kv = ci.gaussian(seed, ci.TID_KV, (B, cap, D), clip=ci.NORM_BOUND)
    kidx = ci.gaussian(seed, ci.TID_K_IDX, (B, cap, d_I), dtype=torch.bfloat16)
    for b in range(B):
        kidx[b, ctx[b]:] = 0
    codes = torch.zeros((B, cap, D // 2), dtype=torch.uint8, device=dev)
    scales = torch.zeros((B, cap, D // 16), dtype=torch.uint8, device=dev)
    rows = torch.cat([torch.arange(b * cap, b * cap + ctx[b]) for b in range(B)]).to(dev)
    K.mxfp4_kv_write(kv.reshape(B * cap, D).to(dev)[rows], rows, codes, scales)
    cache = DecodeCache(codes=codes, scales=scales, k_idx=K.tile_indexer_cache(kidx.to(dev)),
                        ctx_len=torch.tensor(ctx, dtype=torch.int32, device=dev),
                        swa_len=torch.tensor(swa_len, dtype=torch.int32, device=dev))
    layers = []
    for li in range(4):
        q = ci.gaussian(seed + li, ci.TID_Q, (B, H, D), dtype=torch.bfloat16)
        swa = ci.gaussian(seed + li, ci.TID_SWA, (B, W, D), dtype=torch.bfloat16)
        src = 0 if li == 1 else li
        qi = ci.gaussian(seed + src, ci.TID_Q_IDX, (B, 1, H_I, d_I), dtype=torch.bfloat16)
        wi = ci.uniform(seed + src, ci.TID_W, (B, 1, H_I))
        layers.append((q, swa, qi, wi))
    lin = [LayerInputs(q=q.to(dev), swa=swa.to(dev), q_idx=qi.to(dev), w=wi.to(dev)) for q, swa, qi, wi in layers]
    step = DecodeStep("FXXR", cache, lin, k=k, P_b=P_b)
    step.run()
    torch.cuda.synchronize()
    sm = 1.0 / math.sqrt(D)
    for b in range(B):
        oc, osc = oracle.mxfp4_encode(kv[b, :ctx[b]])
        _, _, qi0, wi0 = layers[0]
        sc = oracle.full_scores(qi0[b, 0], wi0[b, 0], kidx[b], ctx[b], cap)
        n_blocks = (ctx[b] + 7) // 8
        opool = oracle.candidate_pool(oracle.block_max(sc, ctx[b], cap // 8), P_b)
        assert np.array_equal(opool[:n_blocks], np.arange(n_blocks)) and (opool[n_blocks:] == -1).all()
        assert np.array_equal(step.pool[b, 0].cpu().numpy(), opool), b
        of = oracle.topk(sc, k)
        got_f = step.idx_bufs[0][b, 0].cpu().numpy()
        assert np.array_equal(got_f, of), b
        # Reindex with the Full layer's own query: the Full top-k again
        got_x1 = step.idx_bufs[1][b, 0].cpu().numpy()
        assert np.array_equal(got_x1, got_f), b
        _, _, qi2, wi2 = layers[2]
        ps = oracle.pool_scores(qi2[b, 0], wi2[b, 0], kidx[b], ctx[b], opool)
        ox = oracle.pool_topk(ps, opool, k)
        assert np.array_equal(step.idx_bufs[2][b, 0].cpu().numpy(), ox), b
        if ctx[b] < k:
            assert np.array_equal(ox[:ctx[b]], np.arange(ctx[b])) and (ox[ctx[b]:] == -1).all()
        for li, oidx in ((0, of), (1, of), (2, ox), (3, ox)):
            q, swa = layers[li][0], layers[li][1]
            want = oracle.attn_decode(q[b], oc, osc, oidx, swa[b], swa_len[b], sm)
            err = float(np.max(np.abs(step.outs[li][b].cpu().numpy() - want)))
            assert err < ATOL, (b, li, err)
