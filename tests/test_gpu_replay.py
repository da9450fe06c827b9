"""The decoder over a replayed window (compressed_sparse_attention_05_amd.replay)
against the oracle: T replayed tokens of one sequence, each a decoder query
with its own candidate pool, through a Full, a Reuse, a Reindex and a Reuse
layer.  Windows are cut at the replay start ("DeepSeek-V4.1-Flash KV Cache
Compression" notes, section 5).  Pools and index lists bit-exact; attention
within 2e-3."""
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


@pytest.mark.parametrize("T,ctx,q_pos0", [(40, 20000, 19960), (130, 9000, 8700)])
def test_decoder_replay_matches_oracle(K, T, ctx, q_pos0):
    # (40, ...): the replay ends at the newest entry; (130, ...): a segment in
    # the middle of a longer cache, so entries past each token stay invisible,
    # and T > W, so late tokens see a full window
    from compressed_sparse_attention_05_amd.replay import DecoderReplay, ReplayLayer
    dev = torch.device("cuda:0")
    cap, D, H, d_I, H_I, W, k, P_b = 20032, 512, 64, 128, 8, 128, 256, 512
    seed = 509 + T
    kv = ci.gaussian(seed, ci.TID_KV, (cap, D), clip=ci.NORM_BOUND)
    kidx = ci.gaussian(seed, ci.TID_K_IDX, (cap, d_I), dtype=torch.bfloat16)
    kidx[ctx:] = 0
    codes = torch.zeros((cap, D // 2), dtype=torch.uint8, device=dev)
    scales = torch.zeros((cap, D // 16), dtype=torch.uint8, device=dev)
    rows = torch.arange(ctx, dtype=torch.int64, device=dev)
    K.mxfp4_kv_write(kv[:ctx].to(dev), rows, codes.view(1, cap, D // 2), scales.view(1, cap, D // 16))
    kcache = K.tile_indexer_cache(kidx.reshape(1, cap, d_I).to(dev))[0]
    schedule = "FRXR"
    layers = []
    for li, mode in enumerate(schedule):
        q = ci.gaussian(seed + li, ci.TID_Q, (T, H, D), dtype=torch.bfloat16)
        swa = ci.gaussian(seed + li, ci.TID_SWA, (T + W - 1, D), dtype=torch.bfloat16)
        qi = ci.gaussian(seed + li, ci.TID_Q_IDX, (T, H_I, d_I), dtype=torch.bfloat16) if mode in "FX" else None
        wi = ci.uniform(seed + li, ci.TID_W, (T, H_I)) if mode in "FX" else None
        layers.append((q, swa, qi, wi))
    lin = [ReplayLayer(q=q.to(dev), swa=swa.to(dev), q_idx=None if qi is None else qi.to(dev),
                       w=None if wi is None else wi.to(dev)) for q, swa, qi, wi in layers]
    rp = DecoderReplay(schedule, codes, scales, kcache, ctx, q_pos0, k, W, lin, P_b=P_b)
    rp.run()
    torch.cuda.synchronize()

    nb = (cap + 7) // 8
    pos = q_pos0 + np.arange(T, dtype=np.int64)
    qF, qX = layers[0], layers[2]
    sc = oracle.prefill_scores(qF[2], qF[3], kidx, pos, ctx, 1, cap)
    pool_g = rp.pool.cpu().numpy()
    idx_f = rp.idx[0].cpu().numpy()
    idx_x = rp.idx[2].cpu().numpy()
    want_f = np.empty((T, k), np.int32)
    want_x = np.empty((T, k), np.int32)
    for t in range(T):
        vis = oracle.prefill_vis(int(pos[t]), ctx, 1)
        assert vis == min(ctx, int(pos[t]) + 1)
        opool = oracle.candidate_pool(oracle.block_max(sc[t], vis, nb), P_b)
        assert np.array_equal(pool_g[t], opool), t
        want_f[t] = oracle.topk(sc[t], k)
        assert np.array_equal(idx_f[t], want_f[t]), t
        ps = oracle.pool_scores(qX[2][t], qX[3][t], kidx, vis, opool)
        want_x[t] = oracle.pool_topk(ps, opool, k)
        assert np.array_equal(idx_x[t], want_x[t]), t
    oc, osc = oracle.mxfp4_encode(kv[:ctx])
    sm = 1.0 / math.sqrt(D)
    for li, oidx in ((0, want_f), (1, want_f), (2, want_x), (3, want_x)):
        q, swa = layers[li][0], layers[li][1]
        want = oracle.attn_prefill(q, oc, osc, oidx, swa, W, q_pos0, q_pos0, sm)
        err = float(np.max(np.abs(rp.out[li].cpu().numpy() - want)))
        assert err < ATOL, (li, err)
