"""The prefill chunk composition (compressed_sparse_attention_05_amd.prefill)
end to end against the oracle: one encoder block, schedule F R R R R R
("DeepSeek-V4.1-Flash KV Cache Compression" notes, section 2: the encoder's
Full layer selects per token, its Reuse layers attend with the same indices),
at m = 2 tokens per entry.

The chunk writes its own complete entries first, so later tokens of the chunk
see them (causal visibility vis(t) = min(ctx_len, floor((q_pos0 + t + 1) / m))).
Every token's index list bit-exact; every layer's output within 2e-3 on
sampled tokens (a float64 oracle over all 520 x 6 queries takes minutes)."""
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


def test_prefill_chunk_every_layer_against_oracle(K):
    from compressed_sparse_attention_05_amd.prefill import PrefillChunk, PrefillLayer
    dev = torch.device("cuda:0")
    schedule = "FRRRRR"
    T, m, D, H, d_I, H_I, W, k = 520, 2, 512, 64, 128, 8, 128, 512
    prior_tokens = 6000
    n_prior = prior_tokens // m               # 3,000 entries before the chunk
    N = n_prior + T // m                      # 3,260 entries once the chunk is written
    cap = 3328                                # multiple of 64; rows past N stay invisible
    seed = 1404
    print(f"prefill chunk {schedule} T={T} entries={N} m={m} k={k}", flush=True)
    kv = ci.gaussian(seed, ci.TID_KV, (cap, D), dtype=torch.bfloat16, clip=ci.NORM_BOUND)
    kidx = ci.gaussian(seed, ci.TID_K_IDX, (cap, d_I), dtype=torch.bfloat16)
    kidx[N:] = 0
    codes = torch.zeros((cap, D // 2), dtype=torch.uint8, device=dev)
    scales = torch.zeros((cap, D // 16), dtype=torch.uint8, device=dev)
    prior = torch.arange(n_prior, dtype=torch.int64, device=dev)
    K.mxfp4_kv_write(kv[:n_prior].to(dev), prior, codes, scales)
    krows = kidx.clone()
    krows[n_prior:] = 0                       # the chunk writes its own indexer rows
    k_tiled = K.tile_indexer_cache(krows.to(dev)[None])[0]
    dst = torch.arange(n_prior, N, dtype=torch.int64, device=dev)
    layers, host = [], []
    for li, mode in enumerate(schedule):
        q = ci.gaussian(seed, ci.layer_tid(ci.TID_Q, li), (T, H, D), torch.bfloat16)
        swa = ci.gaussian(seed, ci.layer_tid(ci.TID_SWA, li), (T + W - 1, D), torch.bfloat16)
        lay = PrefillLayer(q=q.to(dev), swa=swa.to(dev))
        qi = wi = None
        if mode == "F":
            qi = ci.gaussian(seed, ci.layer_tid(ci.TID_Q_IDX, li), (T, H_I, d_I), torch.bfloat16)
            wi = ci.uniform(seed, ci.layer_tid(ci.TID_W, li), (T, H_I))
            lay.q_idx, lay.w = qi.to(dev), wi.to(dev)
        layers.append(lay)
        host.append((q, swa, qi, wi))
    chunk = PrefillChunk(schedule, codes, scales, k_tiled, N, prior_tokens, m, k, W, layers,
                         new_kv=kv[n_prior:N].to(dev), new_kidx=kidx[n_prior:N].to(dev), dst_row=dst)
    chunk.run()
    torch.cuda.synchronize()
    assert len({o.data_ptr() for o in chunk.outs}) == len(schedule)

    # MXFP4 bytes of the entries the chunk wrote, then the index lists
    oc, osc = oracle.mxfp4_encode(kv[:N])
    assert np.array_equal(codes[:N].cpu().numpy(), oc)
    assert np.array_equal(scales[:N].cpu().numpy(), osc)
    q0, _, qi0, wi0 = host[0]
    q_pos = prior_tokens + np.arange(T, dtype=np.int64)
    sc = oracle.prefill_scores(qi0, wi0, kidx[:N], q_pos, N, m, N)
    got_idx = chunk.idx.cpu().numpy()
    want_idx = np.stack([oracle.topk(sc[t], k) for t in range(T)])
    assert np.array_equal(got_idx, want_idx)
    # the last token sees the chunk's own entries
    assert want_idx[-1].max() >= n_prior

    sm = 1.0 / math.sqrt(D)
    errs = []
    for t in (0, 1, 129, 300, T - 1):
        for li in range(len(schedule)):
            q, swa = host[li][0], host[li][1]
            want = oracle.attn_prefill(q[t:t + 1], oc, osc, want_idx[t:t + 1], swa[t:t + W], W,
                                       prior_tokens + t, 0, sm)
            got = chunk.outs[li][t].cpu().numpy()
            err = float(np.max(np.abs(got - want[0])))
            errs.append(err)
            assert err < ATOL, (t, li, err)
    # the layers' outputs differ (each has its own queries and window)
    assert not torch.equal(chunk.outs[0], chunk.outs[1])
    print("max err %.2e" % max(errs), flush=True)
