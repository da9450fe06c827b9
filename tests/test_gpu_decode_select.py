"""csa2_decode_scan + csa2_decode_select (matrix-core scores, exact bands)
against the oracle's exact scores, block maxima, pool and top-k: pool and
indices bit-exact."""
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


def _run(K, q, w, kc, ctx, P_b, k):
    dev = torch.device("cuda:0")
    tiled = K.tile_indexer_cache(kc.to(dev))
    pool, idx = K.csa2_decode_select(q.to(dev), w.to(dev), tiled, torch.tensor(ctx, dtype=torch.int32, device=dev),
                                     P_b, k)
    return pool.cpu().numpy(), idx.cpu().numpy()


def _check(pool, idx, q, w, kc, ctx, P_b, k, rows=None):
    B, cap = kc.shape[0], kc.shape[1]
    for b in (range(B) if rows is None else rows):
        sc = oracle.full_scores(q[b], w[b], kc[b], ctx[b], cap)
        opool = oracle.candidate_pool(oracle.block_max(sc, ctx[b], cap // 8), P_b)
        assert np.array_equal(pool[b], opool), ("pool", b)
        assert np.array_equal(idx[b], oracle.topk(sc, k)), ("topk", b)


@pytest.mark.parametrize("k,P_b", [(2048, 2048), (100, 256)])
def test_decode_select_random_ragged(K, k, P_b):
    B, cap = 4, 20032
    ctx = [20000, 15001, 1500, 64]                    # long, ragged, fewer blocks than P_b, fewer than k
    q = ci.gaussian(601, ci.TID_Q_IDX, (B, 8, 128), dtype=torch.bfloat16)
    w = ci.uniform(601, ci.TID_W, (B, 8))
    kc = ci.gaussian(601, ci.TID_K_IDX, (B, cap, 128), dtype=torch.bfloat16)
    pool, idx = _run(K, q, w, kc, ctx, P_b, k)
    _check(pool, idx, q, w, kc, ctx, P_b, k)


def test_decode_select_exact_ties(K):
    # multiples of 2^-3 in [-4, 4] and weights in quarters: the matrix cores
    # are exact too, and many keys tie at both thresholds
    B, cap, P_b, k = 2, 8192, 256, 200
    g = torch.Generator().manual_seed(12)
    q = (torch.randint(-32, 33, (B, 8, 128), generator=g) / 8.0).to(torch.bfloat16)
    kc = (torch.randint(-4, 5, (B, cap, 128), generator=g) / 8.0).to(torch.bfloat16)
    w = (torch.randint(0, 4, (B, 8), generator=g) / 4.0).float()
    ctx = [cap, cap - 77]
    pool, idx = _run(K, q, w, kc, ctx, P_b, k)
    _check(pool, idx, q, w, kc, ctx, P_b, k)


def test_decode_select_all_keys_equal_falls_back(K):
    # every score equal: both bands hold everything, beyond the on-chip
    # budget, so rows are redone from exact scores; ties -> lowest ids
    B, cap, P_b, k = 2, 16384, 1024, 300
    q = ci.gaussian(602, ci.TID_Q_IDX, (B, 8, 128), dtype=torch.bfloat16)
    w = ci.uniform(602, ci.TID_W, (B, 8))
    kc = ci.gaussian(602, ci.TID_K_IDX, (1, 1, 128), dtype=torch.bfloat16).repeat(B, cap, 1)
    ctx = [cap, cap - 5]
    pool, idx = _run(K, q, w, kc, ctx, P_b, k)
    _check(pool, idx, q, w, kc, ctx, P_b, k)
    assert np.array_equal(pool[0], np.arange(P_b)) and np.array_equal(idx[0], np.arange(k))


def test_decode_select_headline_rows_sampled(K):
    # 8 sequences x 131,072 entries, P_b = k = 2,048, as the benchmark runs it
    B, cap, P_b, k = 8, 131072, 2048, 2048
    q = ci.gaussian(603, ci.TID_Q_IDX, (B, 8, 128), dtype=torch.bfloat16)
    w = ci.uniform(603, ci.TID_W, (B, 8))
    kc = ci.gaussian(603, ci.TID_K_IDX, (B, cap, 128), dtype=torch.bfloat16)
    ctx = [cap] * 7 + [cap - 4099]
    pool, idx = _run(K, q, w, kc, ctx, P_b, k)
    _check(pool, idx, q, w, kc, ctx, P_b, k, rows=[0, 7])
