"""Prefill Full-mode top-k (matrix-core scores with an exact error band)
against the oracle: the oracle's exact fma-chain scores and full-sort top-k
must be reproduced index for index."""
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


def _inputs(seed, T, cap):
    q = ci.gaussian(seed, ci.TID_Q_IDX, (T, 8, 128), torch.bfloat16)
    w = ci.uniform(seed, ci.TID_W, (T, 8))
    kc = ci.gaussian(seed, ci.TID_K_IDX, (cap, 128), torch.bfloat16)
    return q, w, kc


def _run(K, q, w, kc, ctx, q_pos0, m, k):
    tiled = K.tile_indexer_cache(kc.cuda()[None])[0]
    return K.csa2_prefill_topk(q.cuda(), w.cuda(), tiled, ctx, q_pos0, m, k).cpu().numpy()


def _check_rows(got, q, w, kc, ctx, q_pos0, m, k, rows):
    rows = np.asarray(rows)
    sc = oracle.prefill_scores(q[rows], w[rows], kc, q_pos0 + rows, ctx, m, kc.shape[0])
    for i, t in enumerate(rows):
        want = oracle.topk(sc[i], k)
        assert np.array_equal(got[t], want), f"row {t}"


@pytest.mark.parametrize("k", [512, 2048])
def test_prefill_topk_matches_exact_chain(K, k):
    T, cap, m = 96, 8192, 2
    q_pos0 = 2 * cap - 48
    q, w, kc = _inputs(2001, T, cap)
    print(f"prefill topk T={T} cap={cap} k={k}", flush=True)
    got = _run(K, q, w, kc, cap, q_pos0, m, k)
    _check_rows(got, q, w, kc, cap, q_pos0, m, k, range(T))


def test_prefill_topk_rows_shorter_than_k(K):
    # vis(t) runs from 450 to 600 across the chunk: rows at or below k take
    # every visible entry, the others select
    T, cap, m, k = 300, 4096, 2, 512
    q_pos0 = 899
    q, w, kc = _inputs(2002, T, cap)
    got = _run(K, q, w, kc, cap, q_pos0, m, k)
    _check_rows(got, q, w, kc, cap, q_pos0, m, k, range(T))


def test_prefill_topk_exactly_summable_ties(K):
    # multiples of 2^-3 in [-4, 4]: the matrix cores are exact too, and many
    # keys tie at the k-th score, so the tie rule decides
    T, cap, m, k = 64, 4096, 1, 256
    g = torch.Generator().manual_seed(11)
    q = (torch.randint(-32, 33, (T, 8, 128), generator=g) / 8.0).to(torch.bfloat16)
    kc = (torch.randint(-4, 5, (cap, 128), generator=g) / 8.0).to(torch.bfloat16)
    w = (torch.randint(0, 4, (T, 8), generator=g) / 4.0).float()
    q_pos0 = cap - T
    got = _run(K, q, w, kc, cap, q_pos0, m, k)
    _check_rows(got, q, w, kc, cap, q_pos0, m, k, range(T))


def test_prefill_topk_all_keys_equal_uses_exact_fallback(K):
    # every score of a row is equal: the band holds the whole row, more than
    # the rescoring buffer, so the row is redone exactly; ties -> 0..k-1
    T, cap, m, k = 8, 4096, 1, 100
    q, w, _ = _inputs(2003, T, cap)
    kc = ci.gaussian(2003, ci.TID_K_IDX, (1, 128), torch.bfloat16).repeat(cap, 1)
    got = _run(K, q, w, kc, cap, cap - T, m, k)
    _check_rows(got, q, w, kc, cap, cap - T, m, k, range(T))
    assert np.array_equal(got[0], np.arange(k))


def test_prefill_topk_full_chunk_sampled(K):
    # the 8,192-token chunk at positions 262,144.. over 135,168 entries (m=2),
    # k=2048, as the benchmark runs it; sampled rows against the oracle
    w_ = ci.PREFILL_CHUNK
    T, N, m, k = w_.T, w_.N, w_.m, w_.k
    q_pos0 = w_.prior_tokens
    q, w, kc = _inputs(w_.seed, T, N)
    print(f"prefill chunk T={T} N={N}", flush=True)
    got = _run(K, q, w, kc, N, q_pos0, m, k)
    rng = np.random.default_rng(3)
    rows = sorted(set([0, 1, 2047, 4096, T - 1] + list(rng.integers(0, T, 5))))
    _check_rows(got, q, w, kc, N, q_pos0, m, k, rows)


# Rows with more than 12,288 visible entries take the sampled threshold:
# one 32-key block per 512 keys is scored first, the row's candidates are
# the keys at or above a sample quantile, and the final pass checks that
# they cover the band around the k-th score.
@pytest.mark.parametrize("k,T", [(512, 64), (2048, 64), (2048, 13)])
def test_prefill_topk_sampled_threshold(K, k, T):
    # T = 13: the last block of 8 query rows has 3 rows past the chunk,
    # whose sample stores must be dropped
    cap, m = 40960, 2
    q_pos0 = 2 * cap - 2 * T          # vis(t) runs from cap - T to cap
    q, w, kc = _inputs(2004, T, cap)
    print(f"prefill topk sampled T={T} cap={cap} k={k}", flush=True)
    got = _run(K, q, w, kc, cap, q_pos0, m, k)
    _check_rows(got, q, w, kc, cap, q_pos0, m, k, range(T))


def test_prefill_topk_sampled_ragged_context(K):
    # ctx_len 20,000 is not a multiple of the 512-key sample group or of the
    # 4,096-key candidate workgroup: the last group and workgroup are partial
    T, cap, m, k = 40, 20480, 1, 1000
    ctx = 20000
    q_pos0 = 30000
    q, w, kc = _inputs(2005, T, cap)
    got = _run(K, q, w, kc, ctx, q_pos0, m, k)
    _check_rows(got, q, w, kc, ctx, q_pos0, m, k, range(T))


def test_prefill_topk_long_sample_row(K):
    # 266,240 visible entries give 16,640 sampled keys per row, more than the
    # threshold kernel holds in registers: it selects from the workspace
    T, cap, m, k = 4, 266240, 1, 2048
    q_pos0 = cap - T                  # vis(t) runs from cap - 3 to cap
    q, w, kc = _inputs(2008, T, cap)
    print(f"prefill topk long sample T={T} cap={cap} k={k}", flush=True)
    got = _run(K, q, w, kc, cap, q_pos0, m, k)
    _check_rows(got, q, w, kc, cap, q_pos0, m, k, range(T))


def test_prefill_topk_too_many_candidates_falls_back(K):
    # every key equal with 20,480 visible: the sample quantile equals every
    # score, all keys become candidates (more than the 12,288 staged), and
    # the row is redone exactly; ties -> positions 0..k-1
    T, cap, m, k = 4, 20480, 1, 300
    q, w, _ = _inputs(2006, T, cap)
    kc = ci.gaussian(2006, ci.TID_K_IDX, (1, 128), torch.bfloat16).repeat(cap, 1)
    got = _run(K, q, w, kc, cap, cap - T, m, k)
    _check_rows(got, q, w, kc, cap, cap - T, m, k, range(T))
    assert np.array_equal(got[0], np.arange(k))


def test_prefill_topk_misleading_sample_falls_back(K):
    # Only the sampled 32-key blocks hold nonzero keys (the block of 256-key
    # group g is 8g + (g * 0x9E3779B1 mod 2^32) >> 29); every other key
    # scores exactly 0.  The sample then sees only the high scores, its
    # quantile sits above the row's k-th score, too few keys qualify, and the
    # exact fallback must still give the definition's top-k (the high keys,
    # then the zero-score keys by position).
    T, cap, m, k = 8, 20480, 1, 2048
    q, w, kc = _inputs(2007, T, cap)
    keep = torch.zeros(cap, dtype=torch.bool)
    for g in range(cap // 256):
        h = ((g * 0x9E3779B1) & 0xFFFFFFFF) >> 29
        keep[256 * g + 32 * h: 256 * g + 32 * h + 32] = True
    kc = torch.where(keep[:, None], kc, torch.zeros_like(kc))
    got = _run(K, q, w, kc, cap, cap - T, m, k)
    _check_rows(got, q, w, kc, cap, cap - T, m, k, range(T))
