"""The decode steps the benchmark times, at the benchmark's own shapes and in
its own launch configuration (bench.InputSet and bench.make_step build them),
against the oracle.

decode-full-128k-b8: one Full layer for 8 sequences of 131,072 entries (the
scan, the fused pool/top-k over 16,384 blocks, and the split attention
kernel).  All 8 pools and index lists bit-exact; attention within 2e-3 on two
sequences.

decode-20layer-1M-b64: the decoder's 20 layers (F R R R, then 4 x X R R R)
for 64 sequences of 1,048,576 entries (pool built through super-blocks, the
warp-specialised attention plan at 64 units, per-sequence cache offsets of
up to 36 GB).  Sequences 0 and 63 sampled: the pool, the Full and every
Reindex index list bit-exact, attention of layers 0, 4 and 19 within 2e-3.

Inputs come from csa2_inputs (the same seeded generator on either side);
expected values only from oracle/.
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
    return K


def _kidx_rows(seed, b, cap, d_I, dev):
    """Row-major indexer keys of sequence b as float32 on the host (the
    generator's values, computed on the device for speed)."""
    rows = torch.empty((cap, d_I), dtype=torch.bfloat16, device=dev)
    ci.fill_gaussian_(rows, seed, ci.TID_K_IDX, first=b * cap * d_I)
    return oracle.as_f32(rows.cpu())


def _attn_ref(w, seed, b, cap, q, swa, swa_len, idx):
    """Oracle attention of one sequence over the rows its index list names:
    only those rows are generated and encoded, and the list is renumbered
    into that compact set (attention does not depend on where rows sit)."""
    valid = idx[idx >= 0]
    uniq, inv = np.unique(valid, return_inverse=True)
    rows = torch.from_numpy(uniq.astype(np.int64) + b * cap)
    kv = ci.gaussian_rows(seed, ci.TID_KV, rows, w.D, dtype=torch.bfloat16, clip=ci.NORM_BOUND)
    oc, osc = oracle.mxfp4_encode(kv)
    cidx = -np.ones_like(idx)
    cidx[idx >= 0] = inv.astype(np.int32)
    return oracle.attn_decode(q, oc, osc, cidx, swa, swa_len, 1.0 / math.sqrt(w.D))


def test_headline_decode_full_128k_b8(K):
    import bench
    w = ci.DECODE_128K
    dev = torch.device("cuda:0")
    print(f"{w.name}: setting up", flush=True)
    s = bench.InputSet(K, w, w.seed, dev)
    step = bench.make_step(K, w, s)
    step.run()
    torch.cuda.synchronize()
    print(f"{w.name}: step done, checking", flush=True)
    pool = step.pool.cpu().numpy()
    idx = step.idx_bufs[0].cpu().numpy()
    lay = s.layers[0]
    N = w.N
    for b in range(w.B):
        kc = _kidx_rows(s.seed, b, N, w.d_I, dev)
        sc = oracle.full_scores(lay.q_idx[b, 0].cpu(), lay.w[b, 0].cpu(), kc, N, N)
        opool = oracle.candidate_pool(oracle.block_max(sc, N, N // 8), w.P_b)
        assert np.array_equal(pool[b, 0], opool), b
        oidx = oracle.topk(sc, w.k)
        assert np.array_equal(idx[b, 0], oidx), b
        if b in (0, w.B - 1):
            want = _attn_ref(w, s.seed, b, N, lay.q[b].cpu(), lay.swa[b].cpu(), w.W, oidx)
            err = float(np.max(np.abs(step.outs[0][b].cpu().numpy() - want)))
            print(f"  seq {b}: attention err {err:.2e}", flush=True)
            assert err < ATOL, (b, err)


def test_decode_20layer_1m_b64_sampled(K):
    import bench
    w = ci.DECODE_1M_20L
    dev = torch.device("cuda:0")
    print(f"{w.name}: setting up (one input set, 36.5 GB of caches)", flush=True)
    s = bench.InputSet(K, w, w.seed, dev)
    step = bench.make_step(K, w, s)
    step.run()
    torch.cuda.synchronize()
    print(f"{w.name}: step done, checking", flush=True)
    N = w.N
    x_layers = [li for li, m in enumerate(w.schedule) if m == "X"]
    for b in (0, w.B - 1):
        kc = _kidx_rows(s.seed, b, N, w.d_I, dev)
        f = s.layers[0]
        sc = oracle.full_scores(f.q_idx[b, 0].cpu(), f.w[b, 0].cpu(), kc, N, N)
        opool = oracle.candidate_pool(oracle.block_max(sc, N, N // 8), w.P_b)
        assert np.array_equal(step.pool[b, 0].cpu().numpy(), opool), b
        of = oracle.topk(sc, w.k)
        assert np.array_equal(step.idx_bufs[0][b, 0].cpu().numpy(), of), b
        del sc
        per_layer = {}
        cur = of
        xi = 0
        for li, mode in enumerate(w.schedule):
            if mode == "X":
                x = s.layers[li]
                ps = oracle.pool_scores(x.q_idx[b, 0].cpu(), x.w[b, 0].cpu(), kc, N, opool)
                cur = oracle.pool_topk(ps, opool, w.k)
                xi += 1
                assert np.array_equal(step.idx_bufs[xi][b, 0].cpu().numpy(), cur), (b, li)
            per_layer[li] = cur
        assert xi == len(x_layers)
        del kc
        for li in (0, 4, 19):
            lay = s.layers[li]
            want = _attn_ref(w, s.seed, b, N, lay.q[b].cpu(), lay.swa[b].cpu(), w.W, per_layer[li])
            err = float(np.max(np.abs(step.outs[li][b].cpu().numpy() - want)))
            print(f"  seq {b} layer {li}: attention err {err:.2e}", flush=True)
            assert err < ATOL, (b, li, err)
