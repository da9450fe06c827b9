"""A decode step captured into a HIP graph replays the eager step exactly:
three replays, with the program's own eager work and synchronisations in
between, each compared bit for bit with the eager result (outputs, pool and
index lists)."""
import pytest
import torch

import csa2_inputs as ci

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.fail("gpu tests need a GPU")
    import compressed_sparse_attention_05_amd as K
    K.lib()
    return K


def _step(K, seed, B=2, cap=4096, D=512, H=64, d_I=128, H_I=8, W=128, k=128, P_b=256, schedule="FXR"):
    from compressed_sparse_attention_05_amd.decode import DecodeCache, DecodeStep, LayerInputs
    dev = torch.device("cuda:0")
    ctx = [cap - 7, cap // 2 + 3][:B]
    kv = ci.gaussian(seed, ci.TID_KV, (B * cap, D), clip=ci.NORM_BOUND).to(dev)
    kidx = ci.gaussian(seed, ci.TID_K_IDX, (B * cap, d_I), dtype=torch.bfloat16).to(dev)
    codes = torch.zeros((B, cap, D // 2), dtype=torch.uint8, device=dev)
    scales = torch.zeros((B, cap, D // 16), dtype=torch.uint8, device=dev)
    kc = torch.zeros((B, cap, d_I), dtype=torch.bfloat16, device=dev)
    rows = torch.arange(B * cap, dtype=torch.int64, device=dev)
    K.mxfp4_kv_write(kv, rows, codes, scales, kidx, kc)
    cache = DecodeCache(codes=codes, scales=scales, k_idx=kc,
                        ctx_len=torch.tensor(ctx, dtype=torch.int32, device=dev),
                        swa_len=torch.tensor([W, 40][:B], dtype=torch.int32, device=dev))
    layers = [LayerInputs(q=ci.gaussian(seed + i, ci.TID_Q, (B, H, D), dtype=torch.bfloat16).to(dev),
                          swa=ci.gaussian(seed + i, ci.TID_SWA, (B, W, D), dtype=torch.bfloat16).to(dev),
                          q_idx=ci.gaussian(seed + i, ci.TID_Q_IDX, (B, 1, H_I, d_I), dtype=torch.bfloat16).to(dev),
                          w=ci.uniform(seed + i, ci.TID_W, (B, 1, H_I)).to(dev)) for i in range(len(schedule))]
    new_rows = torch.tensor([b * cap + ctx[b] - 1 for b in range(B)], dtype=torch.int64, device=dev)
    return DecodeStep(schedule, cache, layers, k=k, P_b=P_b, new_kv=kv[new_rows].contiguous(),
                      new_kidx=kidx[new_rows].contiguous(), dst_row=new_rows)


def _snapshot(step):
    return [o.clone() for o in step.outs] + [step.pool.clone()] + [i.clone() for i in step.idx_bufs]


def test_decode_step_graph_replays_match_eager(K):
    step = _step(K, 501)
    other = _step(K, 502)
    step.run()
    torch.cuda.synchronize()
    want = _snapshot(step)
    graph = step.capture()
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work of the program between replays, and clobbered outputs
        other.run()
        for o in step.outs:
            o.zero_()
        for i in step.idx_bufs:
            i.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(step)
        for a, b in zip(got, want):
            assert torch.equal(a, b), rep


def _replay_check(make_call, outs, clobber, reps=3):
    """Capture make_call() into a graph; each replay (after eager work that
    clobbers what the call writes) must reproduce the eager outputs bit for
    bit.  outs() returns the written values."""
    make_call()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        make_call()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        make_call()
    torch.cuda.synchronize()
    for rep in range(reps):
        clobber()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for w, o in zip(want, outs()):
            assert torch.equal(w, o), rep


def test_kv_write_project_graph_replays_match_eager(K):
    dev = torch.device("cuda:0")
    n, D, d_I, cap = 64, 512, 128, 1024
    x = ci.gaussian(601, ci.TID_KV, (n, D), dtype=torch.bfloat16, clip=ci.NORM_BOUND).to(dev)
    w_ik = (ci.gaussian(601, ci.TID_W_IK, (D, d_I)) / 22.627).to(dev)
    dst = (torch.arange(n, dtype=torch.int64) * 16 + 3).to(dev)
    codes = torch.zeros((cap, D // 2), dtype=torch.uint8, device=dev)
    scales = torch.zeros((cap, D // 16), dtype=torch.uint8, device=dev)
    kc = torch.zeros((1, cap, d_I), dtype=torch.bfloat16, device=dev)

    def clobber():                      # every byte the call writes, and more
        codes.fill_(0x5A)
        scales.fill_(0xA5)
        kc.fill_(3.0)

    def written():
        return [codes[dst], scales[dst], K.untile_indexer_cache(kc)[0][dst]]

    _replay_check(lambda: K.csa2_kv_write_project(x, dst, codes, scales, w_ik, kc), written, clobber)


def test_mhc_step_graph_replays_match_eager(K):
    import math
    dev = torch.device("cuda:0")
    T, n, d = 200, 4, 1024
    X = ci.gaussian(602, ci.TID_MHC_X, (T, n, d), dtype=torch.bfloat16).to(dev)
    f = ci.gaussian(602, ci.TID_MHC_F, (T, d), dtype=torch.bfloat16).to(dev)
    coef = ci.uniform(602, ci.TID_MHC_COEF, (T, 24)).to(dev)
    A, B, C = coef[:, :4].contiguous(), (0.5 * coef[:, 4:20]).reshape(T, 4, 4).contiguous(), (2 * coef[:, 20:]).contiguous()
    phiT = (ci.gaussian(602, ci.TID_MHC_PHI, (24, n * d)) / math.sqrt(n * d)).to(torch.bfloat16).to(dev)
    bias = (0.5 * ci.gaussian(603, ci.TID_MHC_PHI, (24,))).to(dev)
    out = (torch.empty_like(X), torch.empty_like(f), torch.empty_like(A), torch.empty_like(B), torch.empty_like(C))

    def clobber():
        for o in out:
            o.fill_(-1.0)

    _replay_check(lambda: K.csa2_mhc_step(X, f, A, B, C, phiT, bias, (1.0, 1.0, 1.0), iters=20, out=out),
                  lambda: list(out), clobber)
