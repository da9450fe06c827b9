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
