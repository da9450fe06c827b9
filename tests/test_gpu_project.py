"""GPU parity of csa2_kv_write_project (MXFP4 write with the indexer key
projected from the same latent rows) against the oracle: codes, scales and the
bfloat16 keys bit-exact, rows outside the cache untouched."""
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


def _weights(seed, D, d_I):
    return ci.gaussian(seed, ci.TID_W_IK, (D, d_I)) * np.float32(1.0 / np.sqrt(D))


def _case(K, seed, n, D, d_I, cap, dtype, dst=None, x=None, W=None):
    if x is None:
        x = ci.gaussian(seed, ci.TID_KV, (n, D), clip=ci.NORM_BOUND).to(dtype)
    if W is None:
        W = _weights(seed, D, d_I)
    if dst is None:
        dst = torch.randperm(cap, generator=torch.Generator().manual_seed(seed))[:n].to(torch.int64)
    print(f"case seed={seed} n={n} D={D} d_I={d_I} cap={cap} {dtype}", flush=True)
    codes = torch.full((cap, D // 2), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((cap, D // 16), 0xCD, dtype=torch.uint8, device="cuda")
    kc = torch.full((1, cap, d_I), -7.0, dtype=torch.bfloat16, device="cuda")
    K.csa2_kv_write_project(x.cuda(), dst.cuda(), codes, scales, W.cuda(), kc)
    torch.cuda.synchronize()
    xf = x.float()
    want_c, want_s = oracle.mxfp4_encode(xf)
    want_k = oracle.project_kidx(xf, W)
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    got_k = K.untile_indexer_cache(kc)[0].cpu().view(torch.int16).numpy().view(np.uint16)
    written = set()
    for i in range(n):
        d = int(dst[i])
        if 0 <= d < cap:
            written.add(d)
            assert np.array_equal(got_c[d], want_c[i]), ("codes", i)
            assert np.array_equal(got_s[d], want_s[i]), ("scales", i)
            assert np.array_equal(got_k[d], want_k[i]), ("key", i, np.flatnonzero(got_k[d] != want_k[i])[:8])
    sentinel = np.uint16(torch.tensor([-7.0], dtype=torch.bfloat16).view(torch.int16).item() & 0xFFFF)
    for d in set(range(cap)) - written:
        assert (got_c[d] == 0xAB).all() and (got_s[d] == 0xCD).all() and (got_k[d] == sentinel).all(), d


def test_project_decode_batch_bf16(K):
    # one new entry per sequence for 64 sequences, scattered over the cache
    _case(K, 31, 64, 512, 128, 1024, torch.bfloat16)


def test_project_fp32_rows_and_ragged_group(K):
    # 37 rows (8-row tiles below 513 rows): four full tiles and a ragged one of 5
    _case(K, 32, 37, 512, 128, 256, torch.float32)


def test_project_tiny_shape_and_single_row(K):
    _case(K, 33, 1, 64, 32, 64, torch.float32)
    _case(K, 34, 19, 64, 32, 64, torch.float32)
    # a column count that is not a multiple of the 32-column slice
    _case(K, 39, 21, 128, 40, 64, torch.bfloat16)


def test_project_skips_rows_outside_the_cache(K):
    dst = torch.tensor([3, -1, 70, 128, 5, 200, 127], dtype=torch.int64)
    _case(K, 35, 7, 512, 128, 128, torch.bfloat16, dst=dst)


def test_project_prefill_chunk_entries(K):
    # a prefill chunk's 4,096 new m = 2 entries, written contiguously
    n, cap = 4096, 8192
    dst = torch.arange(n, dtype=torch.int64) + 2048
    _case(K, 36, n, 512, 128, cap, torch.bfloat16, dst=dst)


def test_project_many_rows_ragged_group(K):
    # 1,100 rows (32-row tiles above 512 rows): 34 full tiles and a ragged one of 12
    n, cap = 1100, 2048
    dst = torch.randperm(cap, generator=torch.Generator().manual_seed(38))[:n].to(torch.int64)
    dst[17] = -1
    _case(K, 38, n, 512, 128, cap, torch.float32, dst=dst)


def test_project_exactly_summable_and_rounding_ties(K):
    # x and W on coarse grids: every chain is exact, and the products land on
    # bfloat16 midpoints (ties to even) and on values past the largest bfloat16
    n, D, d_I = 32, 512, 128
    g = torch.Generator().manual_seed(37)
    x = (torch.randint(-16, 17, (n, D), generator=g).float() * 0.25)
    W = (torch.randint(-8, 9, (D, d_I), generator=g).float() * 0.125)
    W[:, 0] = 0.0
    W[0, 0] = 1.0 + 2.0 ** -8          # x[r][0] * (1 + 2^-8): a bfloat16 midpoint when x is a power of two
    x[:, 0] = 2.0
    W[:, 1] = 0.0
    W[0, 1] = 1.7e38                   # 2 * 1.7e38 = 3.4e38, past the largest bfloat16: stays finite
    _case(K, 37, n, D, d_I, 64, torch.float32, x=x, W=W, dst=torch.arange(n, dtype=torch.int64))
