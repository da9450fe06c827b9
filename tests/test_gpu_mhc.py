"""GPU parity of csa2_mhc_step (single-pass mHC) against the float64 oracle.

Tolerances, from the arithmetic:
  * X_next: the kernel rounds a float32 value, the result of four fmas and a
    product, whose error is at most 5 * 2^-24 times the sum of the terms'
    magnitudes; so X_next is the exactly rounded bfloat16 or, next to a
    rounding midpoint (or after cancellation), a value within
    2^-7 |exact| + 2^-21 * sum|terms|, and almost every value matches bit for bit.
  * u_next and H are functions of the stored X_next, and a one-ulp flip of
    one of its n*d values moves a logit by about |phi| * 2^-8 |x| ~ 1e-4.  So
    they are checked against the oracle applied to the X_next the kernel
    stored: u_next within one bfloat16 rounding (2^-8 |u|) plus float32 error
    (2^-21 sum|A x|); A, B, C within 2e-5 (relative above 1: B without
    Sinkhorn rounds is unnormalised), from a float32 projection over n*d
    exact bfloat16 products, sigmoid and a 4 x 4 Sinkhorn.  End to end
    against the oracle's own X_next they agree within 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import csa2_inputs as ci
from oracle import mhc as omhc

pytestmark = pytest.mark.gpu
N = 4
K_OUT = 2 * N + N * N


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.fail("gpu tests need a GPU")
    import compressed_sparse_attention_05_amd as K
    K.lib()
    return K


def make_inputs(seed, T, d):
    X = ci.gaussian(seed, ci.TID_MHC_X, (T, N, d), dtype=torch.bfloat16)
    f = ci.gaussian(seed, ci.TID_MHC_F, (T, d), dtype=torch.bfloat16)
    coef = ci.uniform(seed, ci.TID_MHC_COEF, (T, N + N * N + N))
    A = (0.1 + 0.9 * coef[:, :N]).contiguous()
    B = (0.5 * coef[:, N:N + N * N]).reshape(T, N, N).contiguous()
    C = (0.2 + 1.6 * coef[:, N + N * N:]).contiguous()
    phiT = (ci.gaussian(seed, ci.TID_MHC_PHI, (K_OUT, N * d)) / math.sqrt(N * d)).to(torch.bfloat16)
    bias = 0.5 * ci.gaussian(seed + 1, ci.TID_MHC_PHI, (K_OUT,))
    return X, f, A, B, C, phiT, bias


def run_gpu(K, inp, alphas, iters, pad=32):
    X, f, A, B, C, phiT, bias = [t.cuda() for t in inp]
    T, _, d = X.shape
    big = (torch.full((T + pad, N, d), 7.0, dtype=torch.bfloat16, device="cuda"),
           torch.full((T + pad, d), 7.0, dtype=torch.bfloat16, device="cuda"),
           torch.full((T + pad, N), 7.0, device="cuda"), torch.full((T + pad, N, N), 7.0, device="cuda"),
           torch.full((T + pad, N), 7.0, device="cuda"))
    out = tuple(b[:T] for b in big)
    K.csa2_mhc_step(X, f, A, B, C, phiT, bias, alphas, iters=iters, out=out)
    torch.cuda.synchronize()
    for b in big:                                  # nothing written past T
        assert bool((b[T:] == 7.0).all())
    return [o.double().cpu().numpy() for o in out]


def check(inp, got, alphas, iters, rows=None):
    X, f, A, B, C, phiT, bias = [t.double().numpy() for t in inp]
    if rows is not None:
        X, f, A, B, C = X[rows], f[rows], A[rows], B[rows], C[rows]
        got = [g[rows] for g in got]
    Xn, Xs, u, An, Bn, Cn = omhc.mhc_step(X, f, A, B, C, phiT, bias, alphas, iters)
    gX, gu, gA, gB, gC = got
    mag = np.einsum("tij,tjc->tic", np.abs(B), np.abs(X)) + np.abs(C)[:, :, None] * np.abs(f)[:, None, :]
    assert np.all(np.abs(gX - Xn) <= 2.0 ** -7 * np.abs(Xn) + 2.0 ** -21 * mag)
    assert np.mean(gX == Xs) > 0.999
    # u and H from the X_next the kernel stored
    uref = np.einsum("ti,tic->tc", A, gX)
    ub = 2.0 ** -8 * np.abs(uref) + 2.0 ** -21 * np.einsum("ti,tic->tc", np.abs(A), np.abs(gX)) + 1e-30
    assert np.all(np.abs(gu - uref) <= ub)
    for t in range(gX.shape[0]):
        Ar, Br, Cr = omhc.coefficients(gX[t], phiT, bias, alphas, iters)
        for g, w, nm in ((gA[t], Ar, "A"), (gB[t], Br, "B"), (gC[t], Cr, "C")):
            err = float(np.max(np.abs(g - w) / np.maximum(1.0, np.abs(w))))
            assert err <= 2e-5, (nm, t, err)
    for g, w, nm in ((gA, An, "A"), (gB, Bn, "B"), (gC, Cn, "C")):
        err = float(np.max(np.abs(g - w) / np.maximum(1.0, np.abs(w))))
        assert err <= 1e-3, (nm, err)


@pytest.mark.parametrize("T,d,seed", [(100, 512, 61), (1, 256, 62), (64, 4096, 63), (33, 384, 66), (5, 128, 67)])
def test_mhc_step_matches_oracle(K, T, d, seed):
    print(f"mhc T={T} d={d} seed={seed}", flush=True)
    inp = make_inputs(seed, T, d)
    alphas = (1.0, 0.8, 1.2)
    got = run_gpu(K, inp, alphas, 20)
    check(inp, got, alphas, 20)


def test_mhc_step_no_sinkhorn_rounds(K):
    inp = make_inputs(64, 40, 256)
    alphas = (0.5, 0.5, 0.5)
    got = run_gpu(K, inp, alphas, 0)
    check(inp, got, alphas, 0)


def test_mhc_step_full_chunk_sampled(K):
    # the benchmark's shape: 8,192 tokens x 4 streams x 4,096 channels;
    # sampled tokens in every workgroup position, including the last
    T, d, seed = 8192, 4096, 65
    print(f"mhc T={T} d={d} sampled", flush=True)
    inp = make_inputs(seed, T, d)
    alphas = (1.0, 1.0, 1.0)
    got = run_gpu(K, inp, alphas, 20, pad=0)
    rows = np.unique(np.concatenate([np.arange(0, T, 257), np.arange(T - 40, T), [31, 32, 33]]))
    check(inp, got, alphas, 20, rows=rows)
