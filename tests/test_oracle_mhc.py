"""Pins of the single-pass mHC oracle (oracle/mhc.py) against what the pages
and the mathematics fix: bfloat16 rounding against PyTorch's conversion, the
Sinkhorn limit of a 2 x 2 matrix in closed form, closed-form coefficients when
the projection is zero, the scale invariance of the RMS-normalised logits, and
brute-force loops on tiny inputs for the residual update, the shifted input
mixing and the projection."""
import math

import numpy as np
import torch

from oracle import mhc


def _bf16_grid(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).double().numpy()


def test_bf16_round_matches_torch_conversion():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                        [0.0, -0.0, 1.0, -3.5, 65504.0, 1e-30]]).astype(np.float32)
    want = torch.tensor(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(mhc.bf16_round(x.astype(np.float64)), want)
    # exact midpoints go to the even mantissa: 1 + 2^-8 -> 1, 1 + 3*2^-8 -> 1 + 2^-6
    assert mhc.bf16_round(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert mhc.bf16_round(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6


def test_sinkhorn_2x2_closed_form():
    # the doubly stochastic scaling of [[a, b], [c, d]] is [[p, 1-p], [1-p, p]]
    # with p = sqrt(ad) / (sqrt(ad) + sqrt(bc))
    for a, b, c, d in [(1.0, 2.0, 3.0, 4.0), (0.2, 5.0, 1.5, 0.7), (9.0, 1.0, 1.0, 9.0)]:
        p = math.sqrt(a * d) / (math.sqrt(a * d) + math.sqrt(b * c))
        S = mhc.sinkhorn(np.array([[a, b], [c, d]]), 200)
        assert np.allclose(S, [[p, 1 - p], [1 - p, p]], atol=1e-12, rtol=0)


def test_sinkhorn_ends_on_columns_and_converges():
    rng = np.random.default_rng(2)
    M = np.exp(rng.standard_normal((4, 4)))
    for it in (1, 5, 20):
        S = mhc.sinkhorn(M, it)
        assert np.allclose(S.sum(axis=0), 1.0, atol=1e-14)       # last step normalised columns
    S = mhc.sinkhorn(M, 200)
    assert np.allclose(S.sum(axis=1), 1.0, atol=1e-10)
    assert mhc.sinkhorn(np.ones((4, 4)), 1).tolist() == [[0.25] * 4] * 4


def _inputs(seed, T, n, d):
    rng = np.random.default_rng(seed)
    X = _bf16_grid(rng.standard_normal((T, n, d)))
    f = _bf16_grid(rng.standard_normal((T, d)))
    A = rng.uniform(0.1, 1.0, (T, n))
    B = mhc.sinkhorn(np.exp(rng.standard_normal((T, n, n))), 20)
    C = rng.uniform(0.2, 1.8, (T, n))
    K = 2 * n + n * n
    phiT = _bf16_grid(rng.standard_normal((K, n * d)) / math.sqrt(n * d))
    bias = rng.standard_normal(K) * 0.5
    return X, f, A, B, C, phiT, bias


def test_zero_projection_gives_closed_form_coefficients():
    n, d = 4, 16
    X, f, A, B, C, phiT, _ = _inputs(3, 2, n, d)
    bias = np.zeros(2 * n + n * n)
    _, _, _, An, Bn, Cn = mhc.mhc_step(X, f, A, B, C, np.zeros_like(phiT), bias, (1.0, 1.0, 1.0))
    assert np.all(An == 0.5) and np.all(Cn == 1.0)          # sigmoid(0) = 1/2, 2 sigmoid(0) = 1
    assert np.all(Bn == 0.25)                               # exp(0) = 1 everywhere -> 1/n
    bias[:n] = np.log(3.0)                                  # sigmoid(ln 3) = 3/4
    _, _, _, An, _, _ = mhc.mhc_step(X, f, A, B, C, np.zeros_like(phiT), bias, (1.0, 1.0, 1.0))
    assert np.allclose(An, 0.75, atol=1e-15)


def test_identity_residual_copies_and_mixes_with_incoming_A():
    # B = I, C = 0: X_{l+1} = X_l exactly; u uses the incoming A (the shift)
    n, d, T = 4, 32, 3
    X, f, A, _, _, phiT, bias = _inputs(4, T, n, d)
    B = np.broadcast_to(np.eye(n), (T, n, n))
    C = np.zeros((T, n))
    Xn, Xs, u, An, _, _ = mhc.mhc_step(X, f, A, B, C, phiT, bias, (0.7, 0.9, 1.1))
    assert np.array_equal(Xn, X) and np.array_equal(Xs, X)
    for t in range(T):
        for c in range(d):
            assert abs(u[t, c] - sum(A[t, i] * X[t, i, c] for i in range(n))) < 1e-12
    assert not np.allclose(An, A)       # H(X_{l+1}) is a fresh prediction, not the input A


def test_brute_force_tiny_step():
    n, d, T = 2, 3, 2
    X, f, A, B, C, phiT, bias = _inputs(5, T, n, d)
    al = (0.8, 1.3, 0.6)
    Xn, Xs, u, An, Bn, Cn = mhc.mhc_step(X, f, A, B, C, phiT, bias, al, iters=3)
    for t in range(T):
        for i in range(n):
            for c in range(d):
                want = C[t, i] * f[t, c]
                for j in range(n):
                    want += B[t, i, j] * X[t, j, c]
                assert abs(Xn[t, i, c] - want) < 1e-12
        xs = [Xs[t, i, c] for i in range(n) for c in range(d)]
        r = math.sqrt(sum(v * v for v in xs) / (n * d) + 1e-6)
        z = [sum(phiT[o][k] * xs[k] for k in range(n * d)) / r for o in range(2 * n + n * n)]
        for i in range(n):
            assert abs(An[t, i] - 1 / (1 + math.exp(-(al[0] * z[i] + bias[i])))) < 1e-12
            assert abs(Cn[t, i] - 2 / (1 + math.exp(-(al[1] * z[n + i] + bias[n + i])))) < 1e-12
        M = [[math.exp(al[2] * z[2 * n + i * n + j] + bias[2 * n + i * n + j]) for j in range(n)]
             for i in range(n)]
        for _ in range(3):
            M = [[M[i][j] / sum(M[i]) for j in range(n)] for i in range(n)]
            cs = [sum(M[i][j] for i in range(n)) for j in range(n)]
            M = [[M[i][j] / cs[j] for j in range(n)] for i in range(n)]
        assert np.allclose(Bn[t], M, atol=1e-12)


def test_logits_are_scale_invariant():
    n, d, T = 4, 64, 2
    X, f, A, B, C, phiT, bias = _inputs(6, T, n, d)
    al = (1.0, 1.0, 1.0)
    _, _, _, A1, B1, C1 = mhc.mhc_step(X, f, A, B, C, phiT, bias, al)
    # doubling X and f doubles X_{l+1} exactly (powers of two keep the bfloat16 grid)
    _, _, _, A2, B2, C2 = mhc.mhc_step(2 * X, 2 * f, A, B, C, phiT, bias, al)
    for p, q in ((A1, A2), (B1, B2), (C1, C2)):
        assert np.allclose(p, q, atol=1e-6)
