"""CPU oracle for the single-pass mHC block step (numpy, float64).

TEST INFRASTRUCTURE ONLY.  Only the tests and the benchmark's CPU-baseline
leg may import this module.  It shares no code with the HIP library or its
binding.

Sources (page title, section):
  [KVC] "DeepSeek-V4.1-Flash KV Cache Compression" reading notes, section 6
        (single-pass mHC: the residual stream widened into n streams, the
        one-block shift of the input-mixing coefficients, the (2n+2)d bound).
  [SUM] DeepSeek-V4.1-Flash summary page, Methodology item 4, equation (6).

The pages define the step
    X_{l+1} = B_l X_l + C_l F_l(A_{l-1} X_l),   (A_l, B_l, C_l) = H(X_l)
with X_l in R^{n x d}, A in R^{1 x n}, B in R^{n x n}, C in R^{n x 1}, and
say that one read of X_l does the input mixing and accumulates the statistics
that predict the next coefficients.  One fused pass therefore takes X_l, the
block output f_l = F_l(A_{l-1} X_l) and the coefficients (A_l, B_l, C_l) that
the previous pass predicted, and produces
    X_{l+1} = B_l X_l + C_l f_l                     (residual update)
    u_{l+1} = A_l X_{l+1}                            (input of F_{l+1})
    (A_{l+1}, B_{l+1}, C_{l+1}) = H(X_{l+1})         (next coefficients)
reading n*d + d values and writing n*d + d: the (2n+2)d traffic.

The pages leave H, n, d and the precision open.  Readings taken here:
  * H follows the manifold-constrained hyper-connection form the name refers
    to: x = the n*d stream values flattened (stream-major), r = sqrt(mean(x^2)
    + 1e-6), z = (x . phi) / r with phi in R^{(n*d) x (2n + n^2)}, then
        A = sigmoid(alpha_pre  * z[0:n]       + b[0:n])
        C = 2 * sigmoid(alpha_post * z[n:2n]  + b[n:2n])
        B = Sinkhorn(exp(alpha_res * z[2n:]   + b[2n:]) as an n x n matrix),
    Sinkhorn = `iters` rounds of (divide every row by its sum, then every
    column by its sum), which drives B toward a doubly stochastic matrix.
  * X, f and u are stored as bfloat16; X_{l+1} is rounded to bfloat16 (nearest,
    ties to even) when stored, and u and H read the stored X_{l+1}.
  * phi is given transposed, phiT[o][i*d + c], in bfloat16 (here as float64
    values already on the bfloat16 grid); coefficients and biases are float.
"""
from __future__ import annotations

import numpy as np

RMS_EPS = 1e-6


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value (ties to even) of each finite float64 entry,
    returned as float64.  Rounds the float64 value directly (one rounding)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                   # x = m * 2**e, 0.5 <= |m| < 1
    scaled = m * 256.0                   # 8 significant bits: bfloat16's precision
    r = np.round(scaled)                 # numpy rounds halves to even
    out = np.ldexp(r, e - 8)
    return np.where(x == 0.0, 0.0, out)


def sigmoid(v: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-v))


def sinkhorn(M: np.ndarray, iters: int) -> np.ndarray:
    """Alternate row and column normalisation of a positive matrix (rows first)."""
    M = np.array(M, dtype=np.float64)
    for _ in range(iters):
        M = M / M.sum(axis=-1, keepdims=True)
        M = M / M.sum(axis=-2, keepdims=True)
    return M


def coefficients(Xs: np.ndarray, phiT: np.ndarray, bias: np.ndarray, alphas, iters: int):
    """H of one token's stored streams Xs [n][d] -> (A [n], B [n][n], C [n])."""
    n, d = Xs.shape
    x = Xs.reshape(n * d)
    r = np.sqrt(np.mean(x * x) + RMS_EPS)
    z = (np.asarray(phiT, np.float64) @ x) / r
    a_pre, a_post, a_res = alphas
    A = sigmoid(a_pre * z[0:n] + bias[0:n])
    C = 2.0 * sigmoid(a_post * z[n:2 * n] + bias[n:2 * n])
    B = sinkhorn(np.exp(a_res * z[2 * n:] + bias[2 * n:]).reshape(n, n), iters)
    return A, B, C


def mhc_step(X, f, A, B, C, phiT, bias, alphas, iters: int = 20):
    """One fused pass for T tokens.

    X [T][n][d], f [T][d] (bfloat16 values), A [T][n], B [T][n][n], C [T][n]:
    the coefficients the previous pass predicted.  Returns
    (Xn [T][n][d] float64 before storage rounding, Xs = its bfloat16 values,
     u [T][d] float64 from Xs, A' [T][n], B' [T][n][n], C' [T][n])."""
    X = np.asarray(X, np.float64)
    f = np.asarray(f, np.float64)
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    C = np.asarray(C, np.float64)
    bias = np.asarray(bias, np.float64)
    T, n, d = X.shape
    Xn = np.einsum("tij,tjc->tic", B, X) + C[:, :, None] * f[:, None, :]
    Xs = bf16_round(Xn)
    u = np.einsum("ti,tic->tc", A, Xs)
    An = np.zeros((T, n))
    Bn = np.zeros((T, n, n))
    Cn = np.zeros((T, n))
    for t in range(T):
        An[t], Bn[t], Cn[t] = coefficients(Xs[t], phiT, bias, alphas, iters)
    return Xn, Xs, u, An, Bn, Cn
