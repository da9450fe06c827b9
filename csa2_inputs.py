"""Seeded synthetic inputs for the CSA2 hot path.

This module is shared by the CPU oracle tests, the GPU parity tests and the
benchmark.  It holds no step of the attention method: it only turns
(seed, tensor id, element index) into numbers, and it names the workload
shapes.  Every value depends only on those three integers, so any slice of a
tensor (say the 2,048 rows a query selected out of a 1M-entry cache) can be
regenerated on the host without copying the device tensor back.

Generator (all arithmetic is integer or an exact table lookup, so the CPU and
the GPU produce identical bits):

* counter:  z = idx + tensor_id * 0x9E3779B97F4A7C15 + seed * 0xD1B54A32D192ED03
  (mod 2^64), then the splitmix64 finaliser
  z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27; z *= 0x94D049BB133111EB;
  z ^= z >> 31.
* Gaussian: the top 16 bits of z index a 65,536-entry table of the inverse
  normal CDF at (i + 0.5) / 65536, computed once in float64 and rounded to
  float32; the result is then rounded (RNE) to the storage dtype.
* Uniform [0, 1): the top 24 bits of z times 2^-24 (exact in float32).
"""
from __future__ import annotations

import dataclasses
import statistics
from typing import Optional

import torch

_M64 = (1 << 64) - 1


def _s64(u: int) -> int:
    """Two's-complement view of an unsigned 64-bit constant."""
    u &= _M64
    return u - (1 << 64) if u >= (1 << 63) else u


_K_TID = _s64(0x9E3779B97F4A7C15)
_K_SEED = _s64(0xD1B54A32D192ED03)
_C1 = _s64(0xBF58476D1CE4E5B9)
_C2 = _s64(0x94D049BB133111EB)


def _lsr(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 lanes."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def _hash(seed: int, tid: int, idx: torch.Tensor) -> torch.Tensor:
    base = _s64(_s64(tid) * _K_TID + _s64(seed) * _K_SEED)
    z = idx.to(torch.int64) + base
    z = z ^ _lsr(z, 30)
    z = z * _C1
    z = z ^ _lsr(z, 27)
    z = z * _C2
    z = z ^ _lsr(z, 31)
    return z


_TABLE_CACHE: dict = {}


def normal_table(device="cpu") -> torch.Tensor:
    key = str(device)
    t = _TABLE_CACHE.get(key)
    if t is None:
        if "cpu" not in _TABLE_CACHE:
            nd = statistics.NormalDist()
            vals = [nd.inv_cdf((i + 0.5) / 65536.0) for i in range(65536)]
            _TABLE_CACHE["cpu"] = torch.tensor(vals, dtype=torch.float64).to(torch.float32)
        t = _TABLE_CACHE["cpu"].to(device)
        _TABLE_CACHE[key] = t
    return t


def gaussian_at(seed: int, tid: int, idx: torch.Tensor, dtype=torch.float32,
                clip: Optional[float] = None) -> torch.Tensor:
    """N(0,1) samples (65,536-level quantile table) at flat element indices."""
    z = _hash(seed, tid, idx)
    v = normal_table(idx.device)[_lsr(z, 48)]
    if clip is not None:
        v = v.clamp(-clip, clip)
    return v.to(dtype)


def uniform_at(seed: int, tid: int, idx: torch.Tensor) -> torch.Tensor:
    """U[0,1) float32 samples at flat element indices."""
    z = _hash(seed, tid, idx)
    return _lsr(z, 40).to(torch.float32) * (2.0 ** -24)


_CHUNK = 1 << 25


def fill_gaussian_(out: torch.Tensor, seed: int, tid: int, clip: Optional[float] = None,
                   first: int = 0) -> torch.Tensor:
    """Fill a contiguous tensor in place; element e gets flat index first + e."""
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        idx = torch.arange(first + s, first + e, device=out.device, dtype=torch.int64)
        flat[s:e] = gaussian_at(seed, tid, idx, dtype=out.dtype, clip=clip)
    return out


def gaussian(seed: int, tid: int, shape, dtype=torch.float32, device="cpu",
             clip: Optional[float] = None) -> torch.Tensor:
    out = torch.empty(shape, dtype=dtype, device=device)
    return fill_gaussian_(out, seed, tid, clip)


def uniform(seed: int, tid: int, shape, device="cpu") -> torch.Tensor:
    n = 1
    for d in shape:
        n *= d
    idx = torch.arange(n, device=device, dtype=torch.int64)
    return uniform_at(seed, tid, idx).reshape(shape)


def gaussian_rows(seed: int, tid: int, rows: torch.Tensor, ncols: int, dtype=torch.float32,
                  clip: Optional[float] = None) -> torch.Tensor:
    """Rows `rows` (flat row ids) of a [*, ncols] Gaussian tensor."""
    rows = rows.to(torch.int64)
    idx = rows[:, None] * ncols + torch.arange(ncols, device=rows.device, dtype=torch.int64)[None, :]
    return gaussian_at(seed, tid, idx, dtype=dtype, clip=clip)


# --------------------------------------------------------------------------
# Tensor ids: one per tensor role; per-layer tensors add 64 * layer.
TID_Q_IDX = 1      # indexer query  [B][Tq][H_I][d_I]
TID_W = 2          # indexer head weights [B][Tq][H_I]
TID_K_IDX = 3      # indexer key cache [B][cap][d_I]
TID_KV = 4         # main KV latent before quantisation [B][cap][D]
TID_Q = 5          # attention query [B][H][D]
TID_SWA = 6        # sliding-window KV [B][W][D]
TID_W_IK = 7       # indexer-K projection weights [D][d_I]
TID_MHC_X = 8      # mHC residual streams [T][n][d]
TID_MHC_F = 9      # mHC block output [T][d]
TID_MHC_COEF = 10  # mHC incoming coefficients A, B, C
TID_MHC_PHI = 11   # mHC projection phiT [2n+n^2][n*d] and bias


def layer_tid(role: int, layer: int) -> int:
    return role + 64 * layer


# --------------------------------------------------------------------------
# Workload shapes (no arithmetic of the method lives here).
NORM_BOUND = 512 ** 0.5    # |KV| <= sqrt(512) for a 512-channel RMS-normed latent


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int            # sequences (decode) or 1 (prefill chunk)
    N: int            # context entries per sequence
    D: int            # main-KV latent channels
    d_I: int          # indexer dim
    H_I: int          # indexer heads
    H: int            # attention query heads
    k: int            # top-k
    W: int            # sliding window
    m: int            # tokens per compressed entry
    schedule: str     # F = Full, X = Reindex, R = Reuse, E = encoder Full (one letter per layer)
    P_b: int = 2048   # candidate-pool blocks (8 positions each)
    T: int = 1        # query tokens per sequence (prefill chunk length)
    prior_tokens: int = 0
    fp32: bool = False
    seed: int = 1000
    enc_m: int = 2    # tokens per entry of an encoder KV set (E layers)


TINY = Workload("tiny-full-1k", B=1, N=1024, D=64, d_I=32, H_I=2, H=4, k=64, W=32, m=1,
                schedule="F", fp32=True, seed=1001)
DECODE_128K = Workload("decode-full-128k-b8", B=8, N=131072, D=512, d_I=128, H_I=8, H=64,
                       k=2048, W=128, m=1, schedule="F", seed=1002)
DECODE_1M_BLOCK2 = Workload("decode-block2-1M-b16", B=16, N=1048576, D=512, d_I=128, H_I=8,
                            H=64, k=2048, W=128, m=1, schedule="XRRR", seed=1003)
PREFILL_CHUNK = Workload("prefill-chunk-m2-t8192", B=1, N=135168, D=512, d_I=128, H_I=8, H=64,
                         k=2048, W=128, m=2, schedule="FRRRRR", T=8192, prior_tokens=262144,
                         seed=1004)
DECODE_1M_20L = Workload("decode-20layer-1M-b64", B=64, N=1048576, D=512, d_I=128, H_I=8, H=64,
                         k=2048, W=128, m=1, schedule="FRRR" + "XRRR" * 4, seed=1005)

# one decode token through every CSA2 layer of the network: the encoder's
# three blocks of Full + 5 Reuse at m = 2 (each Full over a KV set of its own,
# 524,288 entries at 1M tokens), then the decoder's 20 layers
DECODE_1M_38L = Workload("decode-38layer-1M-b64", B=64, N=1048576, D=512, d_I=128, H_I=8, H=64,
                         k=2048, W=128, m=1, schedule="ERRRRR" * 3 + "FRRR" + "XRRR" * 4, seed=1006)

# SWA bounded replay: the decoder's 20 layers over the newest n_win = 128
# tokens of one 1M-token sequence, each token a decoder query with its own
# candidate pool, windows cut at the replay start
DECODER_REPLAY = Workload("decoder-replay-1M-t128", B=1, N=1048576, D=512, d_I=128, H_I=8, H=64,
                          k=2048, W=128, m=1, schedule="FRRR" + "XRRR" * 4, T=128,
                          prior_tokens=1048576 - 128, seed=1007)

WORKLOADS = {w.name: w for w in (TINY, DECODE_128K, DECODE_1M_BLOCK2, PREFILL_CHUNK, DECODE_1M_20L,
                                 DECODE_1M_38L, DECODER_REPLAY)}
