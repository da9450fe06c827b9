"""CPU oracle for the CSA2 global-attention hot path (ctypes over csa2_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the HIP
library or its binding, and neither imports the other.

bf16 inputs are widened to float32 here (exact: the 16 bits become the high
half of the float32 word); everything else happens in csa2_oracle.c.

Sources (page title, section):
  [KVC] "DeepSeek-V4.1-Flash KV Cache Compression" reading notes, sections 2-5.
  [SUM] DeepSeek-V4.1-Flash summary page, "Methodology / Architecture Components".
  [DR]  "DeepSeek-V4.1-Flash: reading a model through its three memory costs", 03.
  [THR] "Notes on DeepSeek V4.1 Flash" thread, posts 4-6 and 9.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa2_oracle.c")
_LIB = os.path.join(_HERE, "libcsa2_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
                               "-fPIC", "-shared", _SRC, "-lm", "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        sig = {
            "csa2o_e2m1_value": (dbl, [i32]),
            "csa2o_e4m3_value": (dbl, [i32]),
            "csa2o_mxfp4_encode": (None, [P, i64, i32, P, P]),
            "csa2o_mxfp4_decode": (None, [P, P, i64, i32, P]),
            "csa2o_score_one": (ctypes.c_float, [P, P, P, i32, i32]),
            "csa2o_full_scores": (None, [P, P, P, i32, i32, i64, i64, P]),
            "csa2o_block_max": (None, [P, i64, i64, P]),
            "csa2o_topk": (i64, [P, i64, i64, P]),
            "csa2o_pool_scores": (None, [P, P, P, i32, i32, i64, P, i32, P]),
            "csa2o_pool_topk": (i64, [P, P, i32, i64, P]),
            "csa2o_attn_decode": (None, [P, i32, i32, P, P, P, i32, P, i32, dbl, P]),
            "csa2o_prefill_vis": (i64, [i64, i64, i32]),
            "csa2o_prefill_scores": (None, [P, P, P, i32, i32, P, i64, i64, i32, i64, P]),
            "csa2o_attn_prefill": (None, [P, i64, i32, i32, P, P, P, i32, P, i32, i64, i64, dbl, P]),
            "csa2o_bf16_nearest": (ctypes.c_uint16, [ctypes.c_float]),
            "csa2o_project_kidx": (None, [P, i64, i32, P, i32, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


# ---------------------------------------------------------------------------
def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def as_f32(x) -> np.ndarray:
    """float32 view of an input array: float32 as is, bf16 (torch tensor or uint16
    bit array) widened exactly."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu()
            if x.dtype == torch.bfloat16:
                x = x.view(torch.int16).numpy().view(np.uint16)
            else:
                x = x.to(torch.float32).numpy()
    except ImportError:  # pragma: no cover
        pass
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return np.ascontiguousarray((x.astype(np.uint32) << 16).view(np.float32))
    return np.ascontiguousarray(x, dtype=np.float32)


def e2m1_value(nibble: int) -> float:
    return lib().csa2o_e2m1_value(int(nibble))


def e4m3_value(byte: int) -> float:
    return lib().csa2o_e4m3_value(int(byte))


def mxfp4_encode(x) -> tuple[np.ndarray, np.ndarray]:
    """[n][D] values -> (codes [n][D/2] u8, scales [n][D/16] u8)."""
    x = as_f32(x)
    n, D = x.shape
    codes = np.zeros((n, D // 2), np.uint8)
    scales = np.zeros((n, D // 16), np.uint8)
    lib().csa2o_mxfp4_encode(_ptr(x), n, D, _ptr(codes), _ptr(scales))
    return codes, scales


def mxfp4_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    n, half = codes.shape
    out = np.zeros((n, half * 2), np.float64)
    lib().csa2o_mxfp4_decode(_ptr(codes), _ptr(scales), n, half * 2, _ptr(out))
    return out


def bf16_nearest(f: float) -> int:
    """bfloat16 bit pattern nearest to a finite float32 (ties to even)."""
    return lib().csa2o_bf16_nearest(float(np.float32(f)))


def project_kidx(x, W) -> np.ndarray:
    """Indexer-K rows from latent rows: x [n][D], W [D][d_I] float32 ->
    bfloat16 bit patterns [n][d_I] (fp32 fma chain over channels, then
    round to nearest bfloat16)."""
    x, W = as_f32(x), as_f32(W)
    n, D = x.shape
    d_I = W.shape[1]
    assert W.shape[0] == D
    out = np.zeros((n, d_I), np.uint16)
    lib().csa2o_project_kidx(_ptr(x), n, D, _ptr(W), d_I, _ptr(out))
    return out


def score_one(q, w, k) -> np.float32:
    q, w, k = as_f32(q), as_f32(w), as_f32(k)
    H_I, d_I = q.shape
    return np.float32(lib().csa2o_score_one(_ptr(q), _ptr(w), _ptr(k), H_I, d_I))


def full_scores(q, w, kcache, vis: int, n_out: int) -> np.ndarray:
    """q [H_I][d_I], w [H_I], kcache [>=vis][d_I] -> scores [n_out] float32."""
    q, w, kcache = as_f32(q), as_f32(w), as_f32(kcache)
    H_I, d_I = q.shape
    out = np.empty(n_out, np.float32)
    lib().csa2o_full_scores(_ptr(q), _ptr(w), _ptr(kcache), H_I, d_I, vis, n_out, _ptr(out))
    return out


def block_max(scores: np.ndarray, vis: int, n_blocks: int) -> np.ndarray:
    scores = np.ascontiguousarray(scores, np.float32)
    out = np.empty(n_blocks, np.float32)
    lib().csa2o_block_max(_ptr(scores), vis, n_blocks, _ptr(out))
    return out


def topk(vals: np.ndarray, k: int) -> np.ndarray:
    vals = np.ascontiguousarray(vals, np.float32)
    out = np.empty(k, np.int32)
    lib().csa2o_topk(_ptr(vals), vals.shape[0], k, _ptr(out))
    return out


def candidate_pool(bm: np.ndarray, P_b: int) -> np.ndarray:
    """Top-P_b blocks by (block max desc, block id asc), ascending ids ([KVC] section 3)."""
    return topk(bm, P_b)


def pool_scores(q, w, kcache, vis: int, pool: np.ndarray) -> np.ndarray:
    q, w, kcache = as_f32(q), as_f32(w), as_f32(kcache)
    pool = np.ascontiguousarray(pool, np.int32)
    H_I, d_I = q.shape
    out = np.empty(pool.shape[0] * 8, np.float32)
    lib().csa2o_pool_scores(_ptr(q), _ptr(w), _ptr(kcache), H_I, d_I, vis, _ptr(pool),
                            pool.shape[0], _ptr(out))
    return out


def pool_topk(scores: np.ndarray, pool: np.ndarray, k: int) -> np.ndarray:
    scores = np.ascontiguousarray(scores, np.float32)
    pool = np.ascontiguousarray(pool, np.int32)
    out = np.empty(k, np.int32)
    lib().csa2o_pool_topk(_ptr(scores), _ptr(pool), pool.shape[0], k, _ptr(out))
    return out


def attn_decode(q, codes, scales, idx, swa, swa_len: int, sm_scale: float) -> np.ndarray:
    """q [H][D]; codes/scales of one sequence's cache; idx [k]; swa [>=swa_len][D]."""
    q = as_f32(q)
    swa = as_f32(swa)
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    idx = np.ascontiguousarray(idx, np.int32)
    H, D = q.shape
    out = np.empty((H, D), np.float32)
    lib().csa2o_attn_decode(_ptr(q), H, D, _ptr(codes), _ptr(scales), _ptr(idx), idx.shape[0],
                            _ptr(swa), swa_len, float(sm_scale), _ptr(out))
    return out


def prefill_vis(q_pos: int, ctx_len: int, m: int) -> int:
    return lib().csa2o_prefill_vis(q_pos, ctx_len, m)


def prefill_scores(q, w, kcache, q_pos: np.ndarray, ctx_len: int, m: int, ld: int) -> np.ndarray:
    q, w, kcache = as_f32(q), as_f32(w), as_f32(kcache)
    q_pos = np.ascontiguousarray(q_pos, np.int64)
    T, H_I, d_I = q.shape
    out = np.empty((T, ld), np.float32)
    lib().csa2o_prefill_scores(_ptr(q), _ptr(w), _ptr(kcache), H_I, d_I, _ptr(q_pos), T, ctx_len,
                               m, ld, _ptr(out))
    return out


def attn_prefill(q, codes, scales, idx, swa, W: int, q_pos0: int, swa_start: int,
                 sm_scale: float) -> np.ndarray:
    q = as_f32(q)
    swa = as_f32(swa)
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    idx = np.ascontiguousarray(idx, np.int32)
    T, H, D = q.shape
    assert swa.shape[0] == T + W - 1
    out = np.empty((T, H, D), np.float32)
    lib().csa2o_attn_prefill(_ptr(q), T, H, D, _ptr(codes), _ptr(scales), _ptr(idx), idx.shape[1],
                             _ptr(swa), W, q_pos0, swa_start, float(sm_scale), _ptr(out))
    return out
