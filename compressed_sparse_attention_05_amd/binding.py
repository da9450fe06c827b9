"""ctypes binding over libcsa2 (include/csa2.h): same names, argument
marshalling only.  Tensors are torch tensors on the current HIP device; the
binding allocates outputs and workspaces with torch (device memory is
PyTorch's job here) and passes raw pointers plus the current stream.  Every
step of the path runs in the library's kernels: if the library is missing or
no GPU is present, calls raise instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")

CSA2_F32, CSA2_BF16 = 0, 1

P = ctypes.c_void_p
i32, i64 = ctypes.c_int32, ctypes.c_int64


class ScoreArgs(ctypes.Structure):
    _fields_ = [("q_idx", P), ("q_dtype", i32), ("w", P), ("k_idx", P), ("k_dtype", i32),
                ("B", i64), ("Tq", i64), ("cap", i64), ("H_I", i32), ("d_I", i32),
                ("ctx_len", P), ("q_pos", P), ("m", i32), ("pool_blocks", P), ("P_b", i32),
                ("scores", P), ("ld_scores", i64), ("block_max", P)]


class MhcArgs(ctypes.Structure):
    _fields_ = [("X", P), ("f", P), ("A", P), ("B", P), ("C", P), ("phiT", P), ("bias", P),
                ("alpha_pre", ctypes.c_float), ("alpha_post", ctypes.c_float), ("alpha_res", ctypes.c_float),
                ("T", i64), ("n", i32), ("d", i32), ("iters", i32),
                ("X_next", P), ("u_next", P), ("A_next", P), ("B_next", P), ("C_next", P)]


class AttnArgs(ctypes.Structure):
    _fields_ = [("q", P), ("q_dtype", i32), ("codes", P), ("scales", P), ("cap", i64),
                ("idx", P), ("k", i32), ("swa", P), ("swa_dtype", i32), ("W", i32),
                ("swa_len", P), ("B", i64), ("H", i32), ("D", i32), ("sm_scale", ctypes.c_float),
                ("out", P)]


class AttnPrefillArgs(ctypes.Structure):
    _fields_ = [("q", P), ("q_dtype", i32), ("codes", P), ("scales", P), ("cap", i64),
                ("idx", P), ("k", i32), ("swa", P), ("swa_dtype", i32), ("W", i32),
                ("q_pos0", i64), ("swa_start", i64), ("T", i64), ("H", i32), ("D", i32),
                ("sm_scale", ctypes.c_float), ("out", P)]


# Every function the header declares, with its ctypes signature.
class PrefillTopkArgs(ctypes.Structure):
    _fields_ = [("q_idx", P), ("q_dtype", i32), ("w", P), ("k_idx", P), ("k_dtype", i32),
                ("T", i64), ("cap", i64), ("H_I", i32), ("d_I", i32), ("ctx_len", i32),
                ("q_pos0", i64), ("m", i32), ("k", i32), ("out_idx", P)]


class DecodeSelectArgs(ctypes.Structure):
    _fields_ = [("q_idx", P), ("q_dtype", i32), ("w", P), ("k_idx", P), ("k_dtype", i32),
                ("ctx_len", P), ("B", i64), ("cap", i64), ("H_I", i32), ("d_I", i32),
                ("P_b", i32), ("k", i32), ("out_pool", P), ("out_idx", P)]


SIGNATURES = {
    "csa2_version": (ctypes.c_char_p, []),
    "csa2_last_error": (ctypes.c_char_p, []),
    "mxfp4_kv_write": (ctypes.c_int, [P, ctypes.c_int, i64, i32, P, i64, P, P, P, ctypes.c_int, i32, P, P]),
    "csa2_kv_write_project": (ctypes.c_int, [P, ctypes.c_int, i64, i32, P, i64, P, P, P, i32, P, P]),
    "csa2_mhc_step": (ctypes.c_int, [ctypes.POINTER(MhcArgs), P]),
    "csa2_index_score_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(ScoreArgs)]),
    "csa2_index_score": (ctypes.c_int, [ctypes.POINTER(ScoreArgs), P, ctypes.c_size_t, P]),
    "csa2_write_and_score": (ctypes.c_int, [P, ctypes.c_int, i32, P, P, P, P, ctypes.POINTER(ScoreArgs), P,
                                            ctypes.c_size_t, P]),
    "csa2_topk_workspace_size": (ctypes.c_size_t, [i64, i64, i32]),
    "csa2_topk": (ctypes.c_int, [P, i64, i64, i64, i32, P, i32, P, P, ctypes.c_size_t, P]),
    "csa2_build_candidate_pool_workspace_size": (ctypes.c_size_t, [i64, i64, i32]),
    "csa2_build_candidate_pool": (ctypes.c_int, [P, i64, i64, i64, i32, P, P, ctypes.c_size_t, P]),
    "csa2_topk_from_pool": (ctypes.c_int, [P, i64, i64, P, i32, i32, P, P]),
    "csa2_pool_topk": (ctypes.c_int, [P, i64, i64, i64, i32, P, P, i64, i32, P, P]),
    "csa2_decode_select_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(DecodeSelectArgs)]),
    "csa2_decode_scan": (ctypes.c_int, [ctypes.POINTER(DecodeSelectArgs), P, ctypes.c_size_t, P]),
    "csa2_decode_select": (ctypes.c_int, [ctypes.POINTER(DecodeSelectArgs), P, ctypes.c_size_t, P]),
    "csa2_sparse_attn_decode_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(AttnArgs)]),
    "csa2_sparse_attn_decode": (ctypes.c_int, [ctypes.POINTER(AttnArgs), P, ctypes.c_size_t, P]),
    "csa2_sparse_attn_decode_noalloc": (ctypes.c_int, [ctypes.POINTER(AttnArgs), P]),
    "csa2_sparse_attn_prefill_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(AttnPrefillArgs)]),
    "csa2_sparse_attn_prefill": (ctypes.c_int, [ctypes.POINTER(AttnPrefillArgs), P, ctypes.c_size_t, P]),
    "csa2_prefill_topk_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(PrefillTopkArgs)]),
    "csa2_prefill_topk": (ctypes.c_int, [ctypes.POINTER(PrefillTopkArgs), P, ctypes.c_size_t, P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libcsa2.so (built by build.py); raises if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libcsa2.so not built at {LIB_PATH}: run "
                               "`python -m compressed_sparse_attention_05_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def version() -> str:
    return lib().csa2_version().decode()


# --------------------------------------------------------------------------
def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype(t: torch.Tensor, name: str) -> int:
    if t.dtype == torch.float32:
        return CSA2_F32
    if t.dtype == torch.bfloat16:
        return CSA2_BF16
    raise TypeError(f"{name} must be float32 or bfloat16, got {t.dtype}")


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(rc: int) -> None:
    if rc != 0:
        raise RuntimeError(f"libcsa2 error {rc}: {lib().csa2_last_error().decode()}")


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


# --------------------------------------------------------------------------
def tile_indexer_cache(k_rows: torch.Tensor) -> torch.Tensor:
    """Row-major indexer keys [B][cap][d_I] -> the library's tiled layout
    (returned with the same nominal shape).  Pure data movement: tile t of
    64 flat rows stores 16-byte chunk c of row 64t+p at ((t*NCH + c)*64 + p)*16."""
    B, cap, d_I = k_rows.shape
    esz = k_rows.element_size()
    cpc = 16 // esz
    nch = d_I // cpc
    if cap % 64 or (d_I * esz) % 16:
        raise ValueError("tiled indexer cache needs cap % 64 == 0 and 16-byte rows")
    t = k_rows.reshape(B, cap // 64, 64, nch, cpc).permute(0, 1, 3, 2, 4).contiguous()
    return t.view(B, cap, d_I)


def untile_indexer_cache(k_tiled: torch.Tensor) -> torch.Tensor:
    """Inverse of tile_indexer_cache."""
    B, cap, d_I = k_tiled.shape
    cpc = 16 // k_tiled.element_size()
    nch = d_I // cpc
    t = k_tiled.reshape(B, cap // 64, nch, 64, cpc).permute(0, 1, 3, 2, 4).contiguous()
    return t.view(B, cap, d_I)


def mxfp4_kv_write(x, dst_row, codes, scales, idx_k_rows=None, idx_k_cache=None, stream=None):
    """Quantise rows x [n][D] into codes/scales at flat rows dst_row (int64),
    optionally copying idx_k_rows [n][d_I] into idx_k_cache."""
    _dev(x, "x"); _dev(dst_row, "dst_row"); _dev(codes, "codes"); _dev(scales, "scales")
    if dst_row.dtype != torch.int64 or codes.dtype != torch.uint8 or scales.dtype != torch.uint8:
        raise TypeError("dst_row must be int64, codes/scales uint8")
    n, D = x.shape[0], x.shape[-1]
    n_cache_rows = codes.numel() // (D // 2)
    if scales.numel() != n_cache_rows * (D // 16):
        raise ValueError("codes and scales describe different row counts")
    d_I, kdt = 0, 0
    if idx_k_rows is not None:
        _dev(idx_k_rows, "idx_k_rows"); _dev(idx_k_cache, "idx_k_cache")
        d_I = idx_k_rows.shape[-1]
        kdt = _dtype(idx_k_rows, "idx_k_rows")
        if idx_k_cache.dtype != idx_k_rows.dtype or idx_k_cache.numel() != n_cache_rows * d_I:
            raise ValueError("idx_k_cache must match idx_k_rows' dtype and the cache row count")
    _check(lib().mxfp4_kv_write(_ptr(x), _dtype(x, "x"), n, D, _ptr(dst_row), n_cache_rows,
                                _ptr(codes), _ptr(scales), _ptr(idx_k_rows), kdt, d_I,
                                _ptr(idx_k_cache), _stream(stream)))


def csa2_kv_write_project(x, dst_row, codes, scales, w_ik, idx_k_cache, stream=None):
    """Quantise rows x [n][D] into codes/scales at flat rows dst_row (int64)
    and write their projected indexer keys bf16(x . w_ik) (w_ik [D][d_I]
    float32) into the tiled bfloat16 idx_k_cache."""
    for t, nm in ((x, "x"), (dst_row, "dst_row"), (codes, "codes"), (scales, "scales"), (w_ik, "w_ik"),
                  (idx_k_cache, "idx_k_cache")):
        _dev(t, nm)
    if dst_row.dtype != torch.int64 or codes.dtype != torch.uint8 or scales.dtype != torch.uint8:
        raise TypeError("dst_row must be int64, codes/scales uint8")
    if w_ik.dtype != torch.float32 or w_ik.dim() != 2 or not w_ik.is_contiguous():
        raise TypeError("w_ik must be a contiguous float32 [D][d_I] tensor")
    if idx_k_cache.dtype != torch.bfloat16:
        raise TypeError("idx_k_cache must be bfloat16")
    n, D = x.shape[0], x.shape[-1]
    d_I = w_ik.shape[1]
    if w_ik.shape[0] != D:
        raise ValueError(f"w_ik has {w_ik.shape[0]} rows, x has {D} channels")
    n_cache_rows = codes.numel() // (D // 2)
    if scales.numel() != n_cache_rows * (D // 16) or idx_k_cache.numel() != n_cache_rows * d_I:
        raise ValueError("codes, scales and idx_k_cache describe different row counts")
    _check(lib().csa2_kv_write_project(_ptr(x), _dtype(x, "x"), n, D, _ptr(dst_row), n_cache_rows,
                                       _ptr(codes), _ptr(scales), _ptr(w_ik), d_I, _ptr(idx_k_cache),
                                       _stream(stream)))


def csa2_mhc_step(X, f, A, B, C, phiT, bias, alphas, iters: int = 20, out=None, stream=None):
    """One fused single-pass mHC step for T tokens.  X [T][n][d] bf16, f [T][d]
    bf16, A [T][n], B [T][n][n], C [T][n] f32, phiT [2n+n^2][n*d] bf16, bias
    [2n+n^2] f32, alphas = (alpha_pre, alpha_post, alpha_res).  Returns
    (X_next, u_next, A_next, B_next, C_next); `out` may supply them."""
    for t, nm in ((X, "X"), (f, "f"), (A, "A"), (B, "B"), (C, "C"), (phiT, "phiT"), (bias, "bias")):
        _dev(t, nm)
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    if X.dtype != torch.bfloat16 or f.dtype != torch.bfloat16 or phiT.dtype != torch.bfloat16:
        raise TypeError("X, f and phiT must be bfloat16")
    for t, nm in ((A, "A"), (B, "B"), (C, "C"), (bias, "bias")):
        if t.dtype != torch.float32:
            raise TypeError(f"{nm} must be float32")
    T, n, d = X.shape
    K = 2 * n + n * n
    if (tuple(f.shape) != (T, d) or tuple(A.shape) != (T, n) or tuple(B.shape) != (T, n, n)
            or tuple(C.shape) != (T, n) or tuple(phiT.shape) != (K, n * d) or tuple(bias.shape) != (K,)):
        raise ValueError("mHC argument shapes do not match X [T][n][d]")
    if out is None:
        out = (torch.empty_like(X), torch.empty_like(f), torch.empty_like(A), torch.empty_like(B),
               torch.empty_like(C))
    Xn, u, An, Bn, Cn = out
    a = MhcArgs(X=X.data_ptr(), f=f.data_ptr(), A=A.data_ptr(), B=B.data_ptr(), C=C.data_ptr(),
                phiT=phiT.data_ptr(), bias=bias.data_ptr(), alpha_pre=float(alphas[0]),
                alpha_post=float(alphas[1]), alpha_res=float(alphas[2]), T=T, n=n, d=d, iters=iters,
                X_next=Xn.data_ptr(), u_next=u.data_ptr(), A_next=An.data_ptr(), B_next=Bn.data_ptr(),
                C_next=Cn.data_ptr())
    _check(lib().csa2_mhc_step(ctypes.byref(a), _stream(stream)))
    return out


def csa2_index_score(q_idx, w, k_idx, ctx_len, *, q_pos=None, m: int = 1, pool_blocks=None,
                     scores=None, ld: Optional[int] = None, want_block_max: bool = False,
                     block_max=None, stream=None):
    """Indexer scores.  q_idx [B][Tq][H_I][d_I], w [B][Tq][H_I] f32,
    k_idx [B][cap][d_I], ctx_len [B] int32, q_pos [B][Tq] int64 or None,
    pool_blocks [B][Tq][P_b] int32 or None.  Returns (scores, block_max)."""
    for t, nm in ((q_idx, "q_idx"), (w, "w"), (k_idx, "k_idx"), (ctx_len, "ctx_len")):
        _dev(t, nm)
    B, Tq, H_I, d_I = q_idx.shape
    cap = k_idx.shape[1]
    P_b = 0
    if pool_blocks is not None:
        _dev(pool_blocks, "pool_blocks")
        P_b = pool_blocks.shape[-1]
    if ld is None:
        ld = 8 * P_b if pool_blocks is not None else cap
    if scores is None:
        scores = torch.empty((B, Tq, ld), dtype=torch.float32, device=q_idx.device)
    if want_block_max and block_max is None:
        block_max = torch.empty((B, Tq, (ld + 7) // 8), dtype=torch.float32, device=q_idx.device)
    a = ScoreArgs(q_idx=q_idx.data_ptr(), q_dtype=_dtype(q_idx, "q_idx"), w=w.data_ptr(),
                  k_idx=k_idx.data_ptr(), k_dtype=_dtype(k_idx, "k_idx"), B=B, Tq=Tq, cap=cap,
                  H_I=H_I, d_I=d_I, ctx_len=ctx_len.data_ptr(),
                  q_pos=None if q_pos is None else _dev(q_pos, "q_pos").data_ptr(), m=m,
                  pool_blocks=None if pool_blocks is None else pool_blocks.data_ptr(), P_b=P_b,
                  scores=scores.data_ptr(), ld_scores=ld,
                  block_max=None if block_max is None else block_max.data_ptr())
    L = lib()
    ws = _workspace(L.csa2_index_score_workspace_size(ctypes.byref(a)), q_idx.device)
    _check(L.csa2_index_score(ctypes.byref(a), _ptr(ws), 0 if ws is None else ws.numel(),
                              _stream(stream)))
    return scores, block_max


def csa2_write_and_score(x, dst_row, codes, scales, idx_k_rows, q_idx, w, k_idx, ctx_len, *,
                         pool_blocks=None, scores=None, ld: Optional[int] = None,
                         want_block_max: bool = False, block_max=None, stream=None):
    """A decode token's cache write (as mxfp4_kv_write of x [B][D] and
    idx_k_rows [B][d_I] to flat rows dst_row [B] int64) and the scan that
    follows it (as csa2_index_score with Tq == 1) in one launch.  dst_row[b]
    must address a row of sequence b; other rows are not written.  Returns
    (scores, block_max)."""
    for t, nm in ((x, "x"), (dst_row, "dst_row"), (codes, "codes"), (scales, "scales"),
                  (idx_k_rows, "idx_k_rows"), (q_idx, "q_idx"), (w, "w"), (k_idx, "k_idx"),
                  (ctx_len, "ctx_len")):
        _dev(t, nm)
    if dst_row.dtype != torch.int64 or codes.dtype != torch.uint8 or scales.dtype != torch.uint8:
        raise TypeError("dst_row must be int64, codes/scales uint8")
    B, Tq, H_I, d_I = q_idx.shape
    cap = k_idx.shape[1]
    D = x.shape[-1]
    if Tq != 1 or x.shape[0] != B or tuple(idx_k_rows.shape) != (B, d_I) or dst_row.numel() != B:
        raise ValueError("one new row, key and destination per sequence (Tq == 1)")
    if idx_k_rows.dtype != k_idx.dtype:
        raise ValueError("idx_k_rows must have the indexer cache's dtype")
    if codes.numel() != B * cap * (D // 2) or scales.numel() != B * cap * (D // 16):
        raise ValueError("codes/scales must hold B*cap rows of D channels")
    P_b = 0
    if pool_blocks is not None:
        _dev(pool_blocks, "pool_blocks")
        P_b = pool_blocks.shape[-1]
    if ld is None:
        ld = 8 * P_b if pool_blocks is not None else cap
    if scores is None:
        scores = torch.empty((B, 1, ld), dtype=torch.float32, device=q_idx.device)
    if want_block_max and block_max is None:
        block_max = torch.empty((B, 1, (ld + 7) // 8), dtype=torch.float32, device=q_idx.device)
    a = ScoreArgs(q_idx=q_idx.data_ptr(), q_dtype=_dtype(q_idx, "q_idx"), w=w.data_ptr(),
                  k_idx=k_idx.data_ptr(), k_dtype=_dtype(k_idx, "k_idx"), B=B, Tq=1, cap=cap,
                  H_I=H_I, d_I=d_I, ctx_len=ctx_len.data_ptr(), q_pos=None, m=1,
                  pool_blocks=None if pool_blocks is None else pool_blocks.data_ptr(), P_b=P_b,
                  scores=scores.data_ptr(), ld_scores=ld,
                  block_max=None if block_max is None else block_max.data_ptr())
    _check(lib().csa2_write_and_score(_ptr(x), _dtype(x, "x"), D, _ptr(dst_row), _ptr(codes), _ptr(scales),
                                      _ptr(idx_k_rows), ctypes.byref(a), None, 0, _stream(stream)))
    return scores, block_max


def csa2_topk(scores, k: int, *, n: Optional[int] = None, pool_blocks=None, out=None, stream=None):
    """Exact top-k per row of scores [..., ld]; returns int32 [rows..., k]."""
    _dev(scores, "scores")
    ld = scores.shape[-1]
    rows = scores.numel() // ld if ld else 0
    P_b = 0
    if pool_blocks is not None:
        _dev(pool_blocks, "pool_blocks")
        P_b = pool_blocks.shape[-1]
        if n is None:
            n = 8 * P_b
    if n is None:
        n = ld
    if out is None:
        out = torch.empty((*scores.shape[:-1], k), dtype=torch.int32, device=scores.device)
    L = lib()
    ws = _workspace(L.csa2_topk_workspace_size(rows, n, k), scores.device)
    _check(L.csa2_topk(_ptr(scores), rows, n, ld, k, _ptr(pool_blocks), P_b, _ptr(out), _ptr(ws),
                       0 if ws is None else ws.numel(), _stream(stream)))
    return out


def csa2_build_candidate_pool(block_max, P_b: int = 2048, *, n_blocks: Optional[int] = None,
                              out=None, stream=None):
    """Top-P_b blocks per row of block_max [..., ld]; ascending ids, -1 padded."""
    _dev(block_max, "block_max")
    ld = block_max.shape[-1]
    rows = block_max.numel() // ld if ld else 0
    if n_blocks is None:
        n_blocks = ld
    if out is None:
        out = torch.empty((*block_max.shape[:-1], P_b), dtype=torch.int32, device=block_max.device)
    L = lib()
    ws = _workspace(L.csa2_build_candidate_pool_workspace_size(rows, n_blocks, P_b), block_max.device)
    _check(L.csa2_build_candidate_pool(_ptr(block_max), rows, n_blocks, ld, P_b, _ptr(out), _ptr(ws),
                                       0 if ws is None else ws.numel(), _stream(stream)))
    return out


def csa2_topk_from_pool(scores, pool_blocks, k: int, *, out=None, stream=None):
    """Full-mode top-k of position-ordered scores [..., ld] through the
    candidate pool [..., P_b] (k <= P_b); equals csa2_topk over the row."""
    _dev(scores, "scores"); _dev(pool_blocks, "pool_blocks")
    ld = scores.shape[-1]
    rows = scores.numel() // ld if ld else 0
    P_b = pool_blocks.shape[-1]
    if out is None:
        out = torch.empty((*scores.shape[:-1], k), dtype=torch.int32, device=scores.device)
    _check(lib().csa2_topk_from_pool(_ptr(scores), rows, ld, _ptr(pool_blocks), P_b, k, _ptr(out),
                                     _stream(stream)))
    return out


def csa2_pool_topk(block_max, scores, P_b: int, k: int, n_blocks: Optional[int] = None, *,
                   out_blocks=None, out=None, stream=None):
    """Candidate pool [..., P_b] and Full-mode top-k [..., k] in one launch;
    the same results as csa2_build_candidate_pool then csa2_topk_from_pool."""
    _dev(block_max, "block_max"); _dev(scores, "scores")
    ld_bm = block_max.shape[-1]
    ld = scores.shape[-1]
    rows = scores.numel() // ld if ld else 0
    nb = ld_bm if n_blocks is None else n_blocks
    if out_blocks is None:
        out_blocks = torch.empty((*scores.shape[:-1], P_b), dtype=torch.int32, device=scores.device)
    if out is None:
        out = torch.empty((*scores.shape[:-1], k), dtype=torch.int32, device=scores.device)
    _check(lib().csa2_pool_topk(_ptr(block_max), rows, nb, ld_bm, P_b, _ptr(out_blocks), _ptr(scores), ld, k,
                                _ptr(out), _stream(stream)))
    return out_blocks, out


def csa2_sparse_attn_decode(q, codes, scales, idx, swa, swa_len, *, sm_scale: Optional[float] = None,
                            out=None, stream=None):
    """q [B][H][D]; codes [B][cap][D/2]; scales [B][cap][D/16]; idx [B][k] int32;
    swa [B][W][D]; swa_len [B] int32.  Returns out [B][H][D] float32."""
    for t, nm in ((q, "q"), (codes, "codes"), (scales, "scales"), (idx, "idx"), (swa, "swa"),
                  (swa_len, "swa_len")):
        _dev(t, nm)
    B, H, D = q.shape
    cap = codes.shape[1]
    W = swa.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, H, D), dtype=torch.float32, device=q.device)
    a = AttnArgs(q=q.data_ptr(), q_dtype=_dtype(q, "q"), codes=codes.data_ptr(),
                 scales=scales.data_ptr(), cap=cap, idx=idx.data_ptr(), k=idx.shape[-1],
                 swa=swa.data_ptr(), swa_dtype=_dtype(swa, "swa"), W=W, swa_len=swa_len.data_ptr(),
                 B=B, H=H, D=D, sm_scale=sm_scale, out=out.data_ptr())
    L = lib()
    ws = _workspace(L.csa2_sparse_attn_decode_workspace_size(ctypes.byref(a)), q.device)
    _check(L.csa2_sparse_attn_decode(ctypes.byref(a), _ptr(ws), 0 if ws is None else ws.numel(),
                                     _stream(stream)))
    return out


def csa2_sparse_attn_prefill(q, codes, scales, idx, swa, W: int, q_pos0: int, *, swa_start: int = 0,
                             sm_scale: Optional[float] = None, out=None, stream=None):
    """q [T][H][D]; codes [cap][D/2]; scales [cap][D/16]; idx [T][k];
    swa [T+W-1][D] (row r = token q_pos0-(W-1)+r).  Returns out [T][H][D]."""
    for t, nm in ((q, "q"), (codes, "codes"), (scales, "scales"), (idx, "idx"), (swa, "swa")):
        _dev(t, nm)
    T, H, D = q.shape
    if swa.shape[0] != T + W - 1:
        raise ValueError("swa must hold T + W - 1 rows")
    if out is None:
        out = torch.empty((T, H, D), dtype=torch.float32, device=q.device)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    a = AttnPrefillArgs(q=q.data_ptr(), q_dtype=_dtype(q, "q"), codes=codes.data_ptr(),
                        scales=scales.data_ptr(), cap=codes.shape[0], idx=idx.data_ptr(),
                        k=idx.shape[-1], swa=swa.data_ptr(), swa_dtype=_dtype(swa, "swa"), W=W,
                        q_pos0=q_pos0, swa_start=swa_start, T=T, H=H, D=D, sm_scale=sm_scale,
                        out=out.data_ptr())
    L = lib()
    ws = _workspace(L.csa2_sparse_attn_prefill_workspace_size(ctypes.byref(a)), q.device)
    _check(L.csa2_sparse_attn_prefill(ctypes.byref(a), _ptr(ws), 0 if ws is None else ws.numel(),
                                      _stream(stream)))
    return out


def csa2_decode_select(q_idx, w, k_idx, ctx_len, P_b: int, k: int, *, out_pool=None, out=None,
                       workspace=None, stream=None):
    """Decode Full layer: candidate pool [B][P_b] and top-k [B][k] from the
    indexer query q_idx [B][8][128] bf16 (or [B][1][8][128]), w [B][8] f32,
    the tiled indexer cache k_idx [B][cap][128] bf16 and ctx_len [B] int32,
    with the matrix-core scan (csa2_decode_scan then csa2_decode_select).
    Equals csa2_index_score + csa2_build_candidate_pool + csa2_topk_from_pool."""
    for t, nm in ((q_idx, "q_idx"), (w, "w"), (k_idx, "k_idx"), (ctx_len, "ctx_len")):
        _dev(t, nm)
    B, cap, d_I = k_idx.shape
    H_I = q_idx.shape[-2]
    if out_pool is None:
        out_pool = torch.empty((B, P_b), dtype=torch.int32, device=q_idx.device)
    if out is None:
        out = torch.empty((B, k), dtype=torch.int32, device=q_idx.device)
    a = DecodeSelectArgs(q_idx=q_idx.data_ptr(), q_dtype=_dtype(q_idx, "q_idx"), w=w.data_ptr(),
                         k_idx=k_idx.data_ptr(), k_dtype=_dtype(k_idx, "k_idx"), ctx_len=ctx_len.data_ptr(),
                         B=B, cap=cap, H_I=H_I, d_I=d_I, P_b=int(P_b), k=int(k), out_pool=out_pool.data_ptr(),
                         out_idx=out.data_ptr())
    L = lib()
    need = L.csa2_decode_select_workspace_size(ctypes.byref(a))
    ws = workspace if workspace is not None else _workspace(need, q_idx.device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = _stream(stream)
    _check(L.csa2_decode_scan(ctypes.byref(a), _ptr(ws), nbytes, st))
    _check(L.csa2_decode_select(ctypes.byref(a), _ptr(ws), nbytes, st))
    return out_pool, out


def csa2_prefill_topk(q_idx, w, k_idx, ctx_len: int, q_pos0: int, m: int, k: int, *, out=None,
                      workspace=None, stream=None):
    """Full-mode top-k of a prefill chunk.  q_idx [T][8][128] bf16, w [T][8]
    f32, k_idx one sequence's tiled indexer cache [cap][128] (or [1][cap][128])
    bf16; query t sits at position q_pos0 + t.  Returns out [T][k] int32."""
    for t, nm in ((q_idx, "q_idx"), (w, "w"), (k_idx, "k_idx")):
        _dev(t, nm)
    T, H_I, d_I = q_idx.shape
    kc = k_idx.reshape(-1, k_idx.shape[-1])
    if out is None:
        out = torch.empty((T, k), dtype=torch.int32, device=q_idx.device)
    a = PrefillTopkArgs(q_idx=q_idx.data_ptr(), q_dtype=_dtype(q_idx, "q_idx"), w=w.data_ptr(),
                        k_idx=kc.data_ptr(), k_dtype=_dtype(kc, "k_idx"), T=T, cap=kc.shape[0], H_I=H_I,
                        d_I=d_I, ctx_len=int(ctx_len), q_pos0=int(q_pos0), m=int(m), k=int(k),
                        out_idx=out.data_ptr())
    L = lib()
    need = L.csa2_prefill_topk_workspace_size(ctypes.byref(a))
    ws = workspace if workspace is not None else _workspace(need, q_idx.device)
    _check(L.csa2_prefill_topk(ctypes.byref(a), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                               _stream(stream)))
    return out
