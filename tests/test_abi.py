"""The C-ABI library loads and exports every symbol include/csa2.h declares,
and its host-side argument checks return the documented status codes
(these calls return before any device work, so they run without a GPU)."""
import ctypes
import os
import re

import pytest

from compressed_sparse_attention_05_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|const char\s*\*)\s*\*?\s*(\w+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_hot_path_calls():
    names = declared_functions()
    for n in ["mxfp4_kv_write", "csa2_index_score", "csa2_topk", "csa2_build_candidate_pool",
              "csa2_sparse_attn_decode", "csa2_sparse_attn_prefill", "csa2_last_error",
              "csa2_version"]:
        assert n in names, n


def test_library_exports_every_declared_symbol():
    L = binding.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    assert set(declared_functions()) <= set(binding.SIGNATURES)


def test_version_string():
    assert "gfx950" in binding.version()


def _err():
    return binding.lib().csa2_last_error().decode()


def test_topk_rejects_bad_arguments_on_host():
    L = binding.lib()
    rc = L.csa2_topk(None, 4, 10, 10, 0, None, 0, None, None, 0, None)
    assert rc == 1 and "k must be positive" in _err()
    rc = L.csa2_topk(None, 4, 10, 5, 3, None, 0, None, None, 0, None)
    assert rc == 1 and "ld" in _err()
    rc = L.csa2_topk(ctypes.c_void_p(16), 1, 17, 17, 3, ctypes.c_void_p(16), 2, ctypes.c_void_p(16),
                     None, 0, None)
    assert rc == 1 and "8*P_b" in _err()
    assert L.csa2_topk(None, 0, 10, 10, 3, None, 0, None, None, 0, None) == 0  # nothing to do


def test_score_unsupported_shape_and_layout_checks():
    L = binding.lib()
    a = binding.ScoreArgs(q_idx=16, q_dtype=1, w=16, k_idx=16, k_dtype=1, B=1, Tq=1, cap=8, H_I=3,
                          d_I=128, ctx_len=16, m=1, scores=16, ld_scores=8)
    assert L.csa2_index_score(ctypes.byref(a), None, 0, None) == 2
    a.H_I = 8
    assert L.csa2_index_score_workspace_size(ctypes.byref(a)) == 0
    assert L.csa2_index_score(ctypes.byref(a), None, 0, None) == 1  # cap not a multiple of 64
    assert "multiple of 64" in _err()
    a.cap, a.m = 64, 0
    assert L.csa2_index_score(ctypes.byref(a), None, 0, None) == 1


def test_topk_workspace_sizes():
    L = binding.lib()
    assert L.csa2_topk_workspace_size(8, 16384, 2048) == 0          # staged in LDS
    big = L.csa2_topk_workspace_size(8, 131072, 2048)
    assert big > 8 * 4096 * 4
    assert L.csa2_topk(ctypes.c_void_p(256), 8, 131072, 131072, 2048, None, 0,
                       ctypes.c_void_p(256), None, 0, None) == 3     # workspace missing


def test_kv_write_and_attention_argument_checks():
    L = binding.lib()
    assert L.mxfp4_kv_write(None, 0, 1, 20, None, 1, None, None, None, 0, 0, None, None) == 1
    assert "multiple of 16" in _err()
    a = binding.AttnArgs(q=16, q_dtype=1, codes=16, scales=16, cap=4, idx=16, k=4, swa=16, swa_dtype=1,
                         W=4, swa_len=16, B=1, H=48, D=512, sm_scale=0.1, out=16)
    assert L.csa2_sparse_attn_decode(ctypes.byref(a), None, 0, None) == 2
    a.H, a.D = 64, 40
    assert L.csa2_sparse_attn_decode(ctypes.byref(a), None, 0, None) == 1


def test_prefill_topk_argument_checks():
    L = binding.lib()
    a = binding.PrefillTopkArgs(q_idx=256, q_dtype=1, w=256, k_idx=256, k_dtype=1, T=16, cap=1024, H_I=8,
                                d_I=128, ctx_len=1000, q_pos0=1990, m=2, k=64, out_idx=256)
    need = L.csa2_prefill_topk_workspace_size(ctypes.byref(a))
    assert need > 16 * 1000 * 8                      # candidate slots of the chunk
    assert L.csa2_prefill_topk(ctypes.byref(a), None, 0, None) == 3
    assert "workspace" in _err()
    a.H_I = 4
    assert L.csa2_prefill_topk(ctypes.byref(a), None, 0, None) == 2
    assert L.csa2_prefill_topk_workspace_size(ctypes.byref(a)) == 0
    a.H_I, a.q_dtype = 8, 0
    assert L.csa2_prefill_topk(ctypes.byref(a), None, 0, None) == 2
    a.q_dtype, a.k = 1, 5000
    assert L.csa2_prefill_topk(ctypes.byref(a), None, 0, None) == 2
    a.k, a.cap = 64, 1000
    assert L.csa2_prefill_topk(ctypes.byref(a), None, 0, None) == 1
    assert "multiple of 64" in _err()
    a.cap, a.m = 1024, 0
    assert L.csa2_prefill_topk(ctypes.byref(a), None, 0, None) == 1
    a.m, a.ctx_len = 2, 2000
    assert L.csa2_prefill_topk(ctypes.byref(a), None, 0, None) == 1
    a.cap, a.ctx_len, a.q_pos0, a.m = 1 << 25, 1 << 25, 1 << 25, 1     # 2^25 visible entries
    assert L.csa2_prefill_topk(ctypes.byref(a), None, 0, None) == 2
    assert "visible entries" in _err()
    a.cap, a.ctx_len, a.q_pos0, a.m = 1024, 2000, 1990, 2
    a.ctx_len, a.T = 1000, 0
    assert L.csa2_prefill_topk(ctypes.byref(a), None, 0, None) == 0    # nothing to do


def test_pool_topk_argument_checks():
    L = binding.lib()
    f = L.csa2_pool_topk
    # (block_max, rows, n_blocks, ld_bm, P_b, out_blocks, scores, ld, k, out_idx, stream)
    assert f(None, 0, 100, 100, 64, None, None, 800, 32, None, None) == 0        # no rows: nothing to do
    assert f(None, 2, 100, 100, 64, None, None, 800, 32, None, None) == 1        # null pointers
    assert "null" in _err()
    assert f(256, 2, 100, 100, 64, 256, 256, 800, 65, 256, None) == 1            # k > P_b
    assert "k <= P_b" in _err()
    assert f(256, 2, 100, 50, 64, 256, 256, 800, 32, 256, None) == 1             # ld_bm < n_blocks
    assert f(256, 2, 100, 100, 4096, 256, 256, 800, 32, 256, None) == 2          # pool above 2,048 blocks
    assert "csa2_topk_from_pool" in _err()
    assert f(256, 2, 40000, 40000, 64, 256, 256, 800, 32, 256, None) == 2        # pool through super-blocks
    assert f(256, 2, 32768, 32768, 64, 256, 256, 800, 32, 256, None) != 2        # largest direct pool


def test_decode_select_argument_checks():
    L = binding.lib()
    a = binding.DecodeSelectArgs(q_idx=256, q_dtype=1, w=256, k_idx=256, k_dtype=1, ctx_len=256, B=4, cap=4096,
                                 H_I=8, d_I=128, P_b=64, k=32, out_pool=256, out_idx=256)
    need = L.csa2_decode_select_workspace_size(ctypes.byref(a))
    assert need >= 4 * 4096 * 4                       # approximate scores of every cache entry
    assert L.csa2_decode_scan(ctypes.byref(a), None, 0, None) == 3
    assert "workspace" in _err()
    assert L.csa2_decode_select(ctypes.byref(a), None, 0, None) == 3
    a.k = 65                                          # k > P_b: the pool would not hold the top-k
    assert L.csa2_decode_scan(ctypes.byref(a), None, 0, None) == 1
    a.k, a.H_I = 32, 4
    assert L.csa2_decode_scan(ctypes.byref(a), None, 0, None) == 2
    a.H_I, a.cap = 8, 262208                          # beyond the one-workgroup selection
    assert L.csa2_decode_scan(ctypes.byref(a), None, 0, None) == 2
    a.cap, a.q_dtype = 4000, 1                        # not a multiple of 64
    assert L.csa2_decode_scan(ctypes.byref(a), None, 0, None) == 1
    a.cap, a.q_dtype = 4096, 0
    assert L.csa2_decode_scan(ctypes.byref(a), None, 0, None) == 2
    a.q_dtype, a.B = 1, 0
    assert L.csa2_decode_scan(ctypes.byref(a), None, 0, None) == 0  # nothing to do


def test_kv_write_project_rejects_bad_arguments_on_host():
    L = binding.lib()
    p = ctypes.c_void_p(256)
    rc = L.csa2_kv_write_project(p, 0, 4, 500, p, 64, p, p, p, 128, p, None)
    assert rc == 1 and "multiple of 16" in _err()
    rc = L.csa2_kv_write_project(p, 0, 4, 512, p, 64, p, p, p, 12, p, None)
    assert rc == 1 and "multiple of 8" in _err()
    rc = L.csa2_kv_write_project(p, 0, 4, 512, p, 100, p, p, p, 128, p, None)
    assert rc == 1 and "% 64" in _err()
    rc = L.csa2_kv_write_project(p, 0, 4, 1024, p, 64, p, p, p, 128, p, None)
    assert rc == 2 and "D <= 512" in _err()
    rc = L.csa2_kv_write_project(p, 0, 4, 512, p, 64, p, p, None, 128, p, None)
    assert rc == 1 and "null" in _err()
    assert L.csa2_kv_write_project(None, 0, 0, 512, None, 64, None, None, None, 128, None, None) == 0


def test_mhc_step_rejects_bad_arguments_on_host():
    L = binding.lib()
    p = ctypes.c_void_p(256).value
    a = binding.MhcArgs(X=p, f=p, A=p, B=p, C=p, phiT=p, bias=p, alpha_pre=1.0, alpha_post=1.0, alpha_res=1.0,
                        T=4, n=3, d=256, iters=20, X_next=p + 4096, u_next=p + 8192, A_next=p, B_next=p, C_next=p)
    assert L.csa2_mhc_step(ctypes.byref(a), None) == 2 and "n = 4" in _err()
    a.n, a.d = 4, 200
    assert L.csa2_mhc_step(ctypes.byref(a), None) == 2
    a.d = 256
    a.X_next = p
    assert L.csa2_mhc_step(ctypes.byref(a), None) == 1 and "alias" in _err()
    a.X_next, a.phiT = p + 4096, None
    assert L.csa2_mhc_step(ctypes.byref(a), None) == 1 and "null" in _err()
    a.T = 0
    assert L.csa2_mhc_step(ctypes.byref(a), None) == 0


def test_noalloc_attention_rejects_calls_beyond_its_scratch_on_host():
    L = binding.lib()
    a = binding.AttnArgs(q=16, q_dtype=1, codes=16, scales=16, cap=1 << 20, idx=16, k=2048, swa=16,
                         swa_dtype=1, W=128, swa_len=16, B=1408, H=64, D=512, sm_scale=0.1, out=16)
    need = L.csa2_sparse_attn_decode_workspace_size(ctypes.byref(a))
    limit = 64 << 20
    assert need > limit
    assert L.csa2_sparse_attn_decode_noalloc(ctypes.byref(a), None) == 3
    assert "scratch" in _err() and str(limit) in _err()
    a.H = 48
    assert L.csa2_sparse_attn_decode_noalloc(ctypes.byref(a), None) == 2
    assert L.csa2_sparse_attn_decode_noalloc(None, None) == 1
    a.H, a.B = 64, 0
    assert L.csa2_sparse_attn_decode_noalloc(ctypes.byref(a), None) == 0    # nothing to do


def test_write_and_score_argument_checks():
    L = binding.lib()
    P = 1 << 12                 # stands in for a device address: only host checks run
    a = binding.ScoreArgs(q_idx=P, q_dtype=1, w=P, k_idx=P, k_dtype=1, B=2, Tq=1, cap=128,
                     H_I=8, d_I=128, ctx_len=P, q_pos=None, m=1, pool_blocks=None, P_b=0, scores=P,
                     ld_scores=128, block_max=None)
    call = lambda D=512, x=P, dst=P, kr=P, dt=1: L.csa2_write_and_score(
        x, dt, D, dst, P, P, kr, ctypes.byref(a), None, 0, None)
    assert call(D=8) == 1 and "multiple of 16" in _err()
    assert call(dt=7) == 1
    assert call(x=None) == 1 and "null" in _err()
    assert call(kr=None) == 1
    assert call(kr=P + 8) == 1 and "aligned" in _err()
    # one workgroup writes a row: D/16 blocks plus 16 indexer chunks must fit 256 threads
    assert call(D=4096) == 2
    a.Tq = 2
    assert call() == 1 and "Tq" in _err()
    a.Tq, a.cap = 1, 100
    assert call() == 1       # the scan's own checks (tiled cache needs cap % 64 == 0)
    a.cap, a.B = 128, 0
    assert call() == 0
