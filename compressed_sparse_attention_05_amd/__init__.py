"""MI355X (gfx950) CSA2 global-attention hot path of DeepSeek-V4.1-Flash.

The work runs in libcsa2.so (hand-written HIP kernels behind the C ABI in
include/csa2.h); this package is its Python binding plus the host-side
composition of the three layer modes (Full, Reindex, Reuse).
"""
from .binding import (CSA2_BF16, CSA2_F32, csa2_build_candidate_pool, csa2_index_score,
                      csa2_kv_write_project, csa2_mhc_step, csa2_decode_select, csa2_pool_topk, csa2_prefill_topk, csa2_sparse_attn_decode, csa2_sparse_attn_prefill, csa2_topk,
                      csa2_topk_from_pool, csa2_write_and_score, lib,
                      mxfp4_kv_write, tile_indexer_cache, untile_indexer_cache, version)

__all__ = ["CSA2_BF16", "CSA2_F32", "csa2_build_candidate_pool", "csa2_index_score",
           "csa2_kv_write_project", "csa2_mhc_step", "csa2_decode_select", "csa2_pool_topk", "csa2_prefill_topk", "csa2_sparse_attn_decode", "csa2_sparse_attn_prefill", "csa2_topk",
           "csa2_topk_from_pool", "csa2_write_and_score", "lib",
           "mxfp4_kv_write", "tile_indexer_cache", "untile_indexer_cache", "version"]
