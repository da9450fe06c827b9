"""Host-side composition of CSA2 decode layers over one shared KV set.

Layer modes ("DeepSeek-V4.1-Flash KV Cache Compression" notes, section 2;
"...reading a model through its three memory costs", section 03 table):
  F  Full:    score every visible entry, take top-k, attend; the first Full
              layer of the decoder also builds the candidate pool (block max
              over 8 positions, top 2,048 blocks; notes section 3).
  X  Reindex: score only the pool with the layer's own indexer query, take
              top-k inside it, attend.
  R  Reuse:   attend with the index list (and KV set) of the preceding F,
              X or E layer.
  E  encoder Full: the same as F over an encoder KV set of its own, whose
              entries each compress m = 2 tokens, so the token at absolute
              position i sees min(ctx_len, floor((i + 1) / m)) entries (notes
              section 2: the encoder compresses every m tokens and only
              complete entries are visible).  It builds no pool (the encoder
              has no Reindex layers); its top-k is taken inside a pool of
              its own block maxima, which is exact for k <= P_b.
Every layer attends with its own query and its own sliding-window KV; the
decoder's layers read the decoder's MXFP4 main-KV and indexer-K caches, an
encoder Full layer and the Reuse layers after it read that layer's set.

DecodeStep pre-binds the ctypes argument structs of every library call of a
step once, so a step costs one C call per kernel group and no Python-side
allocation.  All arithmetic happens in libcsa2.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch

from . import binding as bd


@dataclass
class LayerInputs:
    q: torch.Tensor                      # [B][H][D] bf16
    swa: torch.Tensor                    # [B][W][D] bf16
    q_idx: Optional[torch.Tensor] = None  # [B][1][H_I][d_I] (F and X layers)
    w: Optional[torch.Tensor] = None      # [B][1][H_I] f32


@dataclass
class DecodeCache:
    codes: torch.Tensor       # [B][cap][D/2] u8
    scales: torch.Tensor      # [B][cap][D/16] u8
    k_idx: torch.Tensor       # [B][cap][d_I]
    ctx_len: torch.Tensor     # [B] int32 (entries visible after this step's write)
    swa_len: torch.Tensor     # [B] int32


class DecodeStep:
    """One decode token for B sequences through a layer schedule.

    schedule: string over {F, X, R}; the first F builds the pool when
    build_pool is set (X layers need a pool: built here or passed in).
    new_kv / new_kidx / dst_row: the token's main-KV row and indexer-K row,
    written first (mxfp4_kv_write) so the new entry is visible to scoring.
    mfma_select: the Full layer that builds the pool scores on the matrix
    cores and selects with exact rescoring near the thresholds
    (csa2_decode_scan + csa2_decode_select) where that path applies (8 x 128
    bf16 indexer, cap <= 262,144, k <= P_b <= 2048); the results are the same
    as the exact scan's.  Off by default: on MI355X at 128K x 8 rows its scan
    is only 3 us faster than the exact one, while its one-workgroup-per-row
    selection (band rescoring) takes about 73 us against 26 us for the fused
    pool/top-k.
    """

    def __init__(self, schedule: str, cache: DecodeCache, layers: List[LayerInputs], *, k: int,
                 P_b: int = 2048, new_kv: Optional[torch.Tensor] = None,
                 new_kidx: Optional[torch.Tensor] = None, dst_row: Optional[torch.Tensor] = None,
                 pool: Optional[torch.Tensor] = None, sm_scale: Optional[float] = None,
                 build_pool: bool = True, mfma_select: bool = False,
                 enc_caches: Optional[List[DecodeCache]] = None, enc_q_pos: Optional[torch.Tensor] = None,
                 enc_m: int = 2, enc_writes: Optional[List[Optional[tuple]]] = None,
                 w_ik: Optional[torch.Tensor] = None, fuse_write: bool = True):
        """w_ik: [D][d_I] float32 indexer-K projection weights; when given, the
        token's indexer key is projected from new_kv in the same launch as its
        MXFP4 write (csa2_kv_write_project) instead of passed as new_kidx.
        enc_caches: one KV set per E layer, in schedule order.
        enc_q_pos: [B] int64 absolute position of the token in each sequence
        (E layers' visibility).  enc_writes: per E layer, None or
        (new_kv [B][D], new_kidx [B][d_I], dst_row [B] int64) for an entry
        the token completes, written before any scoring.
        fuse_write: when the step's first call after the write is the scan
        of the main cache, do both in one launch (csa2_write_and_score); then
        dst_row[b] must address a row of sequence b (other rows are not
        written), as a decode token's entry always does."""
        assert len(schedule) == len(layers)
        n_enc = schedule.count("E")
        enc_caches = list(enc_caches or [])
        if len(enc_caches) != n_enc:
            raise ValueError(f"schedule has {n_enc} encoder Full layers but {len(enc_caches)} encoder caches")
        if n_enc and enc_q_pos is None:
            raise ValueError("encoder Full layers need enc_q_pos")
        if enc_writes is not None and len(enc_writes) != n_enc:
            raise ValueError("enc_writes needs one entry per encoder Full layer")
        self.schedule, self.cache, self.layers, self.k, self.P_b = schedule, cache, layers, k, P_b
        B, cap, half = cache.codes.shape
        D = half * 2
        d_I = cache.k_idx.shape[-1]
        dev = cache.codes.device
        self.B, self.cap, self.D = B, cap, D
        self.L = bd.lib()
        self.calls = []          # (name, fn, args) in launch order
        self._fusable_write = None
        self.sm_scale = sm_scale if sm_scale is not None else 1.0 / math.sqrt(D)
        self._keep = []          # keep ctypes structs and tensors alive

        # ---- write of the new token's entry
        if new_kv is not None and w_ik is not None:
            if new_kidx is not None:
                raise ValueError("pass either new_kidx or w_ik, not both")
            if w_ik.dtype != torch.float32 or tuple(w_ik.shape) != (D, d_I) or not w_ik.is_contiguous():
                raise ValueError("w_ik must be a contiguous float32 [D][d_I] tensor")
            if cache.k_idx.dtype != torch.bfloat16:
                raise ValueError("projected indexer keys go to a bfloat16 indexer cache")
            args = (bd._ptr(new_kv), bd._dtype(new_kv, "new_kv"), new_kv.shape[0], D, bd._ptr(dst_row),
                    B * cap, bd._ptr(cache.codes), bd._ptr(cache.scales), bd._ptr(w_ik), d_I,
                    bd._ptr(cache.k_idx), None)
            self.calls.append(("write", self.L.csa2_kv_write_project, args))
        elif new_kv is not None:
            n_cache_rows = B * cap
            kdt = bd._dtype(new_kidx, "new_kidx") if new_kidx is not None else 0
            args = (bd._ptr(new_kv), bd._dtype(new_kv, "new_kv"), new_kv.shape[0], D, bd._ptr(dst_row),
                    n_cache_rows, bd._ptr(cache.codes), bd._ptr(cache.scales), bd._ptr(new_kidx), kdt,
                    d_I if new_kidx is not None else 0, bd._ptr(cache.k_idx), None)
            self.calls.append(("write", self.L.mxfp4_kv_write, args))
            nch = d_I * new_kidx.element_size() // 16 if new_kidx is not None else 0
            if (fuse_write and new_kidx is not None and new_kv.shape[0] == B and D // 16 + nch <= 256
                    and new_kidx.dtype == cache.k_idx.dtype and tuple(new_kidx.shape) == (B, d_I)):
                # (x, x_dtype, D, dst_row, codes, scales, idx_k_rows): the
                # write half of csa2_write_and_score
                self._fusable_write = (bd._ptr(new_kv), bd._dtype(new_kv, "new_kv"), D, bd._ptr(dst_row),
                                       bd._ptr(cache.codes), bd._ptr(cache.scales), bd._ptr(new_kidx))
        for ei, wr in enumerate(enc_writes or []):
            if wr is None:
                continue
            ec = enc_caches[ei]
            e_kv, e_kidx, e_dst = wr
            e_cap = ec.codes.shape[1]
            args = (bd._ptr(e_kv), bd._dtype(e_kv, "enc new_kv"), e_kv.shape[0], D, bd._ptr(e_dst),
                    B * e_cap, bd._ptr(ec.codes), bd._ptr(ec.scales), bd._ptr(e_kidx),
                    bd._dtype(e_kidx, "enc new_kidx"), ec.k_idx.shape[-1], bd._ptr(ec.k_idx), None)
            self.calls.append((f"write_enc{ei}", self.L.mxfp4_kv_write, args))

        self.scores = torch.empty((B, 1, cap), dtype=torch.float32, device=dev)
        self.block_max = torch.empty((B, 1, (cap + 7) // 8), dtype=torch.float32, device=dev)
        self.pool = pool if pool is not None else torch.full((B, 1, P_b), -1, dtype=torch.int32, device=dev)
        self.pool_scores = torch.empty((B, 1, 8 * P_b), dtype=torch.float32, device=dev)
        self.outs = [torch.empty((B, l.q.shape[1], D), dtype=torch.float32, device=dev) for l in layers]
        self.idx_bufs = []
        pool_built = pool is not None
        cur_idx = None
        cur_cache = cache
        n_e = 0
        for li, (mode, lay) in enumerate(zip(schedule, layers)):
            if mode == "E":
                ec = enc_caches[n_e]
                n_e += 1
                cur_idx = self._encoder_full(li, lay, ec, enc_q_pos, enc_m, k, P_b)
                cur_cache = ec
                self._attn(li, lay, cur_idx, cur_cache)
                continue
            if mode in "FX":
                cur_cache = cache
                idx = torch.empty((B, 1, k), dtype=torch.int32, device=dev)
                self.idx_bufs.append(idx)
                use_pool = mode == "X"
                if use_pool and not pool_built:
                    raise ValueError("a Reindex layer needs a pool from an earlier Full layer")
                want_bm = mode == "F" and build_pool and not pool_built
                if (want_bm and mfma_select and lay.q_idx.dtype == torch.bfloat16
                        and cache.k_idx.dtype == torch.bfloat16 and lay.q_idx.shape[-2:] == (8, 128)
                        and cap % 64 == 0 and cap <= 262144 and k <= P_b <= 2048):
                    da = bd.DecodeSelectArgs(
                        q_idx=lay.q_idx.data_ptr(), q_dtype=bd.CSA2_BF16, w=lay.w.data_ptr(),
                        k_idx=cache.k_idx.data_ptr(), k_dtype=bd.CSA2_BF16, ctx_len=cache.ctx_len.data_ptr(),
                        B=B, cap=cap, H_I=8, d_I=128, P_b=P_b, k=k, out_pool=self.pool.data_ptr(),
                        out_idx=idx.data_ptr())
                    dn = self.L.csa2_decode_select_workspace_size(ctypes.byref(da))
                    dws = torch.empty(max(dn, 256), dtype=torch.uint8, device=dev)
                    self._keep += [da, dws]
                    self.calls.append((f"score{li}", self.L.csa2_decode_scan, (ctypes.byref(da), bd._ptr(dws), dn, None)))
                    self.calls.append((f"pool{li}", self.L.csa2_decode_select,
                                       (ctypes.byref(da), bd._ptr(dws), dn, None)))
                    pool_built = True
                    cur_idx = idx
                    self._attn(li, lay, cur_idx, cur_cache)
                    continue
                sa = bd.ScoreArgs(
                    q_idx=lay.q_idx.data_ptr(), q_dtype=bd._dtype(lay.q_idx, "q_idx"), w=lay.w.data_ptr(),
                    k_idx=cache.k_idx.data_ptr(), k_dtype=bd._dtype(cache.k_idx, "k_idx"), B=B, Tq=1,
                    cap=cap, H_I=lay.q_idx.shape[2], d_I=d_I, ctx_len=cache.ctx_len.data_ptr(), q_pos=None,
                    m=1, pool_blocks=self.pool.data_ptr() if use_pool else None,
                    P_b=P_b if use_pool else 0,
                    scores=(self.pool_scores if use_pool else self.scores).data_ptr(),
                    ld_scores=8 * P_b if use_pool else cap,
                    block_max=self.block_max.data_ptr() if want_bm else None)
                nws = self.L.csa2_index_score_workspace_size(ctypes.byref(sa))
                ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)
                self._keep += [sa, ws]
                if self._fusable_write is not None and len(self.calls) == 1 and self.calls[0][0] == "write":
                    # nothing runs between the write and this scan: one launch
                    self.calls[0] = (f"score{li}", self.L.csa2_write_and_score,
                                     self._fusable_write + (ctypes.byref(sa), bd._ptr(ws), nws, None))
                else:
                    self.calls.append((f"score{li}", self.L.csa2_index_score,
                                       (ctypes.byref(sa), bd._ptr(ws), nws, None)))
                fused = False
                # The Full top-k may be taken inside a pool only when that pool
                # was selected from this same layer's block maxima (the top-k
                # lies inside its own layer's pool for k <= P_b).  A pool from
                # another layer's scores, or one passed in, says nothing about
                # this layer's scores, so a later Full layer selects over the
                # whole visible context.
                own_pool = False
                if want_bm:
                    nb = (cap + 7) // 8
                    fused = k <= P_b <= 2048 and nb <= 32768
                if fused:
                    # pool and the Full top-k inside it in one launch
                    self.calls.append((f"pool{li}", self.L.csa2_pool_topk,
                                       (bd._ptr(self.block_max), B, nb, nb, P_b, bd._ptr(self.pool),
                                        bd._ptr(self.scores), cap, k, bd._ptr(idx), None)))
                    pool_built = True
                    own_pool = True
                elif want_bm:
                    pws_n = self.L.csa2_build_candidate_pool_workspace_size(B, nb, P_b)
                    pws = torch.empty(max(pws_n, 256), dtype=torch.uint8, device=dev)
                    self._keep.append(pws)
                    self.calls.append((f"pool{li}", self.L.csa2_build_candidate_pool,
                                       (bd._ptr(self.block_max), B, nb, nb, P_b,
                                        bd._ptr(self.pool), bd._ptr(pws), pws_n, None)))
                    pool_built = True
                    own_pool = True
                if fused:
                    pass
                elif mode == "F" and own_pool and k <= P_b and 8 * P_b <= 32768:
                    # the Full top-k lies inside the pool: select among its 8*P_b scores
                    self.calls.append((f"topk{li}", self.L.csa2_topk_from_pool,
                                       (bd._ptr(self.scores), B, cap, bd._ptr(self.pool), P_b, k,
                                        bd._ptr(idx), None)))
                else:
                    src = self.pool_scores if use_pool else self.scores
                    n = 8 * P_b if use_pool else cap
                    tws_n = self.L.csa2_topk_workspace_size(B, n, k)
                    tws = torch.empty(max(tws_n, 256), dtype=torch.uint8, device=dev)
                    self._keep.append(tws)
                    self.calls.append((f"topk{li}", self.L.csa2_topk,
                                       (bd._ptr(src), B, n, n, k, bd._ptr(self.pool) if use_pool else None,
                                        P_b if use_pool else 0, bd._ptr(idx), bd._ptr(tws), tws_n, None)))
                cur_idx = idx
            elif mode == "R":
                if cur_idx is None:
                    raise ValueError("a Reuse layer needs an earlier Full, Reindex or encoder Full layer")
            else:
                raise ValueError(f"unknown layer mode {mode!r}")
            self._attn(li, lay, cur_idx, cur_cache)

    def _encoder_full(self, li: int, lay: "LayerInputs", ec: DecodeCache, q_pos: torch.Tensor, m: int,
                      k: int, P_b: int) -> torch.Tensor:
        """Score every visible entry of the encoder set (q_pos, m visibility),
        then its top-k; returns the index buffer."""
        B = self.B
        dev = ec.codes.device
        e_cap = ec.codes.shape[1]
        d_I = ec.k_idx.shape[-1]
        nb = (e_cap + 7) // 8
        idx = torch.empty((B, 1, k), dtype=torch.int32, device=dev)
        self.idx_bufs.append(idx)
        scores = torch.empty((B, 1, e_cap), dtype=torch.float32, device=dev)
        bm = torch.empty((B, 1, nb), dtype=torch.float32, device=dev)
        qp = q_pos.to(device=dev, dtype=torch.int64).reshape(B, 1).contiguous()
        inner = k <= P_b and 8 * P_b <= 32768        # top-k inside a pool of its own
        sa = bd.ScoreArgs(
            q_idx=lay.q_idx.data_ptr(), q_dtype=bd._dtype(lay.q_idx, "q_idx"), w=lay.w.data_ptr(),
            k_idx=ec.k_idx.data_ptr(), k_dtype=bd._dtype(ec.k_idx, "k_idx"), B=B, Tq=1,
            cap=e_cap, H_I=lay.q_idx.shape[2], d_I=d_I, ctx_len=ec.ctx_len.data_ptr(), q_pos=qp.data_ptr(),
            m=m, pool_blocks=None, P_b=0, scores=scores.data_ptr(), ld_scores=e_cap,
            block_max=bm.data_ptr() if inner else None)
        nws = self.L.csa2_index_score_workspace_size(ctypes.byref(sa))
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)
        self._keep += [sa, ws, scores, bm, qp]
        self.calls.append((f"score{li}", self.L.csa2_index_score, (ctypes.byref(sa), bd._ptr(ws), nws, None)))
        if inner:
            epool = torch.empty((B, 1, P_b), dtype=torch.int32, device=dev)
            self._keep.append(epool)
            if P_b <= 2048 and nb <= 32768:
                self.calls.append((f"pool{li}", self.L.csa2_pool_topk,
                                   (bd._ptr(bm), B, nb, nb, P_b, bd._ptr(epool), bd._ptr(scores), e_cap, k,
                                    bd._ptr(idx), None)))
            else:
                pws_n = self.L.csa2_build_candidate_pool_workspace_size(B, nb, P_b)
                pws = torch.empty(max(pws_n, 256), dtype=torch.uint8, device=dev)
                self._keep.append(pws)
                self.calls.append((f"pool{li}", self.L.csa2_build_candidate_pool,
                                   (bd._ptr(bm), B, nb, nb, P_b, bd._ptr(epool), bd._ptr(pws), pws_n, None)))
                self.calls.append((f"topk{li}", self.L.csa2_topk_from_pool,
                                   (bd._ptr(scores), B, e_cap, bd._ptr(epool), P_b, k, bd._ptr(idx), None)))
        else:
            tws_n = self.L.csa2_topk_workspace_size(B, e_cap, k)
            tws = torch.empty(max(tws_n, 256), dtype=torch.uint8, device=dev)
            self._keep.append(tws)
            self.calls.append((f"topk{li}", self.L.csa2_topk,
                               (bd._ptr(scores), B, e_cap, e_cap, k, None, 0, bd._ptr(idx), bd._ptr(tws),
                                tws_n, None)))
        return idx

    def _attn(self, li: int, lay: "LayerInputs", cur_idx: torch.Tensor, cache: DecodeCache) -> None:
        B, D, k = self.B, self.D, self.k
        cap = cache.codes.shape[1]
        aa = bd.AttnArgs(q=lay.q.data_ptr(), q_dtype=bd._dtype(lay.q, "q"), codes=cache.codes.data_ptr(),
                         scales=cache.scales.data_ptr(), cap=cap, idx=cur_idx.data_ptr(), k=k,
                         swa=lay.swa.data_ptr(), swa_dtype=bd._dtype(lay.swa, "swa"), W=lay.swa.shape[1],
                         swa_len=cache.swa_len.data_ptr(), B=B, H=lay.q.shape[1], D=D,
                         sm_scale=self.sm_scale, out=self.outs[li].data_ptr())
        nws = self.L.csa2_sparse_attn_decode_workspace_size(ctypes.byref(aa))
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=cache.codes.device)
        self._keep += [aa, ws]
        self.calls.append((f"attn{li}", self.L.csa2_sparse_attn_decode,
                           (ctypes.byref(aa), bd._ptr(ws), nws, None)))
        self.layer_idx = cur_idx

    def capture(self):
        """Record one step into a HIP graph (torch.cuda.CUDAGraph) and return
        it; graph.replay() then enqueues the whole step with one launch.  The
        step allocates nothing and uses no memset, so every replay repeats
        exactly the recorded kernels on the pre-bound buffers."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.run()                      # warm-up on the capture stream
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            self.run()
        return graph

    def run(self, stream=None, events=None):
        """Enqueue the whole step on `stream` (default: torch's current).
        events: optional dict name -> (start_event, end_event) to bracket calls."""
        st = bd._stream(stream)
        for name, fn, args in self.calls:
            args = args[:-1] + (st,)
            ev = events.get(name) if events else None
            if ev is not None:
                ev[0].record()
            rc = fn(*args)
            if ev is not None:
                ev[1].record()
            if rc != 0:
                raise RuntimeError(f"{name}: libcsa2 error {rc}: {self.L.csa2_last_error().decode()}")
