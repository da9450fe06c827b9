"""Host-side composition of the decoder over a replayed window of tokens.

SWA bounded replay ("DeepSeek-V4.1-Flash KV Cache Compression" notes,
section 5): after a cache miss on local state, only the most recent
n_win = 128 tokens are run again, and each layer's sliding window is cut to
the replayed segment, [max(s, i - n_win + 1), i] for the token at position
i with replay start s.  The global KV of those tokens is already cached, so
the decoder's forward pass over the segment is T = n_win queries against
that cache, every query a decoder query of its own:

  F  Full:    score the entries visible to the token (min(ctx_len, i + 1)
              at m = 1), build the token's candidate pool (top P_b blocks of
              8 by block max; notes section 3), and take its top-k, which
              lies inside its pool when k <= P_b;
  X  Reindex: score the token's own pool with the layer's indexer query and
              take the top-k inside it;
  R  Reuse:   the index list of the preceding F or X layer.
Every layer attends with its own queries over the selected entries plus the
token's window rows from the replay start on (csa2_sparse_attn_prefill with
swa_start = s).

All arithmetic happens in libcsa2; the calls are pre-bound once, so a run is
one C call per kernel group.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass
from typing import List, Optional

import torch

from . import binding as bd


@dataclass
class ReplayLayer:
    q: torch.Tensor                       # [T][H][D] bf16
    swa: torch.Tensor                     # [T + W - 1][D] bf16 (row r = token q_pos0 - (W-1) + r)
    q_idx: Optional[torch.Tensor] = None  # [T][H_I][d_I] (F and X layers)
    w: Optional[torch.Tensor] = None      # [T][H_I] f32


class DecoderReplay:
    """The decoder's layers over T replayed tokens of one sequence at
    positions q_pos0 .. q_pos0 + T - 1 (q_pos0 is the replay start s).

    codes [cap][D/2], scales [cap][D/16]: the sequence's MXFP4 main KV;
    k_idx [cap][d_I]: its tiled indexer-K cache; ctx_len: entries cached.
    Outputs: idx[li] [T][k] per F/X layer, pool [T][P_b], out[li] [T][H][D]."""

    def __init__(self, schedule: str, codes: torch.Tensor, scales: torch.Tensor, k_idx: torch.Tensor,
                 ctx_len: int, q_pos0: int, k: int, W: int, layers: List[ReplayLayer], *,
                 P_b: int = 2048, sm_scale: Optional[float] = None):
        if len(schedule) != len(layers) or not schedule or schedule[0] != "F" or set(schedule) - set("FXR"):
            raise ValueError("a decoder replay schedule starts with a Full layer and uses F, X and R")
        if k > P_b:
            raise ValueError("the replay selects the Full top-k inside each token's pool: need k <= P_b")
        cap, half = codes.shape
        D = 2 * half
        d_I = k_idx.shape[-1]
        T = layers[0].q.shape[0]
        dev = codes.device
        self.L = bd.lib()
        self.calls = []
        self._keep = []
        self.T, self.k, self.P_b = T, k, P_b
        nb = (cap + 7) // 8
        ctx_t = torch.tensor([ctx_len], dtype=torch.int32, device=dev)
        q_pos = (q_pos0 + torch.arange(T, dtype=torch.int64, device=dev)).reshape(1, T).contiguous()
        self.scores = torch.empty((T, cap), dtype=torch.float32, device=dev)
        self.block_max = torch.empty((T, nb), dtype=torch.float32, device=dev)
        self.pool = torch.empty((T, P_b), dtype=torch.int32, device=dev)
        self.pool_scores = torch.empty((T, 8 * P_b), dtype=torch.float32, device=dev)
        self._keep += [ctx_t, q_pos]
        self.idx = {}
        self.out = [torch.empty((T, l.q.shape[1], D), dtype=torch.float32, device=dev) for l in layers]
        scale = sm_scale if sm_scale is not None else 1.0 / math.sqrt(D)
        cur = None
        for li, (mode, lay) in enumerate(zip(schedule, layers)):
            if mode in "FX":
                full = mode == "F"
                idx = torch.empty((T, k), dtype=torch.int32, device=dev)
                self.idx[li] = idx
                sa = bd.ScoreArgs(
                    q_idx=lay.q_idx.data_ptr(), q_dtype=bd._dtype(lay.q_idx, "q_idx"), w=lay.w.data_ptr(),
                    k_idx=k_idx.data_ptr(), k_dtype=bd._dtype(k_idx, "k_idx"), B=1, Tq=T, cap=cap,
                    H_I=lay.q_idx.shape[1], d_I=d_I, ctx_len=ctx_t.data_ptr(), q_pos=q_pos.data_ptr(), m=1,
                    pool_blocks=None if full else self.pool.data_ptr(), P_b=0 if full else P_b,
                    scores=(self.scores if full else self.pool_scores).data_ptr(),
                    ld_scores=cap if full else 8 * P_b,
                    block_max=self.block_max.data_ptr() if full else None)
                nws = self.L.csa2_index_score_workspace_size(ctypes.byref(sa))
                ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)
                self._keep += [sa, ws]
                self.calls.append((f"score{li}", self.L.csa2_index_score, (ctypes.byref(sa), bd._ptr(ws), nws, None)))
                if full and P_b <= 2048 and nb <= 32768:
                    # each token's pool and its top-k inside it, one launch
                    self.calls.append((f"pool{li}", self.L.csa2_pool_topk,
                                       (bd._ptr(self.block_max), T, nb, nb, P_b, bd._ptr(self.pool),
                                        bd._ptr(self.scores), cap, k, bd._ptr(idx), None)))
                elif full:
                    pws_n = self.L.csa2_build_candidate_pool_workspace_size(T, nb, P_b)
                    pws = torch.empty(max(pws_n, 256), dtype=torch.uint8, device=dev)
                    self._keep.append(pws)
                    self.calls.append((f"pool{li}", self.L.csa2_build_candidate_pool,
                                       (bd._ptr(self.block_max), T, nb, nb, P_b, bd._ptr(self.pool),
                                        bd._ptr(pws), pws_n, None)))
                    self.calls.append((f"topk{li}", self.L.csa2_topk_from_pool,
                                       (bd._ptr(self.scores), T, cap, bd._ptr(self.pool), P_b, k, bd._ptr(idx),
                                        None)))
                else:
                    n = 8 * P_b
                    tws_n = self.L.csa2_topk_workspace_size(T, n, k)
                    tws = torch.empty(max(tws_n, 256), dtype=torch.uint8, device=dev)
                    self._keep.append(tws)
                    self.calls.append((f"topk{li}", self.L.csa2_topk,
                                       (bd._ptr(self.pool_scores), T, n, n, k, bd._ptr(self.pool), P_b,
                                        bd._ptr(idx), bd._ptr(tws), tws_n, None)))
                cur = idx
            aa = bd.AttnPrefillArgs(q=lay.q.data_ptr(), q_dtype=bd._dtype(lay.q, "q"), codes=codes.data_ptr(),
                                    scales=scales.data_ptr(), cap=cap, idx=cur.data_ptr(), k=k,
                                    swa=lay.swa.data_ptr(), swa_dtype=bd._dtype(lay.swa, "swa"), W=W,
                                    q_pos0=int(q_pos0), swa_start=int(q_pos0), T=T, H=lay.q.shape[1], D=D,
                                    sm_scale=scale, out=self.out[li].data_ptr())
            n = self.L.csa2_sparse_attn_prefill_workspace_size(ctypes.byref(aa))
            aws = torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
            self._keep += [aa, aws]
            self.calls.append((f"attn{li}", self.L.csa2_sparse_attn_prefill, (ctypes.byref(aa), bd._ptr(aws), n, None)))

    def run(self, stream=None, events=None):
        """Enqueue the replay on `stream`; events: name -> (start, end) events."""
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
