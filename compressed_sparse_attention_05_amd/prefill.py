"""Host-side composition of one prefill chunk through an encoder layer schedule.

An encoder block ("DeepSeek-V4.1-Flash KV Cache Compression" notes, section 2;
"...reading a model through its three memory costs", section 03) has one
Full layer followed by Reuse layers (schedule "FRRRRR").  For a chunk of T
query tokens at positions q_pos0 .. q_pos0+T-1 with m tokens per entry:

  1. mxfp4_kv_write appends the chunk's complete entries (main KV and
     indexer K) so they are visible to the chunk's later tokens;
  2. the Full layer selects, per token, the top-k of the entries visible to it
     (csa2_prefill_topk: vis(t) = min(ctx_len, floor((q_pos0 + t + 1) / m)));
  3. every layer attends with its own queries over the selected entries plus
     the token's own window [i - W + 1, i] of sliding-window rows
     (csa2_sparse_attn_prefill); Reuse layers keep the Full layer's indices.

All arithmetic happens in libcsa2; this module pre-binds the ctypes argument
structs and workspaces once so a run is one C call per kernel group.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass
from typing import List, Optional

import torch

from . import binding as bd


@dataclass
class PrefillLayer:
    q: torch.Tensor                       # [T][H][D] bf16
    swa: torch.Tensor                     # [T + W - 1][D] bf16 (row r = token q_pos0 - (W-1) + r)
    q_idx: Optional[torch.Tensor] = None  # [T][8][128] bf16 (Full layer)
    w: Optional[torch.Tensor] = None      # [T][8] f32 (Full layer)


class PrefillChunk:
    def __init__(self, schedule: str, codes: torch.Tensor, scales: torch.Tensor, k_idx: torch.Tensor,
                 ctx_len: int, q_pos0: int, m: int, k: int, W: int, layers: List[PrefillLayer], *,
                 new_kv: Optional[torch.Tensor] = None, new_kidx: Optional[torch.Tensor] = None,
                 dst_row: Optional[torch.Tensor] = None, swa_start: int = 0,
                 sm_scale: Optional[float] = None, outs: Optional[List[torch.Tensor]] = None):
        """outs: optional per-layer outputs, each [T][H][D] float32; every layer
        writes its own (a Reuse layer attends with its own queries and window,
        so its output differs from the Full layer's)."""
        if len(schedule) != len(layers) or not schedule or schedule[0] != "F" or set(schedule[1:]) - {"R"}:
            raise ValueError("an encoder chunk schedule is one Full layer then Reuse layers")
        cap, half = codes.shape
        D = 2 * half
        d_I = k_idx.shape[-1]
        T = layers[0].q.shape[0]
        dev = codes.device
        self.L = bd.lib()
        self.calls = []
        self._keep = []
        if new_kv is not None:
            kdt = bd._dtype(new_kidx, "new_kidx") if new_kidx is not None else 0
            self.calls.append(("write", self.L.mxfp4_kv_write,
                               (bd._ptr(new_kv), bd._dtype(new_kv, "new_kv"), new_kv.shape[0], D,
                                bd._ptr(dst_row), cap, bd._ptr(codes), bd._ptr(scales), bd._ptr(new_kidx),
                                kdt, d_I if new_kidx is not None else 0, bd._ptr(k_idx), None)))
        self.idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        f = layers[0]
        pa = bd.PrefillTopkArgs(q_idx=f.q_idx.data_ptr(), q_dtype=bd._dtype(f.q_idx, "q_idx"), w=f.w.data_ptr(),
                                k_idx=k_idx.data_ptr(), k_dtype=bd._dtype(k_idx, "k_idx"), T=T, cap=cap,
                                H_I=f.q_idx.shape[1], d_I=d_I, ctx_len=int(ctx_len), q_pos0=int(q_pos0),
                                m=int(m), k=int(k), out_idx=self.idx.data_ptr())
        nws = self.L.csa2_prefill_topk_workspace_size(ctypes.byref(pa))
        ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
        self._keep += [pa, ws]
        self.calls.append(("topk", self.L.csa2_prefill_topk, (ctypes.byref(pa), bd._ptr(ws), nws, None)))
        if outs is not None and len(outs) != len(layers):
            raise ValueError("outs needs one [T][H][D] tensor per layer")
        self.outs = list(outs) if outs is not None else [
            torch.empty((T, lay.q.shape[1], D), dtype=torch.float32, device=dev) for lay in layers]
        for o, lay in zip(self.outs, layers):
            if (o.dtype != torch.float32 or tuple(o.shape) != (T, lay.q.shape[1], D) or not o.is_contiguous()
                    or o.device != dev):
                raise ValueError("each layer output must be a contiguous float32 [T][H][D] tensor on the cache's device")
        if len({o.data_ptr() for o in self.outs}) != len(self.outs):
            raise ValueError("layer outputs must not share memory")
        scale = sm_scale if sm_scale is not None else 1.0 / math.sqrt(D)
        for li, lay in enumerate(layers):
            aa = bd.AttnPrefillArgs(q=lay.q.data_ptr(), q_dtype=bd._dtype(lay.q, "q"), codes=codes.data_ptr(),
                                    scales=scales.data_ptr(), cap=cap, idx=self.idx.data_ptr(), k=k,
                                    swa=lay.swa.data_ptr(), swa_dtype=bd._dtype(lay.swa, "swa"), W=W,
                                    q_pos0=int(q_pos0), swa_start=int(swa_start), T=T, H=lay.q.shape[1], D=D,
                                    sm_scale=scale, out=self.outs[li].data_ptr())
            n = self.L.csa2_sparse_attn_prefill_workspace_size(ctypes.byref(aa))
            aws = torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
            self._keep += [aa, aws]
            self.calls.append((f"attn{li}", self.L.csa2_sparse_attn_prefill,
                               (ctypes.byref(aa), bd._ptr(aws), n, None)))

    def run(self, stream=None, events=None):
        """Enqueue the chunk on `stream`; events: name -> (start, end) events."""
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
