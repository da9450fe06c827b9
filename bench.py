#!/usr/bin/env python3
"""Benchmark of the CSA2 decode hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-secondary]

A step is one decode token for B sequences through the whole path of the
workload's layer schedule: mxfp4_kv_write of the token's entry, the Full
scan with fused block max, the candidate pool, top-k and the sparse
attention (plus Reindex/Reuse layers where the schedule has them).  Inputs
are seeded synthetic tensors (csa2_inputs) already resident in HBM; two
independent input sets alternate so the 256 MiB MALL cannot serve a step
from the previous one.  Each input set's step is captured once into a HIP
graph and the timed steps are graph replays; a second pass launches the same
steps kernel group by kernel group, with HIP events around the scan, for the
roofline and for "eager_ms_per_step".

Prints ONE JSON line: queries/s for the workload, the dominant kernel's
roofline (the Full-mode indexer scan, timed live with HIP events on the
stream it runs on), the CPU oracle timed on a bounded sample, and under
"secondary" the 1M-context decode workloads (decoder block 2 with its
Reindex layer, the decoder's 20-layer step at B=64, and the 38-layer step
that adds the encoder's three Full + 5 Reuse blocks at m = 2) and the
prefill chunk.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch  # noqa: E402

import csa2_inputs as ci  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0 # MI355X dense bf16/fp16 matrix peak, vendor figure
METRIC = "CSA2 decode queries/s & achieved HBM GB/s at 128K and 1M ctx (1 GPU)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "score_scan_traffic.json")
ATTN_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic.json")


# --------------------------------------------------------------------------
def fill_kv_cache(K, codes, scales, seed, n_valid, D, chunk_rows=1 << 16):
    """Quantise generated main-KV rows [b][0..n_valid) into the MXFP4 cache
    with the library's writer (cache build, untimed)."""
    B, cap, _ = codes.shape
    dev = codes.device
    for b in range(B):
        for p0 in range(0, n_valid, chunk_rows):
            p1 = min(n_valid, p0 + chunk_rows)
            rows = torch.arange(b * cap + p0, b * cap + p1, device=dev, dtype=torch.int64)
            x = ci.gaussian_rows(seed, ci.TID_KV, rows, D, dtype=torch.bfloat16, clip=ci.NORM_BOUND)
            K.mxfp4_kv_write(x, rows, codes, scales)


class InputSet:
    """One complete set of decode inputs for a workload, on the GPU."""

    def __init__(self, K, w: ci.Workload, seed: int, dev):
        from compressed_sparse_attention_05_amd.decode import DecodeCache, LayerInputs
        B, N, D, d_I, H_I, H, W = w.B, w.N, w.D, w.d_I, w.H_I, w.H, w.W
        cap = N
        self.seed = seed
        self.codes = torch.empty((B, cap, D // 2), dtype=torch.uint8, device=dev)
        self.scales = torch.empty((B, cap, D // 16), dtype=torch.uint8, device=dev)
        fill_kv_cache(K, self.codes, self.scales, seed, N - 1, D)
        # indexer keys: generated row-major (flat index (b*cap + pos)*d_I + c),
        # stored in the library's tiled layout
        self.k_idx = torch.empty((B, cap, d_I), dtype=torch.bfloat16, device=dev)
        for b in range(B):
            rows = torch.empty((1, cap, d_I), dtype=torch.bfloat16, device=dev)
            ci.fill_gaussian_(rows, seed, ci.TID_K_IDX, first=b * cap * d_I)
            self.k_idx[b] = K.tile_indexer_cache(rows)[0]
            del rows
        self.cache = DecodeCache(self.codes, self.scales, self.k_idx,
                                 torch.full((B,), N, dtype=torch.int32, device=dev),
                                 torch.full((B,), W, dtype=torch.int32, device=dev))
        # the token written by the step: entry N-1 of every sequence
        self.dst_row = torch.arange(B, device=dev, dtype=torch.int64) * cap + (N - 1)
        self.new_kv = ci.gaussian_rows(seed, ci.TID_KV, self.dst_row, D, dtype=torch.bfloat16,
                                       clip=ci.NORM_BOUND)
        self.new_kidx = ci.gaussian_rows(seed, ci.TID_K_IDX, self.dst_row, d_I, dtype=torch.bfloat16)
        # encoder KV sets (one per E layer): N / enc_m complete entries; the
        # step's token (position N-1) completes the last one and writes it
        self.enc_caches, self.enc_writes = [], []
        self.enc_q_pos = torch.full((B,), N - 1, dtype=torch.int64, device=dev)
        for e in range(w.schedule.count("E")):
            seed_e = seed + 7919 * (e + 1)
            cap_e = N // w.enc_m
            codes_e = torch.empty((B, cap_e, D // 2), dtype=torch.uint8, device=dev)
            scales_e = torch.empty((B, cap_e, D // 16), dtype=torch.uint8, device=dev)
            fill_kv_cache(K, codes_e, scales_e, seed_e, cap_e - 1, D)
            k_idx_e = torch.empty((B, cap_e, d_I), dtype=torch.bfloat16, device=dev)
            for b in range(B):
                rows = torch.empty((1, cap_e, d_I), dtype=torch.bfloat16, device=dev)
                ci.fill_gaussian_(rows, seed_e, ci.TID_K_IDX, first=b * cap_e * d_I)
                k_idx_e[b] = K.tile_indexer_cache(rows)[0]
                del rows
            self.enc_caches.append(DecodeCache(codes_e, scales_e, k_idx_e,
                                               torch.full((B,), cap_e, dtype=torch.int32, device=dev),
                                               torch.full((B,), W, dtype=torch.int32, device=dev)))
            dst_e = torch.arange(B, device=dev, dtype=torch.int64) * cap_e + (cap_e - 1)
            self.enc_writes.append((
                ci.gaussian_rows(seed_e, ci.TID_KV, dst_e, D, dtype=torch.bfloat16, clip=ci.NORM_BOUND),
                ci.gaussian_rows(seed_e, ci.TID_K_IDX, dst_e, d_I, dtype=torch.bfloat16), dst_e))
        self.layers = []
        for li, mode in enumerate(w.schedule):
            q = ci.gaussian(seed, ci.layer_tid(ci.TID_Q, li), (B, H, D), torch.bfloat16, dev)
            swa = ci.gaussian(seed, ci.layer_tid(ci.TID_SWA, li), (B, W, D), torch.bfloat16, dev)
            qi = wt = None
            if mode in "FXE":
                qi = ci.gaussian(seed, ci.layer_tid(ci.TID_Q_IDX, li), (B, 1, H_I, d_I), torch.bfloat16, dev)
                wt = ci.uniform(seed, ci.layer_tid(ci.TID_W, li), (B, 1, H_I), dev)
            self.layers.append(LayerInputs(q=q, swa=swa, q_idx=qi, w=wt))


def make_step(K, w: ci.Workload, s: InputSet, pool=None):
    from compressed_sparse_attention_05_amd.decode import DecodeStep
    has_full = "F" in w.schedule
    has_enc = "E" in w.schedule
    return DecodeStep(w.schedule, s.cache, s.layers, k=w.k, P_b=w.P_b,
                      new_kv=s.new_kv if has_full else None,
                      new_kidx=s.new_kidx if has_full else None,
                      dst_row=s.dst_row if has_full else None, pool=pool,
                      enc_caches=s.enc_caches, enc_q_pos=s.enc_q_pos if has_enc else None, enc_m=w.enc_m,
                      enc_writes=s.enc_writes if has_enc else None)


def build_pool_for(K, w: ci.Workload, s: InputSet):
    """Reindex workloads: the pool comes from a preceding Full layer (untimed)."""
    from compressed_sparse_attention_05_amd.decode import DecodeStep, LayerInputs
    dev = s.codes.device
    qi = ci.gaussian(s.seed, ci.layer_tid(ci.TID_Q_IDX, 63), (w.B, 1, w.H_I, w.d_I), torch.bfloat16, dev)
    wt = ci.uniform(s.seed, ci.layer_tid(ci.TID_W, 63), (w.B, 1, w.H_I), dev)
    full = LayerInputs(q=s.layers[0].q, swa=s.layers[0].swa, q_idx=qi, w=wt)
    st = DecodeStep("F", s.cache, [full], k=w.k, P_b=w.P_b, new_kv=s.new_kv, new_kidx=s.new_kidx,
                    dst_row=s.dst_row)
    st.run()
    torch.cuda.synchronize()
    return st.pool.clone()


# --------------------------------------------------------------------------
def algorithmic_bytes_per_query(w: ci.Workload):
    """Bytes the method must move per query (one sequence, one step):
    indexer keys scanned, selected rows gathered (288 B MXFP4 each), window
    rows, queries, outputs, index lists.  Score scratch and re-reads excluded."""
    D, d_I = w.D, w.d_I
    row = D // 2 + D // 16
    per_layer_attn = w.k * row + w.W * D * 2 + w.H * D * 2 + w.H * D * 4 + w.k * 4
    idx_q = w.H_I * d_I * 2 + w.H_I * 4
    total = 0
    written = row + d_I * 2 + D * 2 + d_I * 2     # one written entry (read + write)
    for mode in w.schedule:
        if mode == "F":
            total += w.N * d_I * 2 + idx_q
        elif mode == "E":
            total += (w.N // w.enc_m) * d_I * 2 + idx_q + written
        elif mode == "X":
            total += w.P_b * 8 * d_I * 2 + w.P_b * 4 + idx_q
        total += per_layer_attn
    if "F" in w.schedule:
        total += written
    return total


def scan_bytes_per_launch(w: ci.Workload):
    """Full scan (dominant kernel): indexer-K rows of every visible entry plus
    the indexer queries and head weights, for the B rows of one launch; the
    launch also writes the token's entry (bf16 latent row and indexer key
    read, MXFP4 row and key written)."""
    write = w.D * 2 + w.d_I * 2 + w.D // 2 + w.D // 16 + w.d_I * 2
    return w.B * (w.N * w.d_I * 2 + w.H_I * w.d_I * 2 + w.H_I * 4 + write)


def source_hash(f="score.hip"):
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "compressed_sparse_attention_05_amd", "csrc", f), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def attn_traffic_for(workload_name):
    """Counter-measured bytes per launch of the attention and combine kernels
    (profiles/attn_traffic.json), while attn.hip is the source they were
    taken on; None otherwise."""
    try:
        with open(ATTN_TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash("attn.hip"):
        return None
    out = {k["kernel"]: {"read_bytes": k["read_bytes"], "written_bytes": k["written_bytes"],
                         "algorithmic_read_bytes": k["algorithmic_read_bytes"]}
           for k in rec.get("kernels", []) if k.get("workload") == workload_name}
    return out or None


def traffic_for(workload_name):
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash() or rec.get("workload") != workload_name:
        return None
    return rec.get("hbm_bytes_per_launch")


# --------------------------------------------------------------------------
def run_workload(K, w: ci.Workload, steps: int, warmup: int, dev, n_sets: int = 2):
    """Time `steps` decode steps.  n_sets independent input sets alternate
    (two when a step's working set could sit in the 256 MiB MALL)."""
    sets = [InputSet(K, w, w.seed + 100 * i, dev) for i in range(n_sets)]
    pools = [build_pool_for(K, w, s) if "X" in w.schedule and "F" not in w.schedule else None
             for s in sets]
    runners = [make_step(K, w, s, pool=p) for s, p in zip(sets, pools)]
    torch.cuda.synchronize()
    scan_name = next((f"score{i}" for i, m in enumerate(w.schedule) if m == "F"), None)
    if scan_name is None:
        scan_name = next(f"score{i}" for i, m in enumerate(w.schedule) if m == "X")
    for i in range(warmup):
        runners[i % n_sets].run()
    torch.cuda.synchronize()
    # each step captured once into a HIP graph: a replay enqueues the whole
    # step (write, scan, selection, attention) with one launch
    graphs = [r.capture() for r in runners]
    for i in range(warmup):
        graphs[i % n_sets].replay()
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(steps):
        graphs[i % n_sets].replay()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / steps
    # the same steps launched one kernel group at a time, with HIP events on
    # the launch stream around the scan (the roofline kernel)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e_start.record()
    for i in range(steps):
        runners[i % n_sets].run(events={scan_name: evs[i]})
    e_end.record()
    torch.cuda.synchronize()
    eager_ms = e_start.elapsed_time(e_end) / steps
    scan_ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    return dict(sets=sets, runners=runners, ms_per_step=ms_step, wall_s=wall, scan_ms=scan_ms,
                scan_name=scan_name, eager_ms_per_step=eager_ms)


def run_prefill(K, w: ci.Workload, steps: int, warmup: int, dev):
    """The encoder prefill chunk: T query tokens at positions prior..prior+T-1
    (m tokens per entry), the chunk's T/m new entries written, the Full
    layer's per-token top-k over the visible entries, and attention for every
    layer of the schedule.  One input set (a step moves several GB)."""
    from compressed_sparse_attention_05_amd.prefill import PrefillChunk, PrefillLayer
    seed, N, D, d_I, T, m, W, H = w.seed, w.N, w.D, w.d_I, w.T, w.m, w.W, w.H
    n_prior = w.prior_tokens // m
    codes = torch.empty((1, N, D // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((1, N, D // 16), dtype=torch.uint8, device=dev)
    fill_kv_cache(K, codes, scales, seed, n_prior, D)
    rows = torch.empty((1, N, d_I), dtype=torch.bfloat16, device=dev)
    ci.fill_gaussian_(rows, seed, ci.TID_K_IDX)
    k_idx = K.tile_indexer_cache(rows)[0]
    del rows
    dst = torch.arange(n_prior, N, device=dev, dtype=torch.int64)
    new_kv = ci.gaussian_rows(seed, ci.TID_KV, dst, D, dtype=torch.bfloat16, clip=ci.NORM_BOUND)
    new_kidx = ci.gaussian_rows(seed, ci.TID_K_IDX, dst, d_I, dtype=torch.bfloat16)
    layers = []
    for li, mode in enumerate(w.schedule):
        lay = PrefillLayer(q=ci.gaussian(seed, ci.layer_tid(ci.TID_Q, li), (T, H, D), torch.bfloat16, dev),
                           swa=ci.gaussian(seed, ci.layer_tid(ci.TID_SWA, li), (T + W - 1, D), torch.bfloat16, dev))
        if mode == "F":
            lay.q_idx = ci.gaussian(seed, ci.layer_tid(ci.TID_Q_IDX, li), (T, w.H_I, d_I), torch.bfloat16, dev)
            lay.w = ci.uniform(seed, ci.layer_tid(ci.TID_W, li), (T, w.H_I), dev)
        layers.append(lay)
    chunk = PrefillChunk(w.schedule, codes[0], scales[0], k_idx, N, w.prior_tokens, m, w.k, W, layers,
                         new_kv=new_kv, new_kidx=new_kidx, dst_row=dst)
    for _ in range(warmup):
        chunk.run()
    torch.cuda.synchronize()
    names = ["topk"] + [f"attn{i}" for i in range(len(w.schedule))]
    evs = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in names}
           for _ in range(steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        chunk.run(events=evs[i])
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    topk_ms = sum(e["topk"][0].elapsed_time(e["topk"][1]) for e in evs) / steps
    attn_ms = sum(e[n][0].elapsed_time(e[n][1]) for e in evs for n in names[1:]) / steps
    pairs = sum(min(N, (w.prior_tokens + t + 1) // m) for t in range(T))
    score_flop = pairs * w.H_I * d_I * 2
    attn_flop = len(w.schedule) * T * w.H * (w.k + W) * D * 2 * 2
    return {"workload": w.name, "tokens": T, "context": N, "schedule": w.schedule,
            "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 3),
            "topk_ms": round(topk_ms, 3),
            "topk_scoring_TFLOPs": round(score_flop / (topk_ms * 1e-3) / 1e12, 1),
            "topk_mfma_frac": round(score_flop / (topk_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "attn_ms": round(attn_ms, 3),
            "attn_TFLOPs": round(attn_flop / (attn_ms * 1e-3) / 1e12, 1),
            "attn_mfma_frac": round(attn_flop / (attn_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}


def run_replay(K, w: ci.Workload, steps: int, warmup: int, dev):
    """SWA bounded replay: the decoder's layers over the newest T tokens of
    one sequence (positions prior_tokens .. prior_tokens + T - 1), every
    token a decoder query with its own pool, windows cut at the replay start.
    The replayed tokens' global KV is already cached."""
    from compressed_sparse_attention_05_amd.replay import DecoderReplay, ReplayLayer
    seed, N, D, d_I, T, W, H = w.seed, w.N, w.D, w.d_I, w.T, w.W, w.H
    codes = torch.empty((1, N, D // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((1, N, D // 16), dtype=torch.uint8, device=dev)
    fill_kv_cache(K, codes, scales, seed, N, D)
    rows = torch.empty((1, N, d_I), dtype=torch.bfloat16, device=dev)
    ci.fill_gaussian_(rows, seed, ci.TID_K_IDX)
    k_idx = K.tile_indexer_cache(rows)[0]
    del rows
    layers = []
    for li, mode in enumerate(w.schedule):
        lay = ReplayLayer(q=ci.gaussian(seed, ci.layer_tid(ci.TID_Q, li), (T, H, D), torch.bfloat16, dev),
                          swa=ci.gaussian(seed, ci.layer_tid(ci.TID_SWA, li), (T + W - 1, D), torch.bfloat16, dev))
        if mode in "FX":
            lay.q_idx = ci.gaussian(seed, ci.layer_tid(ci.TID_Q_IDX, li), (T, w.H_I, d_I), torch.bfloat16, dev)
            lay.w = ci.uniform(seed, ci.layer_tid(ci.TID_W, li), (T, w.H_I), dev)
        layers.append(lay)
    rp = DecoderReplay(w.schedule, codes[0], scales[0], k_idx, N, w.prior_tokens, w.k, W, layers, P_b=w.P_b)
    for _ in range(warmup):
        rp.run()
    torch.cuda.synchronize()
    names = [f"score{i}" for i, mode in enumerate(w.schedule) if mode in "FX"]
    names += [f"attn{i}" for i in range(len(w.schedule))]
    evs = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in names}
           for _ in range(steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        rp.run(events=evs[i])
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    full_ms = sum(e["score0"][0].elapsed_time(e["score0"][1]) for e in evs) / steps
    attn_ms = sum(e[n][0].elapsed_time(e[n][1]) for e in evs for n in names if n.startswith("attn")) / steps
    # the Full layer's keys once (every token shares them), Reindex pools and
    # attention gathers per token
    scan_b = N * d_I * 2
    return {"workload": w.name, "tokens": T, "context": N, "schedule": w.schedule,
            "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 3),
            "full_scan_ms": round(full_ms, 3),
            "full_scan_GBps_per_token": round(T * scan_b / (full_ms * 1e-3) / 1e9, 1),
            "attn_ms": round(attn_ms, 3)}


def run_project(K, dev, reps: int = 50):
    """The MXFP4 write with the indexer key projected from the latent row
    (csa2_kv_write_project, D = 512 -> d_I = 128 bfloat16), against the plain
    write that copies a given key row, for one decode token of 64 sequences
    and for the 4,096 entries of an m = 2 prefill chunk of 8,192 tokens."""
    D, d_I = 512, 128
    w_ik = (ci.gaussian(7, ci.TID_W_IK, (D, d_I)) * (1.0 / math.sqrt(D))).to(dev)
    res = {"workload": "kv-write-project", "latent": D, "indexer": f"{d_I} bf16"}
    for label, n, cap in (("decode_b64", 64, 65536), ("prefill_chunk_4096", 4096, 65536)):
        x = ci.gaussian(8, ci.TID_KV, (n, D), dtype=torch.bfloat16, clip=ci.NORM_BOUND).to(dev)
        kr = ci.gaussian(8, ci.TID_K_IDX, (n, d_I), dtype=torch.bfloat16).to(dev)
        dst = torch.arange(n, dtype=torch.int64, device=dev) * (cap // n)
        codes = torch.zeros((cap, D // 2), dtype=torch.uint8, device=dev)
        scales = torch.zeros((cap, D // 16), dtype=torch.uint8, device=dev)
        kc = torch.zeros((cap, d_I), dtype=torch.bfloat16, device=dev)
        timings = {}
        for name, fn in (("project", lambda: K.csa2_kv_write_project(x, dst, codes, scales, w_ik, kc)),
                         ("copy", lambda: K.mxfp4_kv_write(x, dst, codes, scales, kr, kc))):
            for _ in range(5):
                fn()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            for _ in range(reps):
                fn()
            b.record()
            torch.cuda.synchronize()
            timings[name] = a.elapsed_time(b) / reps * 1e3
        res[label] = {"rows": n, "project_us": round(timings["project"], 2),
                      "copy_us": round(timings["copy"], 2),
                      "project_TFLOPs_fp32": round(2.0 * n * D * d_I / (timings["project"] * 1e-6) / 1e12, 2)}
    return res


def run_mhc(K, dev, reps: int = 20, T: int = 8192, d: int = 4096):
    """Single-pass mHC step (n = 4 streams of d = 4,096 channels, bfloat16)
    for the 8,192 tokens of a prefill chunk.  Algorithmic bytes per launch:
    (2n + 2) * d * 2 per token (read X and f, write X_next and u) plus the
    coefficients in and out and the projection weights once."""
    n, K_out = 4, 24
    sets = []
    for i in range(2):
        seed = 900 + i
        X = ci.gaussian(seed, ci.TID_MHC_X, (T, n, d), dtype=torch.bfloat16, device=dev)
        f = ci.gaussian(seed, ci.TID_MHC_F, (T, d), dtype=torch.bfloat16, device=dev)
        coef = ci.uniform(seed, ci.TID_MHC_COEF, (T, n + n * n + n), device=dev)
        A = (0.1 + 0.9 * coef[:, :n]).contiguous()
        B = (0.5 * coef[:, n:n + n * n]).reshape(T, n, n).contiguous()
        C = (0.2 + 1.6 * coef[:, n + n * n:]).contiguous()
        phiT = (ci.gaussian(seed, ci.TID_MHC_PHI, (K_out, n * d), device=dev) / math.sqrt(n * d)).to(torch.bfloat16)
        bias = 0.5 * ci.gaussian(seed + 1, ci.TID_MHC_PHI, (K_out,), device=dev)
        out = (torch.empty_like(X), torch.empty_like(f), torch.empty_like(A), torch.empty_like(B),
               torch.empty_like(C))
        sets.append((X, f, A, B, C, phiT, bias, out))

    def call(s):
        X, f, A, B, C, phiT, bias, out = s
        K.csa2_mhc_step(X, f, A, B, C, phiT, bias, (1.0, 1.0, 1.0), iters=20, out=out)

    for i in range(4):
        call(sets[i % 2])
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        evs[i][0].record()
        call(sets[i % 2])
        evs[i][1].record()
    torch.cuda.synchronize()
    us = sum(a.elapsed_time(b) for a, b in evs) / reps * 1e3
    alg = T * ((2 * n + 2) * d * 2 + 2 * (n + n * n + n) * 4) + K_out * n * d * 2
    return {"workload": f"mhc-step-t{T}-n{n}-d{d}", "tokens": T, "streams": n, "channels": d,
            "us_per_step": round(us, 2), "tokens_per_s": round(T / (us * 1e-6), 1),
            "algorithmic_bytes": alg, "GBps": round(alg / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w: ci.Workload, s: InputSet, n_queries: int):
    """The oracle, as it stands, on n_queries sequences of the workload's
    first Full layer (write + scan + block max + pool + top-k + attention),
    on every host core available to this process.

    The work is cut into units that the oracle computes independently: the
    scan of a sequence in fixed position ranges (each score is its own fma
    chain, so the ranges reproduce the whole row bit for bit), the block max,
    pool and top-k of a sequence, and its attention in fixed head ranges
    (each head is computed on its own).  Units run on a thread pool (the
    oracle's C calls release the GIL).  The timed passes repeat until they
    hold about 10 s of CPU work (wall time x threads; at least 3 passes).
    A single-thread figure (one sequence, every unit on one thread) is taken
    as well.  Returns a dict."""
    from concurrent.futures import ThreadPoolExecutor
    import numpy as np
    import oracle
    import compressed_sparse_attention_05_amd as K

    B, N, D, H = w.B, w.N, w.D, w.H
    lay = s.layers[0]
    cores = len(os.sched_getaffinity(0))
    threads = max(1, cores)
    oracle.lib()
    seqs = []
    for b in range(n_queries):
        kc_f = oracle.as_f32(K.untile_indexer_cache(s.k_idx[b:b + 1])[0].cpu())   # generator output
        kc_f[N - 1] = oracle.as_f32(s.new_kidx[b:b + 1].cpu())[0]
        seqs.append(dict(kc=kc_f, qi=lay.q_idx[b, 0].cpu(), wt=lay.w[b, 0].cpu(), q=oracle.as_f32(lay.q[b]),
                         swa=lay.swa[b].cpu(), new_kv=s.new_kv[b:b + 1].cpu(),
                         sc=np.empty(N, np.float32), out=np.empty((H, D), np.float32)))
    # scan ranges: enough units for every thread, in whole 8-position blocks
    per_seq = max(1, -(-2 * threads // n_queries))
    step_rows = -(-N // per_seq)
    step_rows = -(-step_rows // 8) * 8
    ranges = [(r0, min(N, r0 + step_rows)) for r0 in range(0, N, step_rows)]
    heads_per = max(1, H // max(1, -(-2 * threads // n_queries)))
    hranges = [(h0, min(H, h0 + heads_per)) for h0 in range(0, H, heads_per)]

    def scan(unit):
        d, r0, r1 = unit
        d["sc"][r0:r1] = oracle.full_scores(d["qi"], d["wt"], d["kc"][r0:r1], r1 - r0, r1 - r0)

    def select(d):
        oracle.mxfp4_encode(d["new_kv"])
        bm = oracle.block_max(d["sc"], N, (N + 7) // 8)
        oracle.candidate_pool(bm, w.P_b)
        d["idx"] = oracle.topk(d["sc"], w.k)

    def attend(unit):
        d, h0, h1 = unit
        d["out"][h0:h1] = oracle.attn_decode(d["q"][h0:h1], d["codes"], d["scales"], d["idx"], d["swa"], w.W,
                                             1.0 / math.sqrt(D))

    scan_units = [(d, r0, r1) for d in seqs for r0, r1 in ranges]
    attn_units = [(d, h0, h1) for d in seqs for h0, h1 in hranges]

    def prepare_rows():
        # the cache rows the attention reads, encoded by the oracle from the
        # generator (the cache existed before this step; untimed)
        for b, d in enumerate(seqs):
            idx = d["idx"]
            sel = torch.from_numpy(idx[idx >= 0].astype(np.int64))
            raw = ci.gaussian_rows(s.seed, ci.TID_KV, b * N + sel, D, dtype=torch.bfloat16, clip=ci.NORM_BOUND)
            codes = np.zeros((N, D // 2), np.uint8)
            scales = np.zeros((N, D // 16), np.uint8)
            c, sc_ = oracle.mxfp4_encode(raw)
            codes[sel.numpy()], scales[sel.numpy()] = c, sc_
            if (sel == N - 1).any():
                c1, s1 = oracle.mxfp4_encode(d["new_kv"])
                codes[N - 1], scales[N - 1] = c1[0], s1[0]
            d["codes"], d["scales"] = codes, scales

    def one_pass(ex):
        t0 = time.perf_counter()
        list(ex.map(scan, scan_units))
        list(ex.map(select, seqs))
        t1 = time.perf_counter()
        if "codes" not in seqs[0]:
            prepare_rows()
        t2 = time.perf_counter()
        list(ex.map(attend, attn_units))
        return (t1 - t0) + (time.perf_counter() - t2)

    with ThreadPoolExecutor(threads) as ex:
        secs = one_pass(ex)
        passes = 1
        while passes < 3 or (secs * threads < 10.0 and passes < 64):
            secs += one_pass(ex)
            passes += 1
    # one thread, one sequence
    d0 = seqs[0]
    t0 = time.perf_counter()
    scan((d0, 0, N))
    select(d0)
    attend((d0, 0, H))
    t_one = time.perf_counter() - t0
    return {"value": passes * n_queries / secs, "secs": secs, "threads": threads, "passes": passes,
            "units": (len(scan_units), len(attn_units)), "one_thread_value": 1.0 / t_one}


def calibrate_copy(mib: int, reps: int, dev):
    """A plain device-to-device copy of known size (torch's copy kernel),
    for scaling the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "reps": reps}), flush=True)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=ci.DECODE_128K.name, choices=sorted(ci.WORKLOADS))
    ap.add_argument("--cpu-queries", type=int, default=8, help="oracle sample size (0 = skip)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only time the prefill chunk workload (profiling)")
    ap.add_argument("--replay-only", action="store_true",
                    help="only time the decoder replay workload (profiling)")
    ap.add_argument("--project-only", action="store_true",
                    help="only time the write with the projected indexer key (profiling)")
    ap.add_argument("--mhc-only", action="store_true",
                    help="only time the single-pass mHC step (profiling)")
    ap.add_argument("--decode-only", default=None, choices=sorted(ci.WORKLOADS), metavar="WORKLOAD",
                    help="only time this decode workload, any schedule (profiling)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB (counter calibration) and exit")
    ap.add_argument("--no-secondary", dest="secondary", action="store_false",
                    help="skip the 1M-context decode workloads")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(decode shards by sequence across GPUs with no exchange; see the design notes)",
              file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    import compressed_sparse_attention_05_amd as K
    K.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, 4, dev)
        return 0
    if args.prefill_only:
        print(json.dumps(run_prefill(K, ci.PREFILL_CHUNK, args.steps, args.warmup, dev)), flush=True)
        return 0
    if args.replay_only:
        print(json.dumps(run_replay(K, ci.DECODER_REPLAY, args.steps, args.warmup, dev)), flush=True)
        return 0
    if args.project_only:
        print(json.dumps(run_project(K, dev)), flush=True)
        return 0
    if args.mhc_only:
        print(json.dumps(run_mhc(K, dev)), flush=True)
        return 0
    if args.decode_only:
        w = ci.WORKLOADS[args.decode_only]
        big = w.B * w.N >= (1 << 24)
        r = run_workload(K, w, args.steps, args.warmup, dev, n_sets=1 if big else 2)
        print(json.dumps({"workload": w.name, "schedule": w.schedule, "batch": w.B, "context": w.N,
                          "ms_per_step": round(r["ms_per_step"], 4),
                          "value": round(w.B / (r["ms_per_step"] * 1e-3), 1), "unit": "queries/s",
                          "scan": {"kernel": r["scan_name"], "us": round(r["scan_ms"] * 1e3, 2)}}), flush=True)
        return 0
    w = ci.WORKLOADS[args.workload]
    if "F" not in w.schedule:
        print("bench.py: the headline workload must contain a Full layer", file=sys.stderr)
        return 2

    print(f"# setting up {w.name}", file=sys.stderr, flush=True)
    r = run_workload(K, w, args.steps, args.warmup, dev)
    ms = r["ms_per_step"]
    qps = w.B / (ms * 1e-3)
    alg_q = algorithmic_bytes_per_query(w)
    scan_bytes = scan_bytes_per_launch(w)
    scan_gbs = scan_bytes / (r["scan_ms"] * 1e-3) / 1e9
    traffic = traffic_for(w.name)

    result = {
        "metric": METRIC,
        "value": round(qps, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "eager_ms_per_step": round(r["eager_ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 scores and softmax; f16 MFMA with f32 accumulation for attention",
        "data": "synthetic (seeded counter-based Gaussian/uniform; MXFP4 KV, bf16 indexer K, Q, SWA)",
        "config": {"workload": w.name, "batch": w.B, "context": w.N, "schedule": w.schedule,
                   "top_k": w.k, "window": w.W, "heads": w.H, "latent": w.D,
                   "indexer": f"{w.H_I}x{w.d_I} bf16", "pool_blocks": w.P_b},
        "algorithmic_GBps": round(alg_q * w.B / (ms * 1e-3) / 1e9, 1),
        "roofline": {
            "kernel": "score_kernel (Full-mode indexer scan with fused block max and the token's cache write)",
            "bound": "hbm",
            "achieved": round(scan_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(scan_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "scan_us": round(r["scan_ms"] * 1e3, 2),
            "bytes_per_launch": scan_bytes,
        },
        # HBM bytes per launch of the attention kernels from FETCH_SIZE /
        # WRITE_SIZE (calibrated), null once their source has changed
        "attention_traffic": attn_traffic_for(w.name),
    }
    if args.cpu_queries > 0:
        print("# timing the CPU oracle", file=sys.stderr, flush=True)
        nq = min(args.cpu_queries, w.B)
        cb = cpu_baseline(w, r["sets"][0], nq)
        result["cpu_baseline"] = {
            "value": round(cb["value"], 4), "unit": "queries/s", "cores": cb["threads"], "kind": "oracle",
            "cpu_model": cpu_model(),
            "one_thread_value": round(cb["one_thread_value"], 4),
            "sample": f"{nq} of {w.B} sequences of {w.name} (full work each: write, "
                      f"scan of {w.N} entries, block max, pool, top-{w.k}, attention), "
                      f"{cb['passes']} passes, {cb['secs']:.2f} s wall on {cb['threads']} threads "
                      f"(all cores available to the process); units: {cb['units'][0]} scan ranges and "
                      f"{cb['units'][1]} attention head ranges; one_thread_value: one sequence on one thread",
        }
    if args.secondary:
        sec = []
        # (workload, input sets, timed steps): the 20- and 38-layer steps move
        # ~19 and ~46 GB, far beyond the MALL, so one input set suffices there
        for name, n_sets, steps2 in ((ci.DECODE_1M_BLOCK2.name, 2, max(20, args.steps // 4)),
                                     (ci.DECODE_1M_20L.name, 1, 10),
                                     (ci.DECODE_1M_38L.name, 1, 5)):
            w2 = ci.WORKLOADS[name]
            del r
            torch.cuda.empty_cache()
            print(f"# setting up {w2.name}", file=sys.stderr, flush=True)
            t_setup = time.perf_counter()
            r = run_workload(K, w2, steps2, 3, dev, n_sets=n_sets)
            print(f"# {w2.name}: {time.perf_counter() - t_setup:.1f} s incl. setup", file=sys.stderr, flush=True)
            ms2 = r["ms_per_step"]
            alg2 = algorithmic_bytes_per_query(w2) * w2.B
            scan_b = (scan_bytes_per_launch(w2) if "F" in w2.schedule
                      else w2.B * (w2.P_b * 8 * w2.d_I * 2 + w2.P_b * 4 + w2.H_I * w2.d_I * 2 + w2.H_I * 4))
            sec.append({"workload": w2.name, "batch": w2.B, "context": w2.N, "schedule": w2.schedule,
                        "value": round(w2.B / (ms2 * 1e-3), 1), "unit": "queries/s",
                        "ms_per_step": round(ms2, 4),
                        "algorithmic_GBps": round(alg2 / (ms2 * 1e-3) / 1e9, 1),
                        "hbm_frac": round(alg2 / (ms2 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "scan": {"kernel": r["scan_name"], "us": round(r["scan_ms"] * 1e3, 2),
                                 "GBps": round(scan_b / (r["scan_ms"] * 1e-3) / 1e9, 1)}})
        del r
        torch.cuda.empty_cache()
        print(f"# setting up {ci.PREFILL_CHUNK.name}", file=sys.stderr, flush=True)
        sec.append(run_prefill(K, ci.PREFILL_CHUNK, 3, 1, dev))
        torch.cuda.empty_cache()
        print(f"# setting up {ci.DECODER_REPLAY.name}", file=sys.stderr, flush=True)
        sec.append(run_replay(K, ci.DECODER_REPLAY, 3, 1, dev))
        sec.append(run_project(K, dev))
        torch.cuda.empty_cache()
        sec.append(run_mhc(K, dev))
        result["secondary"] = sec
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
