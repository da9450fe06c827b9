"""Build libcsa2.so (the HIP library behind include/csa2.h) for gfx950.

Every translation unit is compiled with hipcc for gfx950 only, with
floating-point contraction off (the indexer score is an exact fma chain) and
packed fp32 arithmetic disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libcsa2.so")
SOURCES = ["csa2_api.hip", "kv_write.hip", "score.hip", "topk.hip", "attn.hip", "prefill_topk.hip",
           "decode_select.hip", "mhc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-I" + os.path.join(HERE, "..", "include")]


def build(verbose: bool = False) -> str:
    """Compile every source and link libcsa2.so (always recompiles)."""
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = "\n".join(l for l in out.decode(errors="replace").splitlines()
                         if "not a recognized feature" not in l)
        if p.returncode != 0:
            failed.append((src, text))
        elif verbose and text.strip():
            print(text)
    if failed:
        for src, text in failed:
            print(f"--- {src} ---\n{text}", file=sys.stderr)
        raise RuntimeError("libcsa2 build failed: " + ", ".join(s for s, _ in failed))
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
