"""Compile the HIP sources of the library into ``libpark.so`` (gfx950 only).

Usage: python -m block_sparse_attention_qrkc_amd.build [--jobs N]
Objects go to ``_build/`` at the repository root; the shared library is written next to this file.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libpark.so")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["metric.hip", "kmeans.hip", "pama.hip", "select.hip", "attn.hip", "merge.hip", "permute.hip",
           "park_api.hip"]

CFLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-Wall", "-Wno-unused-result",
    "-munsafe-fp-atomics",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Per-file flags. kmeans.hip, pama.hip and metric.hip: MFMA results in ordinary VGPRs (the
# assignment's argmax, the map's exponentials and the metric's fp64 flushes read every accumulator
# with VALU instructions, which cannot take AGPR operands, so AGPR results would cost a copy each).
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
FILE_FLAGS = {"kmeans.hip": _VGPR_FORM, "pama.hip": _VGPR_FORM, "metric.hip": _VGPR_FORM}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if msgs:
        print(f"[{src}]\n" + "\n".join(msgs), file=sys.stderr)
    return obj


def build(jobs: int | None = None, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    r = subprocess.run([HIPCC, "-shared", "--offload-arch=gfx950", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    build(ap.parse_args().jobs)
