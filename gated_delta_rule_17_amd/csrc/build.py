"""Build libgdr.so (all HIP kernels + the C-ABI host code) for gfx950.

    python gated_delta_rule_17_amd/csrc/build.py [-j N]

Objects go to ``_build/`` at the repository root; the shared library is
written next to the Python binding (``gated_delta_rule_17_amd/libgdr.so``).
Every translation unit is compiled on each call.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgdr.so")

SOURCES = ["chan_gm0.hip", "chan_gm1.hip", "chan_gm2.hip", "chan_gm3.hip", "pipe_gm0.hip", "pipe_gm3.hip",
           "chan_split_gm0.hip", "chan_split_gm1.hip", "chan_split_gm2.hip", "chan_split_gm3.hip",
           "chunk_bf16_gm1.hip", "chunk_bf16_gm2.hip",
           "chunk_f32.hip", "plain.hip", "recur.hip", "bwd.hip", "step.hip", "gdr_host.cpp"]

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ARCH = os.environ.get("GDR_OFFLOAD_ARCH", "gfx950")
# Device code is built without packed-fp32 instructions.
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-result", "-Wno-pass-failed",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC, *lang, *CFLAGS, "-c", os.path.join(HERE, src), "-o", obj]
    t = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in line and line.strip())
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{msgs}")
    if msgs:
        print(msgs, file=sys.stderr)
    print(f"  [{time.time() - t:5.1f}s] {src}", flush=True)
    return obj


def build(jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=None)
    args = ap.parse_args()
    t0 = time.time()
    path = build(args.j)
    print(f"built {path} in {time.time() - t0:.1f}s")
