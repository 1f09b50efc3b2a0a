"""Build libgdr.so (all HIP kernels + the C-ABI host code) for gfx950.

    python gated_delta_rule_17_amd/csrc/build.py [-j N] [--sanitize]

Objects go to ``_build/`` at the repository root; the shared library is
written next to the Python binding (``gated_delta_rule_17_amd/libgdr.so``).
Every translation unit is compiled on each call.

``--sanitize`` builds a copy whose host code (the C ABI: validation,
planning, dispatch) runs under AddressSanitizer and UndefinedBehaviorSanitizer
into ``_build/sanitize/libgdr.so``; device code is built as usual.  It is
for the CPU tests of the ABI: load it with the sanitizer runtime preloaded,

    LD_PRELOAD=$(hipcc --print-file-name=libclang_rt.asan-x86_64.so) \
    ASAN_OPTIONS=detect_leaks=0 GDR_LIBRARY=_build/sanitize/libgdr.so \
    python -m pytest tests/test_abi.py -m "not gpu"
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


# host-side sanitizers (each -fsanitize= applies to the host pass only)
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC, *lang, *CFLAGS, *extra, "-c", os.path.join(HERE, src), "-o", obj]
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


def build(jobs: int | None = None, sanitize: bool = False) -> str:
    build_dir = os.path.join(BUILD, "sanitize") if sanitize else BUILD
    lib = os.path.join(build_dir, "libgdr.so") if sanitize else LIB
    os.makedirs(build_dir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    extra = SAN_FLAGS if sanitize else ()
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, extra), SOURCES))
    tmp = lib + ".tmp"
    link_extra = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-shared-libsan"] if sanitize else []
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=None)
    ap.add_argument("--sanitize", action="store_true",
                    help="host code under ASan/UBSan, into _build/sanitize/libgdr.so")
    args = ap.parse_args()
    t0 = time.time()
    path = build(args.j, sanitize=args.sanitize)
    print(f"built {path} in {time.time() - t0:.1f}s")
