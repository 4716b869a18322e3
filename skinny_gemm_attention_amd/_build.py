"""Builds libattnres.so (the gfx950 kernels and the C ABI) in the package folder.

hipcc cross-compiles for gfx950 without a GPU. Packed FP32 instructions are
disabled (``-packed-fp32-ops``); the kernels never rely on them. Implicit FP
contraction is off: every fused multiply-add is written as fmaf.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libattnres.so")
SOURCES = ["api.hip", "wsgemm.hip", "attnres.hip", "fused.hip", "stream_read.hip"]
HEADERS = ["common.hpp", "token.hpp", "gemm.hpp", "launch.hpp"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no implicit multiply-add contraction: every fused multiply-add is an
    # explicit fmaf, so all kernels round the shared AttnRes arithmetic alike
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stderr or "").splitlines() if l.strip() and noise not in l]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(verbose_resources: bool = False) -> str:
    """Compile every source and link libattnres.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if verbose_resources else []
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def stale() -> bool:
    """True when the library is missing or older than a source or header."""
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    inc = os.path.join(os.path.dirname(PKG), "include", "attnres.h")
    files = [os.path.join(CSRC, f) for f in SOURCES + HEADERS] + [inc]
    return any(os.path.getmtime(f) > t for f in files if os.path.exists(f))


if __name__ == "__main__":
    print(build(verbose_resources="-v" in sys.argv))
