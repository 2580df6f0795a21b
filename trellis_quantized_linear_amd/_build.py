"""Build the HIP library libexl3.so in-tree with hipcc for gfx950."""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libexl3.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -ffp-contract=off: identical source gives identical arithmetic in every
# kernel instantiation (no fused multiply-adds chosen per context).
# The packed-fp32 feature is switched off for device code.
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-ffp-contract=off",
          "-fno-gpu-flush-denormals-to-zero", "-I", INCLUDE, "-I", CSRC]
DEVICE = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

# (source, extra flags): the linear kernels compile once per bit width, in
# parallel with the rest
SOURCES = [("exl3_kernels.hip", []), ("exl3_api.cpp", [])] + \
          [("exl3_linear_bits.hip", [f"-DEXL3_BITS={b}", f"-cuid=exl3_linear_bits_{b}"]) for b in range(2, 9)]


def _compile(job, build_dir: str) -> str:
    src, extra = job
    tag = "".join(ch for ch in extra[0] if ch.isalnum()).lower() if extra else ""
    obj = os.path.join(build_dir, os.path.basename(src) + (("." + tag) if tag else "") + ".o")
    cmd = [HIPCC, *COMMON, *(DEVICE if src.endswith(".hip") else []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(verbose: bool = False) -> str:
    build_dir = os.path.join(ROOT, "_build")
    os.makedirs(build_dir, exist_ok=True)
    workers = max(1, min(len(SOURCES), len(os.sched_getaffinity(0)), 16))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc link failed")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
