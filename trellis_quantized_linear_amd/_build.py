"""Build the HIP library libexl3.so in-tree with hipcc for gfx950."""

from __future__ import annotations

import json
import os
import re
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
# the compiler's per-kernel resource report (registers, scratch, spills, LDS,
# occupancy), parsed into RESOURCES
REMARKS = ["-Rpass-analysis=kernel-resource-usage"]
RESOURCES = os.path.join(PKG, "kernel_resources.json")

# (source, extra flags): the linear kernels compile once per bit width, in
# parallel with the rest
SOURCES = [("exl3_kernels.hip", []), ("exl3_api.cpp", [])] + \
          [("exl3_linear_bits.hip", [f"-DEXL3_BITS={b}", f"-cuid=exl3_linear_bits_{b}"]) for b in range(2, 9)]


def _compile(job, build_dir: str) -> str:
    src, extra = job
    tag = "".join(ch for ch in extra[0] if ch.isalnum()).lower() if extra else ""
    obj = os.path.join(build_dir, os.path.basename(src) + (("." + tag) if tag else "") + ".o")
    hip = src.endswith(".hip")
    cmd = [HIPCC, *COMMON, *(DEVICE + REMARKS if hip else []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj, (_parse_remarks(r.stderr) if hip else {})


_FIELDS = {"TotalSGPRs": "sgprs", "VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch",
           "Occupancy [waves/SIMD]": "occupancy", "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill",
           "LDS Size [bytes/block]": "lds"}


def _parse_remarks(text: str) -> dict:
    """Kernel resource records from -Rpass-analysis=kernel-resource-usage
    remarks, keyed by the demangled kernel name without its namespace and
    argument list (e.g. "linear_spread_kernel<4>")."""
    recs, mangled, cur = {}, [], None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = {}
            mangled.append((m.group(1), cur))
            continue
        m = re.search(r"remark:\s+([^:]+(?: \[[^\]]+\])?): (\S+) \[-Rpass-analysis", line)
        if m and cur is not None and m.group(1).strip() in _FIELDS:
            v = m.group(2)
            cur[_FIELDS[m.group(1).strip()]] = int(v) if v.isdigit() else v
    if not mangled:
        return recs
    out = subprocess.run(["c++filt"], input="\n".join(n for n, _ in mangled), capture_output=True, text=True)
    for (raw, rec), name in zip(mangled, out.stdout.splitlines()):
        short = re.sub(r"^void ", "", name)
        short = re.sub(r"^exl3::\(anonymous namespace\)::", "", short)
        short = re.sub(r"\(.*\)$", "", short)
        rec["symbol"] = raw
        recs[short] = rec
    return recs


def build(verbose: bool = False) -> str:
    build_dir = os.path.join(ROOT, "_build")
    os.makedirs(build_dir, exist_ok=True)
    workers = max(1, min(len(SOURCES), len(os.sched_getaffinity(0)), 16))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        done = list(ex.map(lambda s: _compile(s, build_dir), SOURCES))
    objs = [o for o, _ in done]
    resources = {}
    for _, recs in done:
        resources.update(recs)
    with open(RESOURCES + ".tmp", "w") as f:
        json.dump(resources, f, indent=1, sort_keys=True)
    os.replace(RESOURCES + ".tmp", RESOURCES)
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
