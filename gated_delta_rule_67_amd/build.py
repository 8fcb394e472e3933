"""Build libkda.so in-tree with hipcc for gfx950.

    python -m gated_delta_rule_67_amd.build        # or build() from Python

Each translation unit is compiled in parallel (``-c``), then linked into
``gated_delta_rule_67_amd/libkda.so``.  Packed-fp32 VALU instructions are
disabled for device code (``-packed-fp32-ops``); hipcc's host pass warns that
it does not know that feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libkda.so")
# the benchmark's peak probe, a library of its own (not part of libkda)
PEAK_SRC = "kda_peak.hip"
PEAK_OUT = os.path.join(PKG, "libkda_peak.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = os.environ.get("KDA_OFFLOAD_ARCH", "gfx950")

SOURCES = ["kda_api.cpp", "kda_recurrent.hip", "kda_twopass.hip", "kda_backward.hip", "kda_conv.hip", "kda_norm.hip", "kda_static.hip"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: libkda needs ROCm (hipcc) to build")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc(), *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(out)} failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + 1)) as ex:
        objs = list(ex.map(_compile, SOURCES + [PEAK_SRC]))
    _link(objs[:-1], OUT)
    _link(objs[-1:], PEAK_OUT)
    if verbose:
        print(f"built {OUT} and {PEAK_OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
