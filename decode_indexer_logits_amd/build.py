"""Builds the HIP library ``libhisparse.so`` in-tree for gfx950, and the
bandwidth-probe library ``libhsprobe.so`` that only the benchmark loads.

Run ``python -m decode_indexer_logits_amd.build``.  Every source is compiled
with hipcc for gfx950 only (packed-fp32 instruction selection disabled), in
parallel, into ``_build/``; the shared object is written next to this file.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
OUT = PKG / "libhisparse.so"
PROBE_OUT = PKG / "libhsprobe.so"
BUILD = ROOT / "_build"
ARCH = "gfx950"

SOURCES = ["indexer.hip", "topk.hip", "resolve.hip", "mla.hip", "cache_ops.hip", "shard_topk.hip", "hs_api.cpp"]
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", f"-I{ROOT / 'include'}"]
# Matrix-core accumulators in ordinary VGPRs, except for the attention kernel,
# whose 128 output accumulators per lane belong in the accumulation registers
# (the VGPRs then hold the row gathers and the operands of many LDS reads).
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
NO_VGPR_FORM = {"mla.hip"}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, verbose: bool) -> Path:
    obj = BUILD / (Path(src).stem + ".o")
    extra = [] if src in NO_VGPR_FORM else VGPR_FORM
    cmd = [hipcc(), *FLAGS, *extra, "-c", str(CSRC / src), "-o", str(obj)]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> Path:
    BUILD.mkdir(exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = OUT.with_suffix(".so.tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, OUT)
    build_probe()
    return OUT


def build_probe() -> Path:
    """Compiles csrc/probe.hip (benchmark bandwidth probes) into libhsprobe.so."""
    tmp = PROBE_OUT.with_suffix(".so.tmp")
    cmd = [hipcc(), *FLAGS, *VGPR_FORM, "-shared", str(CSRC / "probe.hip"), "-o", str(tmp)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on probe.hip:\n{r.stdout}{r.stderr}")
    os.replace(tmp, PROBE_OUT)
    return PROBE_OUT


if __name__ == "__main__":
    print(build(verbose=True))
