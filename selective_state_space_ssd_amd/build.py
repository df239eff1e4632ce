"""Build libssd_mi355x.so in-tree with hipcc for gfx950.

Usage: python -m selective_state_space_ssd_amd.build  (or __graft_entry__.build()).
Each source compiles to an object in parallel; hipcc then links the shared
library next to this file, where the Python binding looks for it.  The compiler's
per-kernel resource report (VGPRs, spills, scratch) is written to
_build/kernel_resources.txt, and the build fails if any kernel needs scratch memory
(a spilled register would go through the same in-order memory counter that the
kernels' waits depend on).
"""
from __future__ import annotations

import concurrent.futures
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_NAME = "libssd_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = ["ssd_api.hip", "ssd_verify.hip", "ssd_chunk_scan.hip", "ssd_chunk_fused.hip",
           "ssd_selective_scan.hip", "ssd_chunk_bwd.hip",
           "ssd_chunk_bwd_bf16.hip", "ssd_seqpar.hip", "ssd_slice_state.hip"]
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from emitting packed fp32 ALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _resources(stderr: str) -> list[dict]:
    """Per-kernel entries of -Rpass-analysis=kernel-resource-usage remarks."""
    rows, cur = [], None
    for line in stderr.splitlines():
        m = re.search(r"remark: +(.*?) \[-Rpass-analysis=kernel-resource-usage\]", line)
        if not m:
            continue
        text = m.group(1)
        if text.startswith("Function Name:"):
            cur = {"name": text.split(":", 1)[1].strip()}
            rows.append(cur)
        elif cur is not None and ":" in text:
            k, v = text.split(":", 1)
            cur[k.strip()] = v.strip()
    return rows


def _compile(src: str) -> tuple[str, list[dict]]:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c",
           os.path.join(CSRC, src), "-o", obj]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{proc.stderr}")
    return obj, [dict(r, source=src) for r in _resources(proc.stderr)]


def build(verbose: bool = True) -> str:
    """Compile every kernel source and link libssd_mi355x.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        done = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in done]
    kernels = [r for _, rs in done for r in rs]
    keys = ("VGPRs", "AGPRs", "VGPRs Spill", "SGPRs Spill", "ScratchSize [bytes/lane]",
            "Occupancy [waves/SIMD]", "LDS Size [bytes/block]")
    with open(os.path.join(BUILD_DIR, "kernel_resources.txt"), "w") as f:
        f.write("source\tkernel\t" + "\t".join(keys) + "\n")
        for r in kernels:
            f.write(f"{r['source']}\t{r['name']}\t" + "\t".join(r.get(k, "?") for k in keys) + "\n")
    scratch = [r for r in kernels if r.get("ScratchSize [bytes/lane]", "0") != "0"]
    if not kernels:
        raise RuntimeError("hipcc printed no kernel resource report")
    if scratch:
        names = ", ".join(f"{r['name']} ({r['ScratchSize [bytes/lane]']} B/lane)" for r in scratch)
        raise RuntimeError(f"kernels that need scratch memory: {names}")
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc link failed:\n{proc.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}", file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build()
