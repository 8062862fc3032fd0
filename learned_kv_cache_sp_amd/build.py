"""Build libspkv.so (HIP, gfx950) in-tree with hipcc.

Every source under csrc/ is compiled for gfx950 only, with packed-FP32
instruction selection disabled, and linked into one shared library next to
this file.  Objects are compiled in parallel; the whole build takes a few
tens of seconds on a CPU-only machine.

The build fails if any kernel needs scratch (private) memory: in these
kernels that only ever means a register array the compiler could not keep in
registers, which turns a streaming loop into a string of dependent waits.
The compiler's resource-usage remarks give each kernel's figure.
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
LIB = os.path.join(HERE, "libspkv.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["spkv_api.cpp", "spkv_gate.hip", "spkv_compact.hip", "spkv_decode.hip", "spkv_prefill.hip", "spkv_stats.hip", "spkv_ceiling.hip"]

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found (ROCm is required to build libspkv)")
    return p


# Kernels allowed a non-zero scratch size (exact (kernel, bytes per lane)
# pairs, each checked in its ISA to hold no spilled data).  None at present.
SCRATCH_ALLOWED: set = set()


def scratch_kernels(remarks: str) -> list:
    """(kernel, bytes per lane) of every kernel with a non-zero scratch size in
    hipcc's kernel-resource-usage remarks."""
    out, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name is not None and int(m.group(1)) > 0:
            out.append((name, int(m.group(1))))
    return out


def _compile(src: str) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    else:
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    bad = [k for k in scratch_kernels(r.stderr) if k not in SCRATCH_ALLOWED]
    if bad:
        raise RuntimeError(f"{src}: kernels using scratch memory (bytes per lane): {bad}")
    return obj


def build(verbose: bool = False) -> str:
    # a failed build must not leave the previous library behind to be tested
    if os.path.exists(LIB):
        os.remove(LIB)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    # -z defs: an object that lost a kernel stub (or any symbol) fails the link
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
