"""Build libkvsel.so (gfx950) in-tree with hipcc.

    python -m decode_eviction_amd.build        # or __graft_entry__.build()

Each csrc/*.hip file is compiled to an object in _build/ and linked into
decode_eviction_amd/libkvsel.so.  Every HIP compile disables the packed fp32
instructions (-packed-fp32-ops); the host pass warns that it does not know the
feature, which is harmless.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvsel.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"),
]

SOURCES = ["api.hip", "scores.hip", "gram.hip", "select.hip", "cut.hip", "fused.hip"]

# Per-file code generation options.  The Gram kernel folds every matrix-core
# result with fp32 FMAs; keeping the results (and accumulator inputs) in
# ordinary VGPRs avoids a copy out of the accumulation registers per value.
EXTRA_FLAGS = {"gram.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *HIP_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
