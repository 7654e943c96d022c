"""Build libkvsel.so (gfx950) in-tree with hipcc.

    python -m decode_eviction_amd.build        # or __graft_entry__.build()
    python -m decode_eviction_amd.build --debug  # libkvsel_debug.so (KVSEL_DEBUG)

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
LIB_DEBUG = os.path.join(PKG, "libkvsel_debug.so")
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


def _compile(src: str, debug: bool = False) -> str:
    obj = os.path.join(BUILD, ("debug_" if debug else "") + os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *HIP_FLAGS, *EXTRA_FLAGS.get(src, []), *(["-DKVSEL_DEBUG"] if debug else []),
           "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = True, debug: bool = False) -> str:
    """Build libkvsel.so; with debug=True build libkvsel_debug.so instead,
    compiled with -DKVSEL_DEBUG (every launch waited for and a failing kernel
    named on stderr).  The binding loads the library named by the KVSEL_LIB
    environment variable when it is set."""
    os.makedirs(BUILD, exist_ok=True)
    lib = LIB_DEBUG if debug else LIB
    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda src: _compile(src, debug), SOURCES))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(debug="--debug" in sys.argv[1:])
