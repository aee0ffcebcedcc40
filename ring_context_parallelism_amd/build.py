"""Build libcpattn.so (HIP, gfx950) in-tree.

    python -m ring_context_parallelism_amd.build [-v]

Every translation unit is compiled by hipcc for gfx950 only and linked into
``ring_context_parallelism_amd/libcpattn.so`` next to this file.  Objects go
to ``ring_context_parallelism_amd/_build/``.  Always recompiles.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcpattn.so")

SOURCES = ["plan.cpp", "api.hip", "attn_bf16.hip", "attn_f32.hip", "attn_bwd.hip", "attn_bwd_bf16.hip", "layout_merge.hip"]
ARCH = "gfx950"

COMMON = ["-std=c++17", "-O3", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]
# gfx950 device code: no packed-fp32 instructions anywhere.
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-fno-gpu-rdc"]

# Per-file device flags.  The eight-wave key-major backward kernel branches
# on a wave-uniform role into two loops; by default the control-flow
# structurizer sequences the two branches one after the other behind flags,
# and the wait-count insertion then treats one role's loads as in flight in
# the other's loop (stalling its matrix work on them).  Keeping uniform
# regions as they are avoids that.
TU_FLAGS = {"attn_bwd_bf16.hip": ["-mllvm", "-structurizecfg-skip-uniform-regions=true"]}


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src, verbose):
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    if src.endswith(".hip"):
        cmd = [hipcc(), "-x", "hip", *HIP_FLAGS, *TU_FLAGS.get(src, []), *COMMON, "-c", path, "-o", obj]
    else:
        cmd = [hipcc(), *COMMON, "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, flush=True)
    return obj


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
