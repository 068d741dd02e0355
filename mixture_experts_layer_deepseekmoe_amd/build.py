"""Build libmoe_mi355x.so (all HIP kernels + the C ABI) for gfx950 with hipcc.

    python -m mixture_experts_layer_deepseekmoe_amd.build

Objects go to _build/ at the repository root; the shared library is written
next to this file, where the binding loads it from.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# the bounds-checked build (-DMOE_DEBUG: device-side index checks, read back
# after every call), loaded only where asked for
DEBUG_LIB_PATH = os.path.join(PKG, "libmoe_mi355x_debug.so")

SOURCES = ["route.hip", "group.hip", "ggemm.hip", "combine.hip", "bwd.hip", "moe_api.cpp"]
ARCH = "gfx950"
# measured-ceiling probes (MFMA with random / zero operands, HBM stream), a
# standalone program run by `profiling.py peaks`
PROBES_SRC = os.path.join(PKG, "peaks", "peak_probes.hip")
PROBES_BIN = os.path.join(PKG, "peak_probes.bin")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the MoE library)")


def common_flags(debug: bool = False):
    flags = [f"--offload-arch={ARCH}", "-std=c++20", "-fPIC", "-Wall", "-Wno-unused-function",
             "-I", os.path.join(ROOT, "include"),
             # keep every packed-fp32 VALU form out of the generated code
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             # MFMA accumulators in VGPRs: with 256 live accumulator registers
             # the AGPR form makes the allocator rotate them through copies
             "-mllvm", "-amdgpu-mfma-vgpr-form"]
    flags += ["-O3", "-g", "-DMOE_DEBUG=1"] if debug else ["-O3"]
    return flags


def _compile(src: str, debug: bool) -> str:
    obj = os.path.join(BUILD, ("debug_" if debug else "") + os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags(debug) + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj


def build(verbose: bool = True, debug: bool = False) -> str:
    """Build the library (debug: the bounds-checked one, at DEBUG_LIB_PATH)."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, debug), SOURCES))
    path = DEBUG_LIB_PATH if debug else LIB_PATH
    tmp = path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, path)
    if debug:
        if verbose:
            print(f"built {path}")
        return path
    cmd = [hipcc()] + common_flags(debug) + ["-o", PROBES_BIN + ".tmp", PROBES_SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for peak_probes.hip:\n{res.stderr}")
    os.replace(PROBES_BIN + ".tmp", PROBES_BIN)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    if "--debug" in sys.argv:
        build(debug=True)
    else:
        build()
        if "--with-debug" in sys.argv:
            build(debug=True)
