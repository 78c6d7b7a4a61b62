"""Builds libmoe_hip.so in-tree with hipcc for gfx950.

    python -m expert_ffn_layer_router_amd.build

Each HIP source compiles to an object under _build/ (in parallel), then one
shared library is linked next to this file.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libmoe_hip.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["router.hip", "permute.hip", "stream_gemm.hip", "prefill_gemm.hip", "combine.hip", "moe_api.hip",
           "expert_cache.hip", "measure.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is expected
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, defines=(), out_path: str = LIB_PATH, build_dir: str = BUILD_DIR) -> str:
    """Compiles every source and links `out_path`.  `defines` (e.g. "MOE_DOWN_NB=8")
    override the tile-shape constants."""
    os.makedirs(build_dir, exist_ok=True)
    hipcc = _hipcc()

    def compile_one(src):
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        out = _run([hipcc, *HIPCC_FLAGS, *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src),
                    "-o", obj])
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = out_path + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, out_path)
    if verbose:
        print(f"built {out_path}")
    return out_path


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
