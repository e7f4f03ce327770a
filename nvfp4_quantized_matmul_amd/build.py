"""Build libnvfp4.so (HIP kernels + C ABI) for gfx950, in-tree, and the
benchmark's measurement aid libnvfp4_measure.so (not part of the library).

Usage: ``python -m nvfp4_quantized_matmul_amd.build`` (or call :func:`build`).
Every call recompiles; object files go to ``_build/`` at the repository root
and the shared libraries are written next to this file.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libnvfp4.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
MEASURE_DIR = os.path.join(PKG_DIR, "measure")
MEASURE_LIB_PATH = os.path.join(PKG_DIR, "libnvfp4_measure.so")
ARCH = "gfx950"

# Packed-FP32 VALU forms are disabled for every device compile.
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]

# Per-source extra flags.  The one-row decode kernels take their first 16
# argument dwords preloaded into SGPRs by the dispatcher (no scalar load of
# the argument segment before the first address is known): measured 1.5-2%
# faster on the decode workload, 2-3% on the MoE decode gather; the
# multi-row kernel, the matrix-core gather and the GEMMs measured neutral to
# 1% slower with it.
FILE_FLAGS = {
    "decode.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=16"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libnvfp4")


def sources(directory: str = CSRC):
    return sorted(os.path.join(directory, f) for f in os.listdir(directory) if f.endswith(".hip"))


def _compile(src: str, cc: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(os.path.dirname(src)) + "_" + os.path.basename(src) + ".o")
    cmd = [cc, *HIP_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-I", INCLUDE, "-I", os.path.dirname(src), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def _link(cc: str, objs, path: str) -> None:
    tmp = path + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libnvfp4.so (and the benchmark's
    libnvfp4_measure.so); returns the library's path."""
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs, msrcs = sources(), sources(MEASURE_DIR)
    jobs = max(1, min(len(srcs) + len(msrcs), int(os.environ.get("MAX_JOBS", "8")), 16))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, cc), srcs + msrcs))
    _link(cc, objs[:len(srcs)], LIB_PATH)
    _link(cc, objs[len(srcs):], MEASURE_LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources and {MEASURE_LIB_PATH} from {len(msrcs)}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
