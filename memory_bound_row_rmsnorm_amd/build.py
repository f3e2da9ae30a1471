"""Build librmsnorm_mi355x.so (and libcopy_ceiling.so, the copy the benchmark
measures against) in-tree with hipcc for gfx950.

    python -m memory_bound_row_rmsnorm_amd.build

Writes the library next to this file and the compiler's per-kernel resource
remarks (VGPRs, SGPRs, LDS, scratch, occupancy) to
``_build/kernel_resources.txt``.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBRARY = os.path.join(HERE, "librmsnorm_mi355x.so")
BUILD_DIR = os.path.join(HERE, "_build")
RESOURCES = os.path.join(BUILD_DIR, "kernel_resources.txt")

SOURCES = [os.path.join(CSRC, "rmsnorm_kernels.hip"), os.path.join(CSRC, "rmsnorm_bwd_kernels.hip"),
           os.path.join(CSRC, "rmsnorm_api.cpp")]
# the copy the benchmark measures the forward against (not part of the RMSNorm library)
COPY_LIBRARY = os.path.join(HERE, "libcopy_ceiling.so")
COPY_SOURCES = [os.path.join(CSRC, "copy_ceiling.hip")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # keep the compiler away from packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Rpass-analysis=kernel-resource-usage",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False) -> str:
    """Build the RMSNorm library (returned) and the copy-ceiling library."""
    _build_one(COPY_LIBRARY, COPY_SOURCES, os.path.join(BUILD_DIR, "copy_ceiling_resources.txt"), verbose)
    return _build_one(LIBRARY, SOURCES, RESOURCES, verbose)


def _build_one(library: str, sources: list, resources: str, verbose: bool) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    tmp = f"{library}.{os.getpid()}.tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", tmp, *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    remarks = [ln for ln in proc.stderr.splitlines() if "remark:" in ln]
    with open(resources, "w") as f:
        f.write("\n".join(remarks) + "\n")
    other = [ln for ln in proc.stderr.splitlines()
             if "remark:" not in ln and "packed-fp32-ops" not in ln and ln.strip()]
    if proc.returncode != 0:
        sys.stderr.write("\n".join(other) + "\n")
        raise RuntimeError(f"hipcc failed with exit code {proc.returncode}")
    if verbose and other:
        sys.stderr.write("\n".join(other) + "\n")
    os.replace(tmp, library)
    return library


if __name__ == "__main__":
    print(build(verbose=True))
