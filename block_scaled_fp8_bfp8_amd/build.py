"""Build libbfp8.so for gfx950 with hipcc (in-tree, next to this file).

Usage: python -m block_scaled_fp8_bfp8_amd.build
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libbfp8.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["api.hip", "quant_act.hip", "gemm_ksplit.hip", "gemm_tiled.hip", "gemm_g64.hip", "gemm_persistent.hip", "moe.hip",
           "layout.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # never emit packed-FP32 instructions (v_pk_add/mul/fma_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the per-block promotion FMAs read them directly and
    # independent MFMAs do not serialize on one accumulator register quad
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",

]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; install ROCm or put hipcc on PATH")
    return path


PROBES_LIB_NAME = "libbfp8_probes.so"
PROBES_LIB_PATH = os.path.join(PKG_DIR, PROBES_LIB_NAME)
PROBES_SOURCES = ["probes.hip"]


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile every HIP source into libbfp8.so (and the benchmark's probes into
    libbfp8_probes.so); returns the library path."""
    _compile(PROBES_SOURCES, PROBES_LIB_PATH, verbose, extra_flags)
    return _compile(SOURCES, LIB_PATH, verbose, extra_flags)


def _compile(sources: list[str], lib_path: str, verbose: bool, extra_flags: list[str] | None) -> str:
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), "-I", os.path.join(ROOT, "include"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose=True))
