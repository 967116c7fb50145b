"""Build libattn_varlen.so (gfx950) in-tree with hipcc.

    python -m varlen_flashattention_forward_amd.build

Each HIP source is compiled to an object in parallel, then linked into
varlen_flashattention_forward_amd/libattn_varlen.so. Packed FP32 VALU ops are
disabled for the device code (-packed-fp32-ops).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
ROOT = PKG.parent
LIB = Path(os.environ.get("AVF_LIB_OUT", PKG / "libattn_varlen.so"))
# the benchmark's roofline calibration kernel, in a library of its own
PROBE_LIB = PKG / "libavf_probe.so"
PROBE_SOURCE = "avf_probe.hip"
BUILD_DIR = Path(os.environ.get("AVF_BUILD_DIR", PKG / "_build"))
SOURCES = ["avf_api.hip", "avf_kernel.hip", "avf_bwd_kernel.hip", "avf_bwd_dkdv_small.hip", "avf_planner.hip",
           "avf_quant.hip"]
ARCH = os.environ.get("AVF_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libattn_varlen.so)")


def common_flags(src: str = "avf_kernel.hip") -> list:
    flags = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
             f"-I{ROOT / 'include'}", f"-I{CSRC}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    if src != "avf_bwd_kernel.hip":
        # MFMA results in architectural VGPRs, so the softmax (and rescale,
        # epilogue) read them without AGPR<->VGPR copies. avf_bwd_kernel.hip
        # holds the head_dim-128 dK/dV kernel, whose accumulators exceed 256
        # VGPRs, and leaves the choice to the compiler.
        flags += ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
    return flags + extra_flags()


def extra_flags() -> list:
    """Additional hipcc flags from AVF_EXTRA_FLAGS (tuning builds)."""
    return os.environ.get("AVF_EXTRA_FLAGS", "").split()


def _compile(src: str) -> Path:
    obj = BUILD_DIR / (Path(src).stem + ".o")
    cmd = [hipcc(), "-c", str(CSRC / src), "-o", str(obj)] + common_flags(src)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(verbose: bool = False) -> Path:
    BUILD_DIR.mkdir(parents=True, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", str(tmp)] + [str(o) for o in objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("linking libattn_varlen.so failed")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    build_probe(verbose)
    return LIB


def build_probe(verbose: bool = False) -> Path:
    """libavf_probe.so: the MFMA-rate calibration kernel bench.py --mfma-rate runs."""
    BUILD_DIR.mkdir(parents=True, exist_ok=True)
    tmp = PROBE_LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), "-shared", str(CSRC / PROBE_SOURCE), "-o", str(tmp)] + common_flags(PROBE_SOURCE)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("building libavf_probe.so failed")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {PROBE_LIB}")
    return PROBE_LIB


if __name__ == "__main__":
    build(verbose=True)
