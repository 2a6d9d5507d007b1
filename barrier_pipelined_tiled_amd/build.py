"""Build the gfx950 GEMM library (libbpt_gemm.so) in-tree with hipcc.

The library is one translation unit, ``csrc/api.hip``, which includes the
kernel headers.  Packed-fp32 VALU forms are disabled for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
SRC = os.path.join(CSRC, "api.hip")
LIB_NAME = "libbpt_gemm.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-Wl,--no-undefined",           # a missing definition fails the build, not the load
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the GEMM library needs ROCm to build")
    return path


def build(out: str = LIB_PATH, extra: list[str] | None = None) -> str:
    """Compile the library; returns the path of the shared object."""
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra or []), "-o", tmp, SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{res.stderr[-6000:]}")
    os.replace(tmp, out)
    return out


CALIB_SRC = os.path.join(CSRC, "calib.hip")
CALIB_PATH = os.path.join(PKG_DIR, "calib")


def build_calib(out: str = CALIB_PATH) -> str:
    """Compile the measurement companion (copy-kernel counter calibration and
    the MFMA throughput/clock probe); not part of the library."""
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++20",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", out, CALIB_SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{res.stderr[-6000:]}")
    return out


def device_asm(out_dir: str) -> str:
    """Emit the gfx950 assembly of the library into out_dir; returns the .s path."""
    os.makedirs(out_dir, exist_ok=True)
    s_path = os.path.join(out_dir, "api-gfx950.s")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++20",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "--cuda-device-only", "-S", "-o", s_path, SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc -S failed:\n{res.stderr[-6000:]}")
    return s_path


if __name__ == "__main__":
    print(build())
    print(build_calib())
