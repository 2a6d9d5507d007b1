"""Build the gfx950 GEMM library (libbpt_gemm.so) in-tree with hipcc.

The library is one translation unit, ``csrc/api.hip``, which includes the
kernel headers.  Packed-fp32 VALU forms are disabled for all device code.
The same compilation keeps its gfx950 assembly (-save-temps, in ``_build/``)
and writes ``libbpt_gemm.kernels.json`` beside the library: every kernel's
resource use and a hash of its machine code (asm_info).

``build_poison`` compiles the same source with ``BPT_LDS_POISON`` into
``libbpt_gemm_poison.so``, a race-detection build whose every LDS-DMA copy
first fills its destination with NaN (its assembly is kept in
``_build/poison/``).
"""
from __future__ import annotations

import json
import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
SRC = os.path.join(CSRC, "api.hip")
LIB_NAME = "libbpt_gemm.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"
BUILD_DIR = os.path.join(PKG_DIR, "_build")
ASM_PATH = os.path.join(BUILD_DIR, f"api-hip-amdgcn-amd-amdhsa-{ARCH}.s")
KERNELS_JSON = os.path.join(PKG_DIR, "libbpt_gemm.kernels.json")
POISON_LIB_PATH = os.path.join(PKG_DIR, "libbpt_gemm_poison.so")
POISON_BUILD_DIR = os.path.join(BUILD_DIR, "poison")
POISON_ASM_PATH = os.path.join(POISON_BUILD_DIR, f"api-hip-amdgcn-amd-amdhsa-{ARCH}.s")

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


def build(out: str = LIB_PATH, extra: list[str] | None = None, build_dir: str = BUILD_DIR) -> str:
    """Compile the library; returns the path of the shared object.  Also
    keeps the device assembly (in build_dir) and, for the library itself,
    writes the kernel table (kernel_table)."""
    os.makedirs(build_dir, exist_ok=True)
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-save-temps", *(extra or []), "-o", tmp, SRC]
    res = subprocess.run(cmd, capture_output=True, text=True, cwd=build_dir)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{res.stderr[-6000:]}")
    os.replace(tmp, out)
    if out == LIB_PATH:
        write_kernel_table()
    return out


def build_poison() -> str:
    """The LDS-poison race-detection build of the same source."""
    return build(POISON_LIB_PATH, ["-DBPT_LDS_POISON"], POISON_BUILD_DIR)


def write_kernel_table(asm_path: str = ASM_PATH, path: str = KERNELS_JSON) -> dict:
    """name -> {"code": hash of the kernel's machine code, resource use} for
    every kernel of the library, from the kept assembly."""
    try:
        from . import asm_info
    except ImportError:                # run as a script
        import asm_info
    with open(asm_path) as f:
        ks = asm_info.kernels(f.read())
    table = {n: dict(code=asm_info.code_hash(k), **k["meta"]) for n, k in sorted(ks.items())}
    with open(path, "w") as f:
        json.dump(table, f, indent=1)
        f.write("\n")
    return table


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
    """Emit the gfx950 assembly of the library into out_dir (a compilation of
    its own; build() keeps the same text in ASM_PATH); returns the .s path."""
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
    print(build_poison())
    print(build_calib())
