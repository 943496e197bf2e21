"""Build libkvq.so (the C-ABI library with the gfx950 HIP kernels) in the package directory.

    python -m kv_cache_quantization_srft_amd.build

Every source is compiled with hipcc for gfx950 only, in parallel, then linked into
kv_cache_quantization_srft_amd/libkvq.so.  Packed-FP32 VALU instructions are disabled for the
device code (-packed-fp32-ops); hipcc's host pass prints that it does not know that feature,
which is harmless.  MFMA instructions write their results to ordinary VGPRs
(-amdgpu-mfma-vgpr-form), which saves the copies out of accumulator registers.
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
OUT = os.path.join(PKG, "libkvq.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["kvq_dequant.hip", "kvq_quant.hip", "kvq_decode_q128.hip", "kvq_decode_q256.hip", "kvq_decode_f16.hip",
           "kvq_noalloc.hip", "kvq_plan.cpp", "kvq_api.cpp"]
ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fconstexpr-steps=100000000", "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"),
    # MFMA results in VGPRs (gfx950 has one register file): no accumulator-register copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; a ROCm toolchain is required to build libkvq.so")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build()
