"""Builds libpa.so (HIP kernels for gfx950 plus the host block pool) in place.

    python paged_kv_cache_255_amd/build.py

(run as a script: importing the package needs the library this builds).

hipcc compiles the device sources for gfx950 only; the host-only sources are
compiled as plain C++.  Objects go to _build/ at the repository root, the
library next to this file, where the Python binding loads it.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build", "libpa")
LIB = os.path.join(HERE, "libpa.so")
ARCH = "gfx950"

HIP_SOURCES = ["append.hip", "decode_valu.hip", "decode_mfma.hip", "merge.hip", "probe.hip"]
HOST_HIP_API = ["api.cpp"]           # host code that calls the HIP runtime
HOST_ONLY = ["pool.cpp", "errors.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC, "-Wall"]
# Packed-fp32 VALU instructions are kept out of the device code.  MFMA
# accumulators stay in ordinary VGPRs: the decode loop rescales them with
# VALU ops, which cannot read AGPRs, so AGPR accumulators cost a copy of
# every accumulator per block.
DEVICE_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
                "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form"]


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src):
    path = os.path.join(CSRC, src)
    obj = os.path.join(OBJDIR, src + ".o")
    if src in HIP_SOURCES:
        cmd = [_hipcc(), "-x", "hip", *DEVICE_FLAGS, *COMMON, "-c", path, "-o", obj]
    elif src in HOST_HIP_API:
        cmd = [_hipcc(), "-x", "hip", *DEVICE_FLAGS, *COMMON, "-c", path, "-o", obj]
    else:
        cmd = ["g++", *COMMON, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build():
    os.makedirs(OBJDIR, exist_ok=True)
    sources = HIP_SOURCES + HOST_HIP_API + HOST_ONLY
    with ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)
