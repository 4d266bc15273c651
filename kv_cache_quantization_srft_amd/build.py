"""Build libsrftq.so (HIP kernels for gfx950 + the C ABI) in the package dir.

    python -m kv_cache_quantization_srft_amd.build [--jobs N]

Each translation unit is compiled by hipcc in parallel, then linked into one
shared library next to this file.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsrftq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed fp32 VALU ops are disabled (-packed-fp32-ops); fp32 denormals kept.
DEVICE_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC]


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith(".hip") or f.endswith(".cpp"))


# Development only: a comma-separated list of name fragments (e.g. "d256")
# whose already-built objects are linked as they are instead of recompiled.
# Unset (the default), every unit is compiled.
_REUSE = [f for f in os.environ.get("SRFTQ_REUSE_OBJECTS", "").split(",") if f]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    if any(f in src for f in _REUSE) and os.path.exists(obj):
        return obj
    path = os.path.join(CSRC, src)
    flags = DEVICE_FLAGS if src.endswith(".hip") else HOST_FLAGS
    if src.startswith("k_attn"):
        # MFMA results in VGPRs: the attention kernels read every score tile
        # back for VALU work, which AGPR results would have to copy first
        flags = flags + ["-mllvm", "-amdgpu-mfma-vgpr-form"]
    cmd = [HIPCC] + flags + ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    # the d = 256 units take several times longer: start them first
    srcs = sorted(sources(), key=lambda f: (0 if "d256" in f else 1, f))
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    a = ap.parse_args()
    build(a.jobs, verbose=True)
    sys.exit(0)
