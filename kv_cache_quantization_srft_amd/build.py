"""Build libsrftq.so (HIP kernels for gfx950 + the C ABI) in the package dir.

    python -m kv_cache_quantization_srft_amd.build [--jobs N] [--incremental] [--poison]

Each translation unit is compiled by hipcc in parallel, then linked into one
shared library next to this file.  --poison builds the debug variant
libsrftq_poison.so instead (SRFTQ_LDS_POISON=1: the single-wave streaming
kernels fill their LDS buffers with 0xff bytes before each use), which the
tests load through SRFTQ_LIBRARY.  build_memfloor() links
libsrftq_memfloor.so, the benchmark's memory-floor kernels (no arithmetic of
the method; bench.py alone loads it).
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
BUILD_POISON = os.path.join(PKG, "_build_poison")
LIB_POISON = os.path.join(PKG, "libsrftq_poison.so")
MEMFLOOR_SRC = os.path.join(PKG, "memfloor", "memfloor.hip")
LIB_MEMFLOOR = os.path.join(PKG, "libsrftq_memfloor.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed fp32 VALU ops are disabled (-packed-fp32-ops); fp32 denormals kept.
DEVICE_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC]


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith(".hip") or f.endswith(".cpp"))


def _deps(obj: str) -> list[str]:
    """Files an object was built from, as the compiler's -MMD output lists them."""
    dep = obj + ".d"
    if not os.path.exists(dep):
        return []
    text = open(dep).read().replace("\\\n", " ")
    body = text.split(":", 1)[1] if ":" in text else ""
    return [f for f in body.split() if f]


def _up_to_date(src: str, obj: str, flags: list[str]) -> bool:
    """make's rule: the object is newer than its source and every header the
    compiler read for it, and was built with the same flags."""
    if not os.path.exists(obj) or not os.path.exists(obj + ".flags"):
        return False
    if open(obj + ".flags").read() != " ".join(flags):
        return False
    deps = _deps(obj)
    if not deps:
        return False
    t = os.path.getmtime(obj)
    return all(os.path.exists(f) and os.path.getmtime(f) <= t for f in deps + [src])


def _compile(src: str, incremental: bool = False, poison: bool = False) -> str:
    obj = os.path.join(BUILD_POISON if poison else BUILD, src + ".o")
    path = os.path.join(CSRC, src)
    flags = DEVICE_FLAGS if src.endswith(".hip") else HOST_FLAGS
    if poison:
        flags = flags + ["-DSRFTQ_LDS_POISON=1"]
    if src.startswith("k_attn"):
        # MFMA results in VGPRs: the attention kernels read every score tile
        # back for VALU work, which AGPR results would have to copy first
        flags = flags + ["-mllvm", "-amdgpu-mfma-vgpr-form"]
    if incremental and _up_to_date(path, obj, flags):
        return obj
    cmd = [HIPCC] + flags + ["-MMD", "-MF", obj + ".d", "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    with open(obj + ".flags", "w") as f:
        f.write(" ".join(flags))
    return obj


def build_memfloor(verbose: bool = False) -> str:
    """Link libsrftq_memfloor.so: the benchmark's memory-floor kernels, kept
    out of libsrftq.so (they compute nothing of the method)."""
    tmp = LIB_MEMFLOOR + ".tmp"
    cmd = [HIPCC] + DEVICE_FLAGS + ["-shared", "-o", tmp, MEMFLOOR_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_MEMFLOOR)
    if verbose:
        print(f"built {LIB_MEMFLOOR}")
    return LIB_MEMFLOOR


def build(jobs: int | None = None, verbose: bool = False, incremental: bool = False, poison: bool = False) -> str:
    """Compile every unit (incremental: only those whose object is older
    than the source or a header it includes) and link libsrftq.so (poison:
    the debug variant libsrftq_poison.so)."""
    lib_path = LIB_POISON if poison else LIB
    os.makedirs(BUILD_POISON if poison else BUILD, exist_ok=True)
    # the d = 256 units take several times longer: start them first
    srcs = sorted(sources(), key=lambda f: (0 if "d256" in f else 1, f))
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda f: _compile(f, incremental, poison), srcs))
    tmp = lib_path + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--incremental", action="store_true",
                    help="recompile only units whose source or included headers changed")
    ap.add_argument("--poison", action="store_true", help="build the LDS-poison debug variant")
    a = ap.parse_args()
    build(a.jobs, verbose=True, incremental=a.incremental, poison=a.poison)
    if not a.poison:
        build_memfloor(verbose=True)
    sys.exit(0)
