"""Build libkvsel.so for gfx950 with hipcc (in-tree, next to this file).

    python -m token_selection_tsp_amd.build [--debug]

Every source is compiled for gfx950 only.  Packed fp32 instructions are
disabled (``-packed-fp32-ops``): the kernels are written as scalar fp32.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvsel.so")
SOURCES = ["score.hip", "stats.hip", "topk.hip", "gather.hip", "probe.hip", "noalloc.hip", "api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libkvsel")


def flags(debug: bool) -> list:
    f = ["-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-fvisibility=hidden",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-result"]
    f += ["-O1", "-g"] if debug else ["-O3"]
    return f


def build(debug: bool = False, verbose: bool = False) -> str:
    """Compile every source and link ``libkvsel.so``; returns its path."""
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    fl = flags(debug)

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD, src + ".o")
        cmd = [cc, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + fl
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in line)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{out}")
        if verbose and out.strip():
            print(out, file=sys.stderr)
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


HOSTCHECK = os.path.join(HERE, "libkvsel_hostcheck.so")
HOSTCHECK_SOURCES = ["api.cpp", "host_stubs.cpp"]


def build_hostcheck(verbose: bool = False) -> str:
    """Host-only build of the C ABI under AddressSanitizer and
    UndefinedBehaviorSanitizer (``libkvsel_hostcheck.so``): api.cpp's
    validation, workspace sizing and launch planning with every kernel
    launch replaced by a check of its launch description
    (csrc/host_stubs.cpp).  g++ only; no GPU code is built with a sanitizer.
    Returns its path."""
    cxx = shutil.which("g++")
    if cxx is None:
        raise RuntimeError("g++ not found: the host sanitizer build needs it")
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fvisibility=hidden",
           "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"), "-I", INCLUDE, "-I", CSRC,
           "-Wall", "-o", HOSTCHECK + ".tmp"] + [os.path.join(CSRC, f) for f in HOSTCHECK_SOURCES]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host sanitizer build failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    if verbose and (r.stdout + r.stderr).strip():
        print(r.stdout + r.stderr, file=sys.stderr)
    os.replace(HOSTCHECK + ".tmp", HOSTCHECK)
    return HOSTCHECK


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--debug", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--hostcheck", action="store_true", help="also build the host sanitizer library")
    a = ap.parse_args()
    print(build(debug=a.debug, verbose=a.verbose))
    if a.hostcheck:
        print(build_hostcheck(verbose=a.verbose))


if __name__ == "__main__":
    main()
