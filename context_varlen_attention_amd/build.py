"""Build libcva.so in-tree: HIP kernels for gfx950 with hipcc, host C++ with g++.

Usage: python -m context_varlen_attention_amd.build  (or build() from Python).
Every call recompiles everything; objects go to a scratch folder next to the
package and the library to context_varlen_attention_amd/libcva.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
LIB = os.path.join(PKG, "libcva.so")

HOST_SOURCES = ["host/validate.cpp", "host/metadata.cpp", "host/schedule.cpp", "host/placement.cpp",
                "capi/cva.cpp"]
HIP_SOURCES = ["kernels/fwd.hip", "kernels/bwd.hip"]

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=fast",
    # no NaN inputs are expected: lets max/min skip NaN quieting (v_max3 chains)
    "-fno-honor-nans",
    # packed fp32 VALU forms are disabled for every HIP translation unit
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__"]
# Host-only checking build (build_host_sanitized): AddressSanitizer and
# UndefinedBehaviorSanitizer on the host C++ (g++ only; the HIP kernels are
# built exactly as in the product library and are not instrumented).
SANITIZE_HOST_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                       "-fno-sanitize-recover=all"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 8) -> str:
    from concurrent.futures import ThreadPoolExecutor

    objdir = tempfile.mkdtemp(prefix="cva_build_")
    try:
        inc = ["-I", INCLUDE, "-I", CSRC, "-I", os.path.join(ROCM, "include")]
        cmds = []
        objs = []
        for src in HIP_SOURCES:
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            cmds.append([HIPCC, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj])
            objs.append(obj)
        for src in HOST_SOURCES:
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            cmds.append(["g++", *HOST_FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj])
            objs.append(obj)
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            outs = list(ex.map(_run, cmds))
        if verbose:
            for o in outs:
                if o.strip():
                    print(o)
        tmp = LIB + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return LIB


def build_host_sanitized(out_path: str, jobs: int = 8) -> str:
    """libcva with its host C++ (validation, metadata, schedules, placement, C
    ABI) compiled with ASan + UBSan, for CPU test runs with the sanitizer
    runtime preloaded (the binding loads it when CVA_LIBRARY names it)."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = tempfile.mkdtemp(prefix="cva_san_")
    try:
        inc = ["-I", INCLUDE, "-I", CSRC, "-I", os.path.join(ROCM, "include")]
        cmds, objs = [], []
        for src in HIP_SOURCES:
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            cmds.append([HIPCC, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj])
            objs.append(obj)
        host_flags = [f for f in HOST_FLAGS if f != "-O2"] + SANITIZE_HOST_FLAGS
        for src in HOST_SOURCES:
            obj = os.path.join(objdir, os.path.basename(src) + ".san.o")
            cmds.append(["g++", *host_flags, *inc, "-c", os.path.join(CSRC, src), "-o", obj])
            objs.append(obj)
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            list(ex.map(_run, cmds))
        rocm_lib = os.path.join(ROCM, "lib")
        _run(["g++", "-shared", "-fPIC", *SANITIZE_HOST_FLAGS, *objs, "-o", out_path,
              "-L", rocm_lib, "-Wl,-rpath," + rocm_lib, "-lamdhip64"])
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return out_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
