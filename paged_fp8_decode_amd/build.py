"""Build ``libmj.so`` (the C-ABI library) for gfx950 with hipcc, in-tree.

Usage: ``python -m paged_fp8_decode_amd.build`` (or ``__graft_entry__.build()``).
Always recompiles: objects go to ``_build/`` at the repository root and the
library to ``paged_fp8_decode_amd/libmj.so``.

``build_host_sanitized()`` (``python -m paged_fp8_decode_amd.build --sanitize``)
makes a second library, ``_build/san/libmj_san.so``, for host-side checking on
a machine without a GPU: the host code of mj_host.cpp and mj_noalloc.hip
compiled with AddressSanitizer and UndefinedBehaviorSanitizer (host pass only:
every sanitizer flag sits behind ``-Xarch_host``), linked with the device
objects of the last ``build()``.  Load it with ``PAGED_FP8_DECODE_LIB`` set to
its path and the ASan runtime (``asan_runtime()``) in ``LD_PRELOAD``.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmj.so")

HIP_SOURCES = ["mj_qquant.hip", "mj_decode_generic.hip", "mj_decode_mfma.hip", "mj_plan.hip", "mj_write.hip",
               "mj_draft.hip", "mj_combine.hip", "mj_noalloc.hip"]
HOST_SOURCES = ["mj_host.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]
# Device flags: correctly rounded fp32 division (Q quantization is bit-exact
# by definition) and no packed-fp32 instructions.
DEVICE = [f"--offload-arch={ARCH}", "-fhip-fp32-correctly-rounded-divide-sqrt",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([HIPCC, *COMMON, *DEVICE, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([HIPCC, *COMMON, "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    shutil.move(tmp, LIB)
    return LIB


SAN_SOURCES = ["mj_host.cpp", "mj_noalloc.hip"]
SAN_FLAGS = [f for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
                            "-fno-omit-frame-pointer", "-g") for f in ("-Xarch_host", flag)]
SAN_LIB = os.path.join(BUILD, "san", "libmj_san.so")


def asan_runtime() -> str:
    """The shared ASan runtime of hipcc's clang (it carries the UBSan handlers too)."""
    out = _run([HIPCC, "--print-file-name=libclang_rt.asan-x86_64.so"]).strip().splitlines()[-1]
    if not os.path.isabs(out) or not os.path.exists(out):
        raise RuntimeError(f"no shared ASan runtime found (clang printed {out!r})")
    return out


def build_host_sanitized(verbose: bool = False) -> str:
    """Build ``_build/san/libmj_san.so`` (see the module docstring); needs the
    device objects of a previous ``build()``."""
    san = os.path.dirname(SAN_LIB)
    os.makedirs(san, exist_ok=True)
    objs, jobs = [], []
    for src in HIP_SOURCES + HOST_SOURCES:
        if src in SAN_SOURCES:
            obj = os.path.join(san, src + ".o")
            dev = DEVICE if src.endswith(".hip") else ["-D__HIP_PLATFORM_AMD__"]
            jobs.append([HIPCC, *COMMON, *dev, *SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        else:
            obj = os.path.join(BUILD, src + ".o")
            if not os.path.exists(obj):
                raise RuntimeError(f"{obj} is missing: run build() first")
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", SAN_LIB, *objs])
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_host_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
