"""Builds a host-sanitized variant of libdmuon_ns for the CPU test suite.

    python -m matrix_optimizer_muon_amd.build_sanitized [OUT_DIR]

The host sources (argument validation, planning, table building, LPT) are
compiled by g++ with AddressSanitizer and UndefinedBehaviorSanitizer; the HIP
kernels are linked from the regular build's object unchanged (no GPU code is
instrumented).  A Python process loads the result with the ASan runtime
preloaded (``LD_PRELOAD``) and ``DMUON_LIBRARY`` pointing at it.
"""
from __future__ import annotations

import os
import subprocess
import sys

from . import build as _build

HOST_SOURCES = ["abi.cpp", "lpt.cpp"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    return subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


def build(out_dir: str) -> str:
    os.makedirs(out_dir, exist_ok=True)
    kobj = os.path.join(_build.OBJ, "kernels.hip.o")
    if not os.path.exists(kobj):
        _build.build()
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(out_dir, src + ".san.o")
        cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", *SAN, "-D__HIP_PLATFORM_AMD__",
               "-I/opt/rocm/include", "-I", os.path.join(os.path.dirname(_build.HERE), "include"),
               "-c", os.path.join(_build.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"g++ failed for {src}:\n{r.stdout}{r.stderr}")
        objs.append(obj)
    lib = os.path.join(out_dir, "libdmuon_ns_san.so")
    cmd = ["g++", "-shared", *SAN, *objs, kobj, "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib",
           "-lamdhip64", "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    return lib


if __name__ == "__main__":
    print(build(sys.argv[1] if len(sys.argv) > 1 else os.path.join(_build.HERE, "_build", "san")))
