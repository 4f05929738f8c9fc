"""Builds libdmuon_ns.so (the step) and libdmuon_probe.so (the matrix-core
ceiling probe) in-tree with hipcc for gfx950.

    python -m matrix_optimizer_muon_amd.build        (or build() from Python)

Every HIP source is compiled with packed-fp32 instructions disabled; the host
sources are compiled by hipcc as well and linked against the HIP runtime.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdmuon_ns.so")
PROBE_LIB = os.path.join(HERE, "libdmuon_probe.so")
OBJ = os.path.join(HERE, "_build")
SOURCES = ["kernels.hip", "abi.cpp", "lpt.cpp"]
PROBE_SOURCES = ["probe.hip"]
ARCH = os.environ.get("DMUON_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(os.path.dirname(HERE), "include")]


# The probe's MFMAs keep their accumulators in VGPRs, as the step's contraction
# kernels do (the compiler's choice there): with them in AGPRs a wave issues
# 16×16×32 MFMAs at a lower rate and the probe would understate the ceiling.
EXTRA = {"probe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, src + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB, verbose)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
