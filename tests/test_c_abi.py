"""The C ABI from a plain C99 program (CPU): tests/c/abi_host.c is compiled
with gcc against include/dmuon_ns.h (strict C99, warnings as errors), linked
against the in-tree library and run; it checks the host-only entry points."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "matrix_optimizer_muon_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c99_program_uses_the_abi(tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "libdmuon_ns.so")):
        pytest.skip("libdmuon_ns.so is not built")
    exe = tmp_path / "abi_host"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_host.c"), "-o", str(exe), "-L", LIBDIR, "-ldmuon_ns",
           f"-Wl,-rpath,{LIBDIR}", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout, r.stderr)
