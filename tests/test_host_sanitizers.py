"""The host side of libdmuon_ns under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Argument validation, planning, workspace layout, table building and the LPT
partition (``abi.cpp``, ``lpt.cpp``) are rebuilt with both sanitizers
(``matrix_optimizer_muon_amd.build_sanitized``; the HIP kernels are linked
unchanged) and ``tests/test_abi_host.py`` runs against that build in a child
process with the ASan runtime preloaded.  Any sanitizer report fails the test.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_host_suite_under_asan_and_ubsan(tmp_path):
    from matrix_optimizer_muon_amd import build_sanitized as bs
    lib = bs.build(str(tmp_path))
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle" in syms     # instrumented
    env = dict(os.environ, LD_PRELOAD=bs.asan_runtime(), DMUON_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    probe = subprocess.run([sys.executable, "-c", "from matrix_optimizer_muon_amd import _binding as B; "
                            "print(B.lib()._name)"], cwd=ROOT, env=env, capture_output=True, text=True,
                           timeout=300)
    assert probe.returncode == 0 and probe.stdout.strip() == lib, probe.stdout + probe.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join("tests", "test_abi_host.py")], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in r.stdout
