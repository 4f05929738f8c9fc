"""Host-side checks of libdmuon_probe (the matrix-core ceiling probe) that need
no GPU: it loads, exports what include/dmuon_probe.h declares, the header
compiles as strict C99, and bad arguments are rejected before any HIP call."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

from matrix_optimizer_muon_amd import probe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dmuon_probe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(probe.PROBE_LIB_PATH), reason="libdmuon_probe.so is not built")


def header_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(dmuon_probe_[a-z_0-9]+)\s*\(", text)))


def test_probe_exports_every_header_function():
    L = probe.load_probe()
    names = header_functions()
    assert names == sorted(probe.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


@pytest.mark.parametrize("args, code, text", [
    ((8, 0, 1, 4), -3, "shape"),
    ((32, 2, 1, 4), -3, "operands"),
    ((32, 0, 0, 4), -3, "blocks"),
    ((16, 0, 65537, 4), -3, "blocks"),
    ((32, 0, 1, 6), -3, "iters"),
    ((32, 0, 1, 0), -3, "iters"),
    ((16, 1, 1, (1 << 24) + 4), -3, "iters"),
])
def test_probe_rejects_bad_arguments(args, code, text):
    L = probe.load_probe()
    rc = L.dmuon_probe_mfma(*args, ctypes.c_void_p(0x7F0000000000), None)
    assert rc == code
    assert text in L.dmuon_probe_last_error().decode()
    with pytest.raises(ValueError, match=text):
        probe.probe_mfma(*args, 0x7F0000000000, 0)


def test_probe_rejects_null_sink():
    L = probe.load_probe()
    assert L.dmuon_probe_mfma(32, 0, 1, 4, None, None) == -1
    assert "sink" in L.dmuon_probe_last_error().decode()


def test_probe_flop_count():
    # one round: 8 × (32·32·16) or 16 × (16·16·32) multiply-adds per wave
    assert probe.FLOPS_PER_WAVE_ROUND == 2 * 8 * 32 * 32 * 16 == 2 * 16 * 16 * 16 * 32
    assert probe.flops_per_launch(2048, 20000) == 2048 * 4 * 20000 * 262144


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_probe_header_is_c99(tmp_path):
    src = tmp_path / "p.c"
    src.write_text('#include "dmuon_probe.h"\n'
                   "int main(void) { return dmuon_probe_mfma(7, DMUON_PROBE_RANDOM, 1, 4, 0, 0) == DMUON_E_SHAPE ? 0 : 1; }\n")
    exe = tmp_path / "p"
    libdir = os.path.dirname(probe.PROBE_LIB_PATH)
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                        str(src), "-o", str(exe), "-L", libdir, "-ldmuon_probe", f"-Wl,-rpath,{libdir}",
                        "-Wl,-rpath,/opt/rocm/lib"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert subprocess.run([str(exe)], timeout=60).returncode == 0
