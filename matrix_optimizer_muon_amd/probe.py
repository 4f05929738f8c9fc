"""ctypes binding of libdmuon_probe (the matrix-core ceiling probe; argument
marshalling only).  The probe is not part of the Muon step: it measures what
the matrix cores sustain on register operands, under the board's power limit,
as a reference for the step's contraction kernels.  Raises if the library is
not built; there is no fallback."""
from __future__ import annotations

import ctypes
import os

from ._binding import ERRORS, DmuonError

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(HERE, "libdmuon_probe.so")
EXPORTED = ["dmuon_probe_mfma", "dmuon_probe_last_error"]
RANDOM, ZERO = 0, 1
THREADS = 256
FLOPS_PER_WAVE_ROUND = 262144      # 131072 multiply-adds per wave and round, either shape

_lib = None


def load_probe():
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise RuntimeError(f"{PROBE_LIB_PATH} is not built (python -m matrix_optimizer_muon_amd.build)")
        lib = ctypes.CDLL(PROBE_LIB_PATH)
        lib.dmuon_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_void_p, ctypes.c_void_p]
        lib.dmuon_probe_mfma.restype = ctypes.c_int
        lib.dmuon_probe_last_error.argtypes = []
        lib.dmuon_probe_last_error.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def probe_mfma(shape: int, operands: int, blocks: int, iters: int, sink_ptr: int, stream_handle: int) -> None:
    """One probe launch (see dmuon_probe.h); sink_ptr holds blocks × 256 floats."""
    lib = load_probe()
    rc = lib.dmuon_probe_mfma(shape, operands, blocks, iters, ctypes.c_void_p(sink_ptr),
                              ctypes.c_void_p(stream_handle))
    if rc != 0:
        name, exc = ERRORS.get(rc, ("unknown", RuntimeError))
        raise exc(f"dmuon_probe_mfma: {name}: {lib.dmuon_probe_last_error().decode()}")


def flops_per_launch(blocks: int, iters: int) -> int:
    return blocks * (THREADS // 64) * iters * FLOPS_PER_WAVE_ROUND


__all__ = ["load_probe", "probe_mfma", "flops_per_launch", "RANDOM", "ZERO", "DmuonError", "EXPORTED"]
