"""ctypes binding of libdmuon_ns (argument marshalling only).

Every step of the Muon path runs in the HIP library; this module only turns
torch tensors into pointers, sizes and a stream handle, and error codes into
exceptions.  If the library is not built the calls raise: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# DMUON_LIBRARY selects another build of the library (the host-sanitized one of
# the CPU tests); by default the in-tree build is loaded
LIB_PATH = os.environ.get("DMUON_LIBRARY") or os.path.join(HERE, "libdmuon_ns.so")

DMUON_OK = 0
ERRORS = {
    -1: ("DMUON_E_NULL", ValueError),
    -2: ("DMUON_E_NDIM", ValueError),
    -3: ("DMUON_E_SHAPE", ValueError),
    -4: ("DMUON_E_DTYPE", ValueError),
    -5: ("DMUON_E_CFG", ValueError),
    -6: ("DMUON_E_WORKSPACE", ValueError),
    -7: ("DMUON_E_ALIAS", ValueError),
    -8: ("DMUON_E_HIP", RuntimeError),
}
F32, BF16 = 0, 1
PREC = {"bf16": 0, "f32": 1}
PHASES = ["ingest", "norm", "gram", "square", "apply", "update", "gemm_nt", "adamw"]
EXPORTED = ["dmuon_muon_step_workspace_size", "dmuon_muon_step_groups", "dmuon_muon_step",
            "dmuon_muon_step_prepare", "dmuon_muon_step_run", "dmuon_muon_step_noalloc",
            "dmuon_ns_batched_workspace_size",
            "dmuon_ns_batched", "dmuon_lpt_assign", "dmuon_adamw_step_workspace_size",
            "dmuon_adamw_step", "dmuon_gemm_nt", "dmuon_phase_timing", "dmuon_phase_timing_read",
            "dmuon_debug_slice_buffers", "dmuon_last_error", "dmuon_abi_version"]
ABI_VERSION = 5


class DmuonError(Exception):
    pass


class Tensor(ctypes.Structure):
    _fields_ = [("ndim", ctypes.c_int32), ("grad_dtype", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 3), ("grad", ctypes.c_void_p),
                ("momentum", ctypes.c_void_p), ("master", ctypes.c_void_p),
                ("ns_out", ctypes.c_void_p), ("param_out", ctypes.c_void_p)]


class StepCfg(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("momentum", ctypes.c_float),
                ("weight_decay", ctypes.c_float), ("eps", ctypes.c_float),
                ("a", ctypes.c_float), ("b", ctypes.c_float), ("c", ctypes.c_float),
                ("ns_steps", ctypes.c_int32), ("prec", ctypes.c_int32),
                ("grad_scale", ctypes.c_float), ("stream_groups", ctypes.c_int32)]


class DebugSlice(ctypes.Structure):
    _fields_ = [("x_copy", ctypes.c_void_p), ("x_rows", ctypes.c_int64), ("x_ld", ctypes.c_int64),
                ("x_oriented", ctypes.c_int32), ("elem_bytes", ctypes.c_int32),
                ("a_prime", ctypes.c_void_p), ("b_prime", ctypes.c_void_p), ("ld_m", ctypes.c_int64),
                ("scalars", ctypes.c_void_p), ("m", ctypes.c_int32), ("n", ctypes.c_int32),
                ("wide", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class AdamwTensor(ctypes.Structure):
    _fields_ = [("numel", ctypes.c_int64), ("grad_dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("grad", ctypes.c_void_p),
                ("param", ctypes.c_void_p), ("exp_avg", ctypes.c_void_p),
                ("exp_avg_sq", ctypes.c_void_p), ("param_out", ctypes.c_void_p)]


class AdamwCfg(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("grad_scale", ctypes.c_float), ("step", ctypes.c_int32)]


_lib = None


def lib():
    """Load libdmuon_ns.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m matrix_optimizer_muon_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    P = ctypes.POINTER
    L.dmuon_muon_step_workspace_size.argtypes = [P(Tensor), i32, P(StepCfg), P(sz)]
    L.dmuon_muon_step_groups.argtypes = [P(Tensor), i32, P(StepCfg), P(i32)]
    L.dmuon_muon_step.argtypes = [P(Tensor), i32, P(StepCfg), vp, sz, vp, P(vp), i32]
    L.dmuon_muon_step_prepare.argtypes = [P(Tensor), i32, P(StepCfg), vp, sz, vp]
    L.dmuon_muon_step_run.argtypes = [P(Tensor), i32, P(StepCfg), vp, sz, vp, P(vp), i32]
    L.dmuon_muon_step_noalloc.argtypes = [P(Tensor), i32, P(StepCfg), vp]
    L.dmuon_ns_batched_workspace_size.argtypes = [i64, i64, i64, i32, i32, P(sz)]
    L.dmuon_ns_batched.argtypes = [vp, i32, vp, i64, i64, i64, f32, f32, f32, i32, f32, i32, i32,
                                   vp, sz, vp]
    L.dmuon_lpt_assign.argtypes = [i64, vp, vp, vp, vp, i32, i64, i32, vp, vp, i32, vp, vp, vp, vp]
    L.dmuon_adamw_step_workspace_size.argtypes = [P(AdamwTensor), i32, P(sz)]
    L.dmuon_adamw_step.argtypes = [P(AdamwTensor), i32, P(AdamwCfg), vp, sz, vp]
    L.dmuon_gemm_nt.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, vp]
    L.dmuon_debug_slice_buffers.argtypes = [P(Tensor), i32, P(StepCfg), vp, sz, i32, i64, P(DebugSlice)]
    L.dmuon_phase_timing.argtypes = [i32]
    L.dmuon_phase_timing_read.argtypes = [vp, vp, i32]
    L.dmuon_last_error.restype = ctypes.c_char_p
    L.dmuon_last_error.argtypes = []
    L.dmuon_abi_version.restype = i32
    for name in ["dmuon_muon_step_workspace_size", "dmuon_muon_step_groups", "dmuon_muon_step",
                 "dmuon_muon_step_prepare", "dmuon_muon_step_run", "dmuon_muon_step_noalloc",
                 "dmuon_ns_batched_workspace_size", "dmuon_ns_batched", "dmuon_lpt_assign",
                 "dmuon_adamw_step_workspace_size", "dmuon_adamw_step",
                 "dmuon_gemm_nt", "dmuon_phase_timing", "dmuon_phase_timing_read"]:
        getattr(L, name).restype = ctypes.c_int
    if L.dmuon_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH} has ABI {L.dmuon_abi_version()}, expected {ABI_VERSION}: rebuild it")
    _lib = L
    return L


def check(code: int) -> None:
    if code == DMUON_OK:
        return
    name, exc = ERRORS.get(code, ("DMUON_E_?", RuntimeError))
    msg = lib().dmuon_last_error().decode(errors="replace")
    err = exc(f"{name}: {msg}")
    err.code = code
    raise err


# --------------------------------------------------------------------------
# torch-facing helpers
# --------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def resolve_stream(stream):
    """The torch stream a call runs on (the current stream when None)."""
    torch = _torch()
    return torch.cuda.current_stream() if stream is None else stream


def _stream_handle(stream):
    return ctypes.c_void_p(resolve_stream(stream).cuda_stream)


def stream_array(streams):
    """ctypes array of hipStream_t handles (and its length)."""
    arr = (ctypes.c_void_p * max(len(streams), 1))(*[s.cuda_stream for s in streams])
    return arr, len(streams)


def keep_until_done(tensor, streams):
    """Tell torch's caching allocator that ``tensor`` is used on ``streams``, so
    that its block is not handed out again before their queued work completes
    (it only tracks the stream the block was allocated on).  Skipped during
    graph capture, where the graph keeps its memory."""
    torch = _torch()
    if tensor is None or torch.cuda.is_current_stream_capturing():
        return
    for st in streams:
        tensor.record_stream(st)


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise ValueError(f"gradient dtype must be bfloat16 or float32, got {t.dtype}")


def _check_dev(t, what, dtype=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{what} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype}, got {t.dtype}")


def make_cfg(lr, momentum, weight_decay, eps, coeffs, steps, precision, grad_scale=1.0,
             stream_groups=0) -> StepCfg:
    if precision not in PREC:
        raise ValueError(f"precision must be one of {sorted(PREC)}")
    a, b, c = coeffs
    return StepCfg(lr, momentum, weight_decay, eps, a, b, c, int(steps), PREC[precision], grad_scale,
                   int(stream_groups))


def _bf16_words(t, what, shape):
    """A bf16 (or int16/uint16 raw-word) GPU tensor of ``shape``: the published copy."""
    torch = _torch()
    _check_dev(t, what)
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError(f"{what} must hold bf16 words (bfloat16, int16 or uint16)")
    if t.shape != shape:
        raise ValueError(f"{what} must have shape {tuple(shape)}")


def make_descs(grads, momenta, masters, ns_outs=None, param_outs=None):
    torch = _torch()
    n = len(grads)
    if not (len(momenta) == len(masters) == n):
        raise ValueError("grads, momenta and masters differ in length")
    if ns_outs is not None and len(ns_outs) != n:
        raise ValueError("ns_outs differs in length")
    if param_outs is not None and len(param_outs) != n:
        raise ValueError("param_outs differs in length")
    arr = (Tensor * max(n, 1))()
    for i in range(n):
        g, m, w = grads[i], momenta[i], masters[i]
        o = None if ns_outs is None else ns_outs[i]
        q = None if param_outs is None else param_outs[i]
        _check_dev(g, f"grads[{i}]")
        _check_dev(m, f"momenta[{i}]", torch.float32)
        _check_dev(w, f"masters[{i}]", torch.float32)
        if o is not None:
            _check_dev(o, f"ns_outs[{i}]", torch.float32)
        if q is not None:
            _bf16_words(q, f"param_outs[{i}]", g.shape)
        arr[i].param_out = None if q is None else q.data_ptr()
        if m.shape != g.shape or w.shape != g.shape or (o is not None and o.shape != g.shape):
            raise ValueError(f"tensor {i}: shapes of grad, momentum, master (and ns_out) differ")
        arr[i].ndim = g.dim()
        for d in range(min(g.dim(), 3)):
            arr[i].shape[d] = g.shape[d]
        arr[i].grad_dtype = _dtype_code(g)
        arr[i].grad = g.data_ptr()
        arr[i].momentum = m.data_ptr()
        arr[i].master = w.data_ptr()
        arr[i].ns_out = None if o is None else o.data_ptr()
    return arr, n


def make_adamw_descs(params, grads, exp_avgs, exp_avg_sqs, param_outs=None):
    torch = _torch()
    n = len(params)
    if not (len(grads) == len(exp_avgs) == len(exp_avg_sqs) == n):
        raise ValueError("params, grads, exp_avgs and exp_avg_sqs differ in length")
    if param_outs is not None and len(param_outs) != n:
        raise ValueError("param_outs differs in length")
    arr = (AdamwTensor * max(n, 1))()
    for i in range(n):
        p, g, m, v = params[i], grads[i], exp_avgs[i], exp_avg_sqs[i]
        q = None if param_outs is None else param_outs[i]
        _check_dev(p, f"params[{i}]", torch.float32)
        _check_dev(g, f"grads[{i}]")
        _check_dev(m, f"exp_avgs[{i}]", torch.float32)
        _check_dev(v, f"exp_avg_sqs[{i}]", torch.float32)
        if g.shape != p.shape or m.shape != p.shape or v.shape != p.shape:
            raise ValueError(f"tensor {i}: shapes of param, grad, exp_avg, exp_avg_sq differ")
        if q is not None:
            _bf16_words(q, f"param_outs[{i}]", p.shape)
        arr[i].numel = p.numel()
        arr[i].grad_dtype = _dtype_code(g)
        arr[i].reserved = 0
        arr[i].grad = g.data_ptr()
        arr[i].param = p.data_ptr()
        arr[i].exp_avg = m.data_ptr()
        arr[i].exp_avg_sq = v.data_ptr()
        arr[i].param_out = None if q is None else q.data_ptr()
    return arr, n


def muon_step_workspace_size(cfg: StepCfg, descs) -> int:
    arr, n = descs
    out = ctypes.c_size_t(0)
    check(lib().dmuon_muon_step_workspace_size(arr, n, ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def muon_step_groups(cfg: StepCfg, descs) -> int:
    arr, n = descs
    out = ctypes.c_int32(0)
    check(lib().dmuon_muon_step_groups(arr, n, ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def alloc_workspace(nbytes, device, stream=None):
    """uint8 device buffer of ``nbytes`` allocated on ``stream`` (the stream its
    kernels run on, so the allocator orders its reuse after them)."""
    torch = _torch()
    with torch.cuda.stream(resolve_stream(stream)):
        return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def lpt_assign_np(rows, cols, batch, layer_id, n_slots, merge_below_elems=0, cost_kind=0,
                  owner_slot=0):
    """Host-only LPT (no GPU needed); numpy in, dict of numpy out."""
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    batch = np.ascontiguousarray(batch, dtype=np.int64)
    layer_id = np.ascontiguousarray(layer_id, dtype=np.int32)
    n = rows.shape[0]
    slot_of = np.empty(max(n, 1), dtype=np.int32)
    slot_load = np.empty(max(n_slots, 1), dtype=np.int64)
    owner_order = np.empty(max(n, 1), dtype=np.int64)
    n_owned = ctypes.c_int64(0)
    offsets = np.empty(n + 1, dtype=np.int64)
    n_groups = ctypes.c_int32(0)
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    check(lib().dmuon_lpt_assign(n, ptr(rows), ptr(cols), ptr(batch), ptr(layer_id), n_slots,
                                 merge_below_elems, cost_kind, ptr(slot_of), ptr(slot_load),
                                 owner_slot, ptr(owner_order), ctypes.byref(n_owned),
                                 ptr(offsets), ctypes.byref(n_groups)))
    k = n_owned.value
    g = n_groups.value
    return {"slot_of": slot_of[:n].copy(), "slot_load": slot_load[:n_slots].copy(),
            "owner_order": owner_order[:k].copy(), "group_offsets": offsets[:g + 1].copy()}
