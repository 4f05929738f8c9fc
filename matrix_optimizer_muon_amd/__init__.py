"""matrix_optimizer_muon_amd — the owner-rank Muon optimizer step on MI355X.

Python face of libdmuon_ns (C ABI in ``include/dmuon_ns.h``).  The functions
below only marshal arguments: momentum, normalisation, Newton–Schulz and the
update all run in the library's HIP kernels on the caller's current stream.

    muon_step(grads, momenta, masters, lr=0.02, momentum=0.95, ...)
    adamw_step(params, grads, exp_avgs, exp_avg_sqs, step=1, ...)  # the "adamw" route
    ns_batched(x, coeffs=(3.4445, -4.775, 2.0315), steps=5, ...)
    lpt_assign(rows, cols, batch, layer_id, n_slots, ...)   # host only
"""
from __future__ import annotations

import ctypes

from . import _binding as _b
from .workloads import HYPER  # noqa: F401

__all__ = ["muon_step", "muon_step_workspace_size", "adamw_step", "MuonStep", "AdamwStep",
           "ns_batched", "lpt_assign", "gemm_nt",
           "phase_timing", "phase_timing_read", "abi_version", "load_library", "HYPER"]

QUINTIC = (HYPER["a"], HYPER["b"], HYPER["c"])


def load_library():
    """Load the HIP library (raises RuntimeError if it is not built)."""
    return _b.lib()


def abi_version() -> int:
    return int(_b.lib().dmuon_abi_version())


def _cfg(lr, momentum, weight_decay, eps, coeffs, steps, precision):
    return _b.make_cfg(lr, momentum, weight_decay, eps, coeffs, steps, precision)


def muon_step_workspace_size(grads, momenta, masters, *, steps=5, precision="bf16",
                             ns_outs=None) -> int:
    cfg = _cfg(0.0, 0.0, 0.0, 0.0, QUINTIC, steps, precision)
    descs = _b.make_descs(grads, momenta, masters, ns_outs)
    return _b.muon_step_workspace_size(cfg, descs)


class MuonStep:
    """A prepared owner-rank Muon step over a fixed set of tensors.

    The tensors are checked and marshalled once; every call enqueues one step
    (``dmuon_muon_step``) on ``stream``.  The tensors must stay alive and keep
    their storage; ``lr`` may be changed between calls.  Arguments as for
    ``muon_step``.
    """

    def __init__(self, grads, momenta, masters, *, lr=HYPER["lr"], momentum=HYPER["mu"],
                 weight_decay=HYPER["wd"], eps=HYPER["eps"], coeffs=QUINTIC, steps=HYPER["steps"],
                 precision="bf16", grad_scale=1.0, ns_outs=None, param_outs=None, workspace=None):
        self._tensors = (list(grads), list(momenta), list(masters), ns_outs, param_outs)
        self.cfg = _b.make_cfg(lr, momentum, weight_decay, eps, coeffs, steps, precision, grad_scale)
        self.arr, self.n = _b.make_descs(grads, momenta, masters, ns_outs, param_outs)
        self.workspace = None
        if self.n:
            need = _b.muon_step_workspace_size(self.cfg, (self.arr, self.n))
            if workspace is None:
                workspace = _b.alloc_workspace(need, grads[0].device)
            self.workspace = workspace

    @property
    def lr(self):
        return self.cfg.lr

    @lr.setter
    def lr(self, value):
        self.cfg.lr = value

    def __call__(self, stream=None) -> None:
        if self.n == 0:
            return
        ws = self.workspace
        _b.check(_b.lib().dmuon_muon_step(self.arr, self.n, ctypes.byref(self.cfg),
                                          ctypes.c_void_p(ws.data_ptr()),
                                          ws.numel() * ws.element_size(), _b._stream_handle(stream)))


def muon_step(grads, momenta, masters, *, lr=HYPER["lr"], momentum=HYPER["mu"],
              weight_decay=HYPER["wd"], eps=HYPER["eps"], coeffs=QUINTIC, steps=HYPER["steps"],
              precision="bf16", grad_scale=1.0, ns_outs=None, param_outs=None, workspace=None,
              stream=None) -> None:
    """One owner-rank Muon step over all given tensors, enqueued on ``stream``.

    grads: bf16/fp32 GPU tensors (2-D or 3-D), read as grad_scale·grad; momenta,
    masters: fp32, updated in place; ns_outs: optional fp32 tensors that receive
    the Newton–Schulz output; param_outs: optional bf16 tensors that receive the
    updated master rounded to bf16 (the published parameter).
    workspace: optional uint8 GPU tensor of at least ``muon_step_workspace_size``
    bytes (allocated here when omitted).
    """
    MuonStep(grads, momenta, masters, lr=lr, momentum=momentum, weight_decay=weight_decay, eps=eps,
             coeffs=coeffs, steps=steps, precision=precision, grad_scale=grad_scale,
             ns_outs=ns_outs, param_outs=param_outs, workspace=workspace)(stream)


class AdamwStep:
    """A prepared ``adamw``-route step over a fixed set of tensors.

    Marshals once; ``step_fn(step)`` enqueues one AdamW step with bias-correction
    step number ``step`` (≥ 1).  Arguments as for ``adamw_step``.
    """

    def __init__(self, params, grads, exp_avgs, exp_avg_sqs, *, lr=1e-3, betas=(0.9, 0.999),
                 eps=1e-8, weight_decay=0.01, grad_scale=1.0, param_outs=None, workspace=None):
        self._tensors = (list(params), list(grads), list(exp_avgs), list(exp_avg_sqs), param_outs)
        self.arr, self.n = _b.make_adamw_descs(params, grads, exp_avgs, exp_avg_sqs, param_outs)
        self.cfg = _b.AdamwCfg(lr, betas[0], betas[1], eps, weight_decay, grad_scale, 1)
        self.workspace = None
        if self.n:
            need = ctypes.c_size_t(0)
            _b.check(_b.lib().dmuon_adamw_step_workspace_size(self.arr, self.n, ctypes.byref(need)))
            if workspace is None:
                workspace = _b.alloc_workspace(need.value, params[0].device)
            self.workspace = workspace

    @property
    def lr(self):
        return self.cfg.lr

    @lr.setter
    def lr(self, value):
        self.cfg.lr = value

    def __call__(self, step, stream=None) -> None:
        if self.n == 0:
            return
        self.cfg.step = int(step)
        ws = self.workspace
        _b.check(_b.lib().dmuon_adamw_step(self.arr, self.n, ctypes.byref(self.cfg),
                                           ctypes.c_void_p(ws.data_ptr()),
                                           ws.numel() * ws.element_size(), _b._stream_handle(stream)))


def adamw_step(params, grads, exp_avgs, exp_avg_sqs, *, step, lr=1e-3, betas=(0.9, 0.999),
               eps=1e-8, weight_decay=0.01, grad_scale=1.0, param_outs=None, workspace=None,
               stream=None) -> None:
    """One AdamW step (the "adamw" route) over all given tensors in one launch.

    params, exp_avgs, exp_avg_sqs: fp32 GPU tensors updated in place; grads: bf16
    or fp32, read as grad_scale·grad; step ≥ 1 is the bias-correction step number;
    param_outs: optional bf16 tensors that receive the updated parameter.
    """
    AdamwStep(params, grads, exp_avgs, exp_avg_sqs, lr=lr, betas=betas, eps=eps,
              weight_decay=weight_decay, grad_scale=grad_scale, param_outs=param_outs,
              workspace=workspace)(step, stream)


def ns_batched(x, *, coeffs=QUINTIC, steps=HYPER["steps"], eps=HYPER["eps"], normalize=True,
               precision="bf16", out=None, workspace=None, stream=None):
    """Newton–Schulz alone on a 2-D matrix or a 3-D batch (per slice); returns fp32."""
    import torch
    _b._check_dev(x, "x")
    if x.dim() not in (2, 3):
        raise ValueError("x must be 2-D or 3-D")
    batch = 1 if x.dim() == 2 else x.shape[0]
    rows, cols = x.shape[-2], x.shape[-1]
    if out is None:
        out = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    _b._check_dev(out, "out", torch.float32)
    if out.shape != x.shape:
        raise ValueError("out must have x's shape")
    if precision not in _b.PREC:
        raise ValueError(f"precision must be one of {sorted(_b.PREC)}")
    L = _b.lib()
    need = ctypes.c_size_t(0)
    _b.check(L.dmuon_ns_batched_workspace_size(batch, rows, cols, _b.PREC[precision], int(steps),
                                               ctypes.byref(need)))
    if workspace is None:
        workspace = _b.alloc_workspace(need.value, x.device)
    a, b, c = coeffs
    _b.check(L.dmuon_ns_batched(ctypes.c_void_p(x.data_ptr()), _b._dtype_code(x),
                                ctypes.c_void_p(out.data_ptr()), batch, rows, cols, a, b, c,
                                int(steps), eps, 1 if normalize else 0, _b.PREC[precision],
                                ctypes.c_void_p(workspace.data_ptr()),
                                workspace.numel() * workspace.element_size(),
                                _b._stream_handle(stream)))
    return out


def gemm_nt(A, B, K=None, stream=None):
    """C = A·Bᵀ (fp32) on the step's matrix-core contraction kernel (test hook).

    A: M×lda, B: N×ldb (bf16 or fp32, same dtype, ld multiples of 64); only the
    first K columns are meant, the rest must be zero.
    """
    import torch
    _b._check_dev(A, "A")
    _b._check_dev(B, "B")
    if A.dtype != B.dtype:
        raise ValueError("A and B must share a dtype")
    M, lda = A.shape
    N, ldb = B.shape
    K = lda if K is None else K
    C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    _b.check(_b.lib().dmuon_gemm_nt(ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(B.data_ptr()),
                                    ctypes.c_void_p(C.data_ptr()), M, N, K, lda, ldb, N,
                                    _b._dtype_code(A), _b._stream_handle(stream)))
    return C


def lpt_assign(rows, cols, batch, layer_id, n_slots, *, merge_below_elems=0, cost_kind=0,
               owner_slot=0):
    """Global LPT partition (host only, synchronous); see ``dmuon_lpt_assign``."""
    return _b.lpt_assign_np(rows, cols, batch, layer_id, n_slots, merge_below_elems, cost_kind,
                            owner_slot)


def phase_timing(enable: bool) -> None:
    _b.check(_b.lib().dmuon_phase_timing(1 if enable else 0))


def phase_timing_read():
    """{phase: (ms_total, launches)} of the launches since the last read."""
    import numpy as np
    n = len(_b.PHASES)
    ms = np.zeros(n, dtype=np.float64)
    cnt = np.zeros(n, dtype=np.int64)
    _b.check(_b.lib().dmuon_phase_timing_read(ms.ctypes.data_as(ctypes.c_void_p),
                                              cnt.ctypes.data_as(ctypes.c_void_p), n))
    return {name: (float(ms[i]), int(cnt[i])) for i, name in enumerate(_b.PHASES)}
