"""matrix_optimizer_muon_amd — the owner-rank Muon optimizer step on MI355X.

Python face of libdmuon_ns (C ABI in ``include/dmuon_ns.h``).  The functions
below only marshal arguments: momentum, normalisation, Newton–Schulz and the
update all run in the library's HIP kernels, on the caller's current stream
unless a ``stream`` is given.

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


def muon_step_workspace_size(grads, momenta, masters, *, steps=5, precision="bf16",
                             ns_outs=None, stream_groups=0) -> int:
    cfg = _b.make_cfg(0.0, 0.0, 0.0, 0.0, QUINTIC, steps, precision, 1.0, stream_groups)
    descs = _b.make_descs(grads, momenta, masters, ns_outs)
    return _b.muon_step_workspace_size(cfg, descs)


class _Marshalled:
    """Descriptors, cfg, workspace and side streams of one tensor set."""

    def __init__(self, grads, momenta, masters, lr, momentum, weight_decay, eps, coeffs, steps,
                 precision, grad_scale, ns_outs, param_outs, workspace, stream_groups, stream):
        import torch
        self._tensors = (list(grads), list(momenta), list(masters), ns_outs, param_outs)
        self.cfg = _b.make_cfg(lr, momentum, weight_decay, eps, coeffs, steps, precision, grad_scale,
                               stream_groups)
        self.arr, self.n = _b.make_descs(grads, momenta, masters, ns_outs, param_outs)
        self.workspace = None
        self.side = []
        if self.n:
            need = _b.muon_step_workspace_size(self.cfg, (self.arr, self.n))
            groups = _b.muon_step_groups(self.cfg, (self.arr, self.n))
            dev = grads[0].device
            if workspace is None:
                workspace = _b.alloc_workspace(need, dev, stream)
            self.workspace = workspace
            # one caller-owned stream per extra group (default priority)
            self.side = [torch.cuda.Stream(device=dev) for _ in range(max(groups - 1, 0))]
            self.side_arr, self.n_side = _b.stream_array(self.side)
            _b.keep_until_done(workspace, self.side)

    def ws_args(self):
        ws = self.workspace
        return ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size()


class MuonStep:
    """A prepared owner-rank Muon step over a fixed set of tensors.

    The tensors are checked and marshalled once, and ``dmuon_muon_step_prepare``
    writes their tables into the workspace (the constructor waits for it); every
    call then enqueues one step (``dmuon_muon_step_run``, launches only) on
    ``stream``, which may be captured into a CUDA/HIP graph.  The tensors must
    stay alive and keep their storage; ``lr`` may be changed between calls.
    Extra stream groups run on side streams this object owns.  Arguments as for
    ``muon_step``; ``stream_groups`` fixes the group count (0: the library's).
    """

    def __init__(self, grads, momenta, masters, *, lr=HYPER["lr"], momentum=HYPER["mu"],
                 weight_decay=HYPER["wd"], eps=HYPER["eps"], coeffs=QUINTIC, steps=HYPER["steps"],
                 precision="bf16", grad_scale=1.0, ns_outs=None, param_outs=None, workspace=None,
                 stream_groups=0, stream=None):
        st = _b.resolve_stream(stream)
        self._m = _Marshalled(grads, momenta, masters, lr, momentum, weight_decay, eps, coeffs, steps,
                              precision, grad_scale, ns_outs, param_outs, workspace, stream_groups, st)
        self.cfg = self._m.cfg
        self.workspace = self._m.workspace
        self._seen = set()
        if self._m.n:
            ws, nbytes = self._m.ws_args()
            _b.check(_b.lib().dmuon_muon_step_prepare(self._m.arr, self._m.n, ctypes.byref(self.cfg),
                                                      ws, nbytes, ctypes.c_void_p(st.cuda_stream)))
            st.synchronize()       # the tables are in place before a run on any stream

    @property
    def groups(self):
        return len(self._m.side) + 1 if self._m.n else 0

    @property
    def lr(self):
        return self.cfg.lr

    @lr.setter
    def lr(self, value):
        self.cfg.lr = value

    def __call__(self, stream=None) -> None:
        if self._m.n == 0:
            return
        st = _b.resolve_stream(stream)
        if st.cuda_stream not in self._seen:
            _b.keep_until_done(self.workspace, [st])
            self._seen.add(st.cuda_stream)
        ws, nbytes = self._m.ws_args()
        _b.check(_b.lib().dmuon_muon_step_run(self._m.arr, self._m.n, ctypes.byref(self.cfg), ws, nbytes,
                                              ctypes.c_void_p(st.cuda_stream), self._m.side_arr,
                                              self._m.n_side))


def muon_step(grads, momenta, masters, *, lr=HYPER["lr"], momentum=HYPER["mu"],
              weight_decay=HYPER["wd"], eps=HYPER["eps"], coeffs=QUINTIC, steps=HYPER["steps"],
              precision="bf16", grad_scale=1.0, ns_outs=None, param_outs=None, workspace=None,
              stream_groups=0, stream=None) -> None:
    """One owner-rank Muon step over all given tensors, enqueued on ``stream``.

    grads: bf16/fp32 GPU tensors (2-D or 3-D), read as grad_scale·grad; momenta,
    masters: fp32, updated in place; ns_outs: optional fp32 tensors that receive
    the Newton–Schulz output; param_outs: optional bf16 tensors that receive the
    updated master rounded to bf16 (the published parameter).
    workspace: optional uint8 GPU tensor of at least ``muon_step_workspace_size``
    bytes (allocated here, on ``stream``, when omitted).  One call of
    ``dmuon_muon_step`` (tables and launches; no host synchronisation).
    """
    st = _b.resolve_stream(stream)
    m = _Marshalled(grads, momenta, masters, lr, momentum, weight_decay, eps, coeffs, steps,
                    precision, grad_scale, ns_outs, param_outs, workspace, stream_groups, st)
    if m.n == 0:
        return
    _b.keep_until_done(m.workspace, [st])
    ws, nbytes = m.ws_args()
    _b.check(_b.lib().dmuon_muon_step(m.arr, m.n, ctypes.byref(m.cfg), ws, nbytes,
                                      ctypes.c_void_p(st.cuda_stream), m.side_arr, m.n_side))


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
        self._seen = set()

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
        st = _b.resolve_stream(stream)
        if st.cuda_stream not in self._seen:
            _b.keep_until_done(ws, [st])
            self._seen.add(st.cuda_stream)
        _b.check(_b.lib().dmuon_adamw_step(self.arr, self.n, ctypes.byref(self.cfg),
                                           ctypes.c_void_p(ws.data_ptr()),
                                           ws.numel() * ws.element_size(), ctypes.c_void_p(st.cuda_stream)))


def adamw_step(params, grads, exp_avgs, exp_avg_sqs, *, step, lr=1e-3, betas=(0.9, 0.999),
               eps=1e-8, weight_decay=0.01, grad_scale=1.0, param_outs=None, workspace=None,
               stream=None) -> None:
    """One AdamW step (the "adamw" route) over all given tensors in one launch.

    params, exp_avgs, exp_avg_sqs: fp32 GPU tensors updated in place; grads: bf16
    or fp32, read as grad_scale·grad; step ≥ 1 is the bias-correction step number;
    param_outs: optional bf16 tensors that receive the updated parameter.
    """
    st = _b.resolve_stream(stream)
    if workspace is None and len(params):
        arr, n = _b.make_adamw_descs(params, grads, exp_avgs, exp_avg_sqs, param_outs)
        need = ctypes.c_size_t(0)
        _b.check(_b.lib().dmuon_adamw_step_workspace_size(arr, n, ctypes.byref(need)))
        workspace = _b.alloc_workspace(need.value, params[0].device, st)
    AdamwStep(params, grads, exp_avgs, exp_avg_sqs, lr=lr, betas=betas, eps=eps,
              weight_decay=weight_decay, grad_scale=grad_scale, param_outs=param_outs,
              workspace=workspace)(step, st)


def ns_batched(x, *, coeffs=QUINTIC, steps=HYPER["steps"], eps=HYPER["eps"], normalize=True,
               precision="bf16", out=None, workspace=None, stream=None):
    """Newton–Schulz alone on a 2-D matrix or a 3-D batch (per slice); returns fp32."""
    import torch
    _b._check_dev(x, "x")
    if x.dim() not in (2, 3):
        raise ValueError("x must be 2-D or 3-D")
    batch = 1 if x.dim() == 2 else x.shape[0]
    rows, cols = x.shape[-2], x.shape[-1]
    st = _b.resolve_stream(stream)
    if out is None:
        with torch.cuda.stream(st):
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
        workspace = _b.alloc_workspace(need.value, x.device, st)
    _b.keep_until_done(workspace, [st])
    a, b, c = coeffs
    _b.check(L.dmuon_ns_batched(ctypes.c_void_p(x.data_ptr()), _b._dtype_code(x),
                                ctypes.c_void_p(out.data_ptr()), batch, rows, cols, a, b, c,
                                int(steps), eps, 1 if normalize else 0, _b.PREC[precision],
                                ctypes.c_void_p(workspace.data_ptr()),
                                workspace.numel() * workspace.element_size(),
                                ctypes.c_void_p(st.cuda_stream)))
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
    st = _b.resolve_stream(stream)
    with torch.cuda.stream(st):
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    _b.check(_b.lib().dmuon_gemm_nt(ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(B.data_ptr()),
                                    ctypes.c_void_p(C.data_ptr()), M, N, K, lda, ldb, N,
                                    _b._dtype_code(A), ctypes.c_void_p(st.cuda_stream)))
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
