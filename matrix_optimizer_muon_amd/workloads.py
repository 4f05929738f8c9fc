"""Seeded synthetic inputs for the owner-rank Muon step.

This module is the ONLY code shared by the HIP path's tests/bench and the CPU
oracle: it draws gradients, momentum buffers and master weights and holds none
of the method's arithmetic (no momentum, no normalisation, no Newton–Schulz, no
update, no partitioning).  It imports numpy only.

Recipe (every array is reproducible from its seed on any machine):
* seed of one array = ``numpy.random.default_rng([workload_id, tensor_index, role])``
  with role 0 = gradient, 1 = master weight, 2 = left factor U, 3 = right factor V,
  4 = momentum (only when a test asks for a non-zero start);
* Gaussian gradients are drawn in fp32 (``standard_normal(dtype=float32)``) and
  scaled; bf16 gradients are those fp32 values rounded to bf16 with
  round-to-nearest-even and are handed over as their 16-bit patterns;
* decaying-spectrum gradients are U·diag(1/i)·Vᵀ with U, V Haar-random
  (QR of a Gaussian with the signs of R's diagonal folded into Q), in fp64,
  then cast to fp32;
* master weights are N(0, 0.02²) in fp32; momentum starts at zero.

Workloads (shapes are rows × cols of each gradient matrix):
* ``single_256x512``: one fp32 gradient 256×512, N(0, 1).
* ``layer_d2048``: one transformer layer at d = 2048: q, k, v, o 2048×2048,
  gate, up 5632×2048, down 2048×5632; bf16 N(0, 1e-3²).
* ``llama_d4096``: 32 layers × (q, k, v, o 4096×4096, gate, up 11008×4096,
  down 4096×11008) = 224 bf16 N(0, 1e-3²) matrices in registration order; the
  stepped workload is the share of one owner slot (chosen by the caller's
  partition).
* ``merged_small``: 256 matrices 512×512 and 128 matrices 256×1024, fp32 with a
  decaying spectrum.
* ``mlp_moe_large``: 4 matrices 8192×28672 and one expert tensor
  [64, 1408, 2048]; bf16 N(0, 1e-3²).

Inputs of the ``adamw`` route (1-D parameters; role 0 = gradient, 1 = parameter,
4 = first moment, 5 = second moment):
* ``adamw_llama_norms``: the 65 RMSNorm weight vectors of the 32-layer d = 4096
  model (two per layer and the final norm), 4096 elements each, bf16
  N(0, 1e-3²) gradients, parameters 1 + N(0, 0.02²);
* ``adamw_stream``: 16 vectors of 4 Mi elements with the same draws, a size at
  which the step is bound by HBM bandwidth.
The optimizer state is drawn as m ~ N(0, 1e-4²) and v = (N(0, 1e-3²))² (a
valid, non-negative second moment), or zero for a fresh state.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# Hyper-parameters shared by every workload.  lr = 0.02 and momentum = 0.95 are
# the optimizer settings of the DMuon HSDP guide's setup example; weight decay,
# eps, the quintic coefficients and k = 5 are the settings the workloads are
# defined with (the pages give the NS map without coefficients).
HYPER = dict(lr=0.02, mu=0.95, wd=0.01, eps=1e-7, a=3.4445, b=-4.7750, c=2.0315, steps=5)

WORKLOAD_IDS = {
    "single_256x512": 0,
    "layer_d2048": 1,
    "llama_d4096": 2,
    "merged_small": 3,
    "mlp_moe_large": 4,
    "adamw_llama_norms": 5,
    "adamw_stream": 6,
}


@dataclass
class TensorSpec:
    """One parameter of a workload: its shape, gradient dtype and generator."""
    index: int                 # tensor index inside the workload (seed component)
    name: str
    shape: tuple               # (rows, cols) or (batch, rows, cols)
    grad_dtype: str            # "bf16" or "f32"
    kind: str = "gauss"        # "gauss" or "decay"
    scale: float = 1.0         # std of a Gaussian gradient
    layer: int = -1            # transformer layer id (-1: none)


@dataclass
class Workload:
    name: str
    wid: int
    tensors: list = field(default_factory=list)


def _layer_d(d_model, d_ff, layers, wid, name, scale):
    wl = Workload(name, wid)
    idx = 0
    for lay in range(layers):
        for proj, shape in (("q", (d_model, d_model)), ("k", (d_model, d_model)),
                            ("v", (d_model, d_model)), ("o", (d_model, d_model)),
                            ("gate", (d_ff, d_model)), ("up", (d_ff, d_model)),
                            ("down", (d_model, d_ff))):
            nm = f"layers.{lay}.{proj}" if layers > 1 else proj
            wl.tensors.append(TensorSpec(idx, nm, shape, "bf16", "gauss", scale, lay))
            idx += 1
    return wl


def workload(name: str) -> Workload:
    """The tensor list of a named workload (shapes only, no data)."""
    wid = WORKLOAD_IDS[name]
    if name == "single_256x512":
        return Workload(name, wid, [TensorSpec(0, "w", (256, 512), "f32", "gauss", 1.0)])
    if name == "layer_d2048":
        return _layer_d(2048, 5632, 1, wid, name, 1e-3)
    if name == "llama_d4096":
        return _layer_d(4096, 11008, 32, wid, name, 1e-3)
    if name == "merged_small":
        wl = Workload(name, wid)
        for i in range(256):
            wl.tensors.append(TensorSpec(i, f"small.{i}", (512, 512), "f32", "decay", 1.0, 0))
        for i in range(128):
            wl.tensors.append(TensorSpec(256 + i, f"small.{256 + i}", (256, 1024), "f32",
                                         "decay", 1.0, 0))
        return wl
    if name == "mlp_moe_large":
        wl = Workload(name, wid)
        for i in range(4):
            wl.tensors.append(TensorSpec(i, f"mlp.{i}", (8192, 28672), "bf16", "gauss", 1e-3))
        wl.tensors.append(TensorSpec(4, "experts", (64, 1408, 2048), "bf16", "gauss", 1e-3))
        return wl
    if name == "adamw_llama_norms":
        wl = Workload(name, wid)
        names = [f"layers.{lay}.{n}" for lay in range(32) for n in ("input_norm", "post_attn_norm")]
        for i, nm in enumerate(names + ["final_norm"]):
            wl.tensors.append(TensorSpec(i, nm, (4096,), "bf16", "norm", 1e-3, i // 2))
        return wl
    if name == "adamw_stream":
        wl = Workload(name, wid)
        for i in range(16):
            wl.tensors.append(TensorSpec(i, f"vec.{i}", (4 << 20,), "bf16", "norm", 1e-3))
        return wl
    raise KeyError(name)


def rng_for(wid: int, index: int, role: int) -> np.random.Generator:
    return np.random.default_rng([wid, index, role])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even) and return the uint16 patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    rounded = (u + (0x7FFF + ((u >> 16) & 1))) >> 16
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def haar(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    """n×k matrix with orthonormal columns, Haar-distributed (QR with sign fix), fp64."""
    z = rng.standard_normal((n, k))
    q, r = np.linalg.qr(z)
    return q * np.sign(np.diag(r))[None, :]


def gaussian(shape, scale, rng) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)


def decaying_spectrum(rows, cols, wid, index) -> np.ndarray:
    """fp32 U·diag(1/i)·Vᵀ, i = 1..min(rows, cols), U and V Haar-random from seeds."""
    k = min(rows, cols)
    U = haar(rng_for(wid, index, 2), rows, k)
    V = haar(rng_for(wid, index, 3), cols, k)
    s = 1.0 / np.arange(1, k + 1, dtype=np.float64)
    return ((U * s[None, :]) @ V.T).astype(np.float32)


@dataclass
class TensorData:
    """Host arrays of one tensor.

    ``grad`` is fp32 holding exactly the values the GPU sees; for bf16 gradients
    ``grad_bits`` holds the 16-bit patterns (``grad`` is their exact widening).
    """
    spec: TensorSpec
    grad: np.ndarray
    grad_bits: np.ndarray | None
    momentum: np.ndarray
    master: np.ndarray


def make_tensor(wl: Workload, spec: TensorSpec, nonzero_momentum=False) -> TensorData:
    shape = spec.shape
    if spec.kind == "decay":
        lead = shape[:-2]
        rows, cols = shape[-2:]
        if lead:
            raise ValueError("decaying-spectrum tensors are 2-D")
        g = decaying_spectrum(rows, cols, wl.wid, spec.index)
    else:
        g = gaussian(shape, spec.scale, rng_for(wl.wid, spec.index, 0))
    bits = None
    if spec.grad_dtype == "bf16":
        bits = f32_to_bf16_bits(g)
        g = bf16_bits_to_f32(bits)
    w = gaussian(shape, 0.02, rng_for(wl.wid, spec.index, 1))
    if nonzero_momentum:
        m = gaussian(shape, max(spec.scale, 1e-3) if spec.kind == "gauss" else 0.01,
                     rng_for(wl.wid, spec.index, 4))
    else:
        m = np.zeros(shape, dtype=np.float32)
    return TensorData(spec, g.reshape(shape), None if bits is None else bits.reshape(shape),
                      m, w)


def make_custom(shape, grad_dtype="f32", seed=(99, 0), scale=1.0, nonzero_momentum=True,
                kind="gauss") -> TensorData:
    """A single tensor of any shape for parity tests (seeded by ``seed``)."""
    spec = TensorSpec(seed[1], "custom", tuple(shape), grad_dtype, kind, scale)
    wl = Workload("custom", seed[0], [spec])
    return make_tensor(wl, spec, nonzero_momentum=nonzero_momentum)


@dataclass
class AdamwData:
    """Host arrays of one ``adamw``-route parameter (fp32; bf16 gradients as in TensorData)."""
    spec: TensorSpec
    grad: np.ndarray
    grad_bits: np.ndarray | None
    param: np.ndarray
    exp_avg: np.ndarray
    exp_avg_sq: np.ndarray


def make_adamw(wl: Workload, spec: TensorSpec, fresh_state=False) -> AdamwData:
    shape = spec.shape
    g = gaussian(shape, spec.scale, rng_for(wl.wid, spec.index, 0))
    bits = None
    if spec.grad_dtype == "bf16":
        bits = f32_to_bf16_bits(g)
        g = bf16_bits_to_f32(bits).reshape(shape)
    p = gaussian(shape, 0.02, rng_for(wl.wid, spec.index, 1))
    if spec.kind == "norm":
        p = p + np.float32(1.0)
    if fresh_state:
        m = np.zeros(shape, dtype=np.float32)
        v = np.zeros(shape, dtype=np.float32)
    else:
        m = gaussian(shape, 1e-4, rng_for(wl.wid, spec.index, 4))
        r = gaussian(shape, 1e-3, rng_for(wl.wid, spec.index, 5))
        v = r * r
    return AdamwData(spec, g, None if bits is None else bits.reshape(shape), p, m, v)


def make_adamw_custom(numel, grad_dtype="f32", seed=(98, 0), scale=1e-3, fresh_state=False) -> AdamwData:
    """A single ``adamw``-route parameter of ``numel`` elements for parity tests."""
    spec = TensorSpec(seed[1], "custom", (int(numel),), grad_dtype, "norm", scale)
    return make_adamw(Workload("custom", seed[0], [spec]), spec, fresh_state=fresh_state)
