"""fp64 CPU oracle of the owner-rank Muon step.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this module.  It shares no code with the HIP
path.

What it follows
---------------
* DMuon "架构设计" (Architecture design) page, §1 "矩阵优化器的原子性约束"
  (atomicity constraint of matrix optimizers): the Newton–Schulz (NS) map
  X_{t+1} = α X_t + β X_t X_tᵀ X_t + γ X_t (X_tᵀ X_t)², which needs the whole
  matrix at every iteration.
* Same page, §2 "专属归属权——原语" (dedicated ownership) and the "HSDP 训练"
  (HSDP training) page, section "底层发生了什么" (what happens underneath):
  only the owner runs NS + momentum + weight decay + parameter update, on its
  local full-precision copy, with no communication.
* "Pure DMuon 路由" (routing) page, dtype paragraph and the ``param_policy``
  example: master and optimizer arithmetic are fp32 (this oracle uses fp64).
* MindSpore "分布式 Muon 优化器 — 参数分组设计文档（v2）" (parameter grouping
  design) page, §2.1 (1-D tensors are rejected), §2.2 and §6 (tensors with more
  than two dims act on their last two dims), §4.1 (``_validate_param_ndim``
  raises ``ValueError`` for fewer than two dims).

Readings taken where the pages are silent
-----------------------------------------
* Momentum is plain heavy-ball B ← μB + G with no dampening and no Nesterov
  term; NS runs on the updated B.
* Normalisation is X₀ = B / (‖B‖_F + eps) per 2-D slice (per expert for 3-D
  tensors).
* A slice with rows > cols is transposed before NS and transposed back after;
  square slices are not transposed.  After that orientation (m ≤ n) the page's
  β X XᵀX + γ X (XᵀX)² is evaluated as (β A + γ A²) X with A = X Xᵀ, which is
  the same matrix by associativity ((X Xᵀ)² X = X (Xᵀ X)²); the test suite pins
  this against the literal form of the page.
* (α, β, γ) of the page are the quintic coefficients (a, b, c).
* Weight decay is decoupled and lr-scaled: W ← (1 − lr·wd)·W − lr·O, with O
  the NS output and no shape-dependent lr scale.
* Order: momentum, then NS, then decay + update.
"""
from __future__ import annotations

import numpy as np


def validate_ndim(shape) -> None:
    """Reject tensors with fewer than two dims.

    MindSpore parameter-grouping page, §2.1 (1-D parameters are not matrices and
    are refused) and §4.1 (``_validate_param_ndim`` raises ``ValueError``).
    """
    if len(shape) < 2:
        raise ValueError(f"Muon needs a tensor with >= 2 dims, got shape {tuple(shape)}")


def momentum_update(B, G, mu, grad_scale=1.0):
    """B ← μ·B + s·G in fp64.

    DMuon architecture page §2 (the owner's step includes momentum) and the HSDP
    guide ("what happens underneath": the owner holds the momentum buffer).  The
    heavy-ball form without dampening is the reading taken (the pages name only
    "momentum").

    s is the gradient-ingest scale.  The pages reduce gradients to the owner with
    an averaging reduce whose net divisor is the number of contributing ranks
    (HSDP guide, "两阶段梯度 Reduce" / two-stage gradient reduce); an owner that
    receives a summed buffer instead applies s = 1/N here.  s = 1 for an
    already-averaged gradient.
    """
    return mu * np.asarray(B, dtype=np.float64) + grad_scale * np.asarray(G, dtype=np.float64)


def frobenius_normalize(X, eps):
    """X / (‖X‖_F + eps), the norm taken in fp64 over the whole 2-D slice.

    Reading: the pages give the NS map but not its start; the plain Muon start
    X₀ = G/(‖G‖_F + eps) is used, with eps added to the norm (not a max).
    """
    X = np.asarray(X, dtype=np.float64)
    s = np.sqrt(np.sum(X * X))
    return X / (s + eps)


def newton_schulz(G, a, b, c, steps, eps, normalize=True):
    """k iterations of the quintic NS map on one 2-D matrix, in fp64.

    DMuon architecture page §1, the NS equation
    X_{t+1} = α X_t + β X_t X_tᵀ X_t + γ X_t (X_tᵀ X_t)², with (α, β, γ) = (a, b, c).

    Steps, in the page's order:
      1. orient: if rows > cols use Xᵀ (so the Gram matrix is m×m with m ≤ n);
      2. X₀ = X / (‖X‖_F + eps) when ``normalize`` (else X₀ = X);
      3. repeat ``steps`` times: A = X Xᵀ; X ← a·X + (b·A + c·A·A)·X;
      4. undo the orientation.
    """
    X = np.asarray(G, dtype=np.float64)
    if X.ndim != 2:
        raise ValueError("newton_schulz takes one 2-D matrix")
    transposed = X.shape[0] > X.shape[1]
    if transposed:
        X = X.T
    if normalize:
        X = frobenius_normalize(X, eps)
    for _ in range(steps):
        A = X @ X.T
        poly = b * A + c * (A @ A)
        X = a * X + poly @ X
    if transposed:
        X = X.T
    return np.ascontiguousarray(X)


def newton_schulz_batched(G, a, b, c, steps, eps, normalize=True):
    """NS on every 2-D slice over the last two dims of a 2-D or 3-D tensor.

    MindSpore parameter-grouping page §2.2 / §6: for an n-dim tensor the matrix
    is the last two dims {n−2, n−1}; leading dims index independent matrices
    (e.g. the experts of an MoE weight).  Each slice is normalised on its own.
    """
    G = np.asarray(G, dtype=np.float64)
    validate_ndim(G.shape)
    if G.ndim == 2:
        return newton_schulz(G, a, b, c, steps, eps, normalize)
    lead = G.shape[:-2]
    flat = G.reshape((-1,) + G.shape[-2:])
    out = np.empty_like(flat)
    for i in range(flat.shape[0]):
        out[i] = newton_schulz(flat[i], a, b, c, steps, eps, normalize)
    return out.reshape(lead + G.shape[-2:])


def decay_update(W, O, lr, wd):
    """W ← (1 − lr·wd)·W − lr·O in fp64.

    DMuon architecture page §2 and HSDP guide ("what happens underneath"): the
    owner's step applies weight decay and the parameter update to its
    full-precision copy.  Reading: decoupled decay scaled by lr (AdamW style).
    """
    W = np.asarray(W, dtype=np.float64)
    return (1.0 - lr * wd) * W - lr * np.asarray(O, dtype=np.float64)


def muon_step(G, B, W, *, lr, mu, wd, eps, a, b, c, steps, grad_scale=1.0):
    """One owner-rank Muon step on one tensor; returns (B_new, O, W_new) in fp64.

    Order: momentum → NS (per 2-D slice over the last two dims) → decay + update.
    DMuon architecture page §2 / §3.3 (owner-gated step) and HSDP guide
    ("what happens underneath", step 3).
    """
    validate_ndim(np.shape(G))
    if np.shape(G) != np.shape(B) or np.shape(G) != np.shape(W):
        raise ValueError("G, B and W must have the same shape")
    B_new = momentum_update(B, G, mu, grad_scale)
    O = newton_schulz_batched(B_new, a, b, c, steps, eps, normalize=True)
    W_new = decay_update(W, O, lr, wd)
    return B_new, O, W_new


def publish_bf16(W32):
    """bf16 bits (uint16) of fp32 values, rounded to nearest, ties to even.

    The publish step: after the update the owner broadcasts its parameter in
    ``param_dtype`` (bf16 in the pages' policy example), cast from the fp32
    master (routing page, dtype paragraph: ``param_dtype`` is the forward
    parameter / communication dtype, ``master_dtype`` the storage precision;
    architecture page §2: the owner broadcasts ``_owned_data`` before forward).

    Written from the definition of the format: bf16 keeps the upper 16 bits of
    the fp32 encoding; the discarded 16 bits round the kept part to nearest,
    and an exact half rounds to the even kept value.  NaN stays a (quiet) NaN.
    Overflow past the largest finite bf16 carries into the exponent and gives
    infinity, as rounding to nearest requires.
    """
    u = np.ascontiguousarray(W32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    upper = u >> 16
    lower = u & 0xFFFF
    half = 0x8000
    round_up = (lower > half) | ((lower == half) & ((upper & 1) == 1))
    out = (upper + round_up.astype(np.uint64)) & 0xFFFF
    is_nan = ((u >> 23) & 0xFF == 0xFF) & ((u & 0x7FFFFF) != 0)
    out = np.where(is_nan, upper | 0x40, out)
    return out.astype(np.uint16)
