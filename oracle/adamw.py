"""fp64 CPU oracle of the ``adamw`` route step.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this module.  It shares no code with the HIP
path.

What it follows
---------------
* "Pure DMuon 路由" (routing) page, route table: the ``adamw`` route runs AdamW
  on the owner for LayerNorm weights, biases and other small parameters, which
  the owner then broadcasts; the dtype paragraph puts master and optimizer
  arithmetic in fp32 (this oracle uses fp64).
* MindSpore parameter-grouping page, §1 and §2.1: 1-D parameters cannot take
  the Muon update and go to an elementwise optimizer such as AdamW.
* The pages do not restate AdamW.  Its steps are taken from the algorithm's
  published definition (Loshchilov & Hutter, "Decoupled Weight Decay
  Regularization", the AdamW algorithm), in the order PyTorch's ``AdamW``
  applies them: decoupled decay of the parameter by lr·wd, first and second
  moment updates, bias correction by 1 − β₁ᵗ and 1 − β₂ᵗ, and the step
  lr·m̂ / (√v̂ + eps).  Hyper-parameters are inputs; the pages give none
  (defaults used by the tests: β₁ 0.9, β₂ 0.999, eps 1e-8).
* The gradient-ingest scale s multiplies the gradient before anything else
  (the same reading as for the Muon route).
"""
from __future__ import annotations

import numpy as np


def adamw_step(p, g, m, v, *, lr, beta1, beta2, eps, wd, step, grad_scale=1.0):
    """One AdamW step at step number ``step`` (≥ 1); returns (p, m, v) in fp64."""
    if step < 1:
        raise ValueError("step counts from 1")
    p = np.asarray(p, dtype=np.float64)
    g = grad_scale * np.asarray(g, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    # decoupled weight decay on the parameter
    p = p * (1.0 - lr * wd)
    # moment estimates
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    # bias-corrected estimates and the step
    m_hat = m / (1.0 - beta1 ** step)
    v_hat = v / (1.0 - beta2 ** step)
    p = p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p, m, v
