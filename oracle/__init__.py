"""Plain, slow fp64 CPU oracle for the owner-rank optimizer step (test infrastructure).

This package is TEST INFRASTRUCTURE ONLY.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The HIP product path (``matrix_optimizer_muon_amd``) never imports
it and shares no code with it: the two meet only through the seeded input
generators in ``matrix_optimizer_muon_amd.workloads``, which hold none of the
method's arithmetic.

Every function cites the passage of the DMuon pages (or of the MindSpore
parameter-grouping design page) that it follows.  Where the pages are silent
the reading taken is stated in the docstring.
"""
from .muon import (  # noqa: F401
    momentum_update,
    frobenius_normalize,
    newton_schulz,
    newton_schulz_batched,
    decay_update,
    muon_step,
    validate_ndim,
    publish_bf16,
)
from .adamw import adamw_step  # noqa: F401
from .lpt import lpt_assign, per_layer_lpt  # noqa: F401
