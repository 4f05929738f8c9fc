"""Writes sampled oracle outputs of the two largest workloads for the full-size GPU tests.

The fp64 oracle needs minutes per 4096-wide matrix and about three minutes per
8192×28672 matrix, too long inside a GPU test, so this script runs it once on
the CPU and stores, per stepped tensor: 256 sampled positions (seeded), the
oracle's Newton–Schulz output O and updated master W at those positions, and
‖O‖_F.  It calls only ``oracle/`` plus the seeded input generators (which hold
no arithmetic of the method).  Run from the repository root:

    python tests/golden/make_fullsize.py llama_d4096
    python tests/golden/make_fullsize.py mlp_moe_large
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from matrix_optimizer_muon_amd.workloads import HYPER, make_tensor, workload  # noqa: E402

SAMPLES = 256


def stepped_tensors(name):
    wl = workload(name)
    if name == "llama_d4096":
        rows = [t.shape[0] for t in wl.tensors]
        cols = [t.shape[1] for t in wl.tensors]
        res = oracle.lpt_assign(rows, cols, [1] * len(rows), [t.layer for t in wl.tensors], 8,
                                owner_slot=0)
        return wl, [wl.tensors[i] for i in res["owner_order"]]
    return wl, list(wl.tensors)


def sample_positions(spec):
    """(SAMPLES, 3) positions (batch, row, col); batch is 0 for a 2-D tensor."""
    rng = np.random.default_rng([77, spec.index])
    shape = spec.shape if len(spec.shape) == 3 else (1,) + tuple(spec.shape)
    return np.stack([rng.integers(0, d, SAMPLES) for d in shape], axis=1).astype(np.int64)


def main(name):
    wl, ts = stepped_tensors(name)
    out = {"tensor_index": [], "positions": [], "O": [], "W": [], "O_norm": []}
    t0 = time.time()
    for spec in ts:
        td = make_tensor(wl, spec)
        B, O, W = oracle.muon_step(td.grad, td.momentum, td.master, lr=HYPER["lr"], mu=HYPER["mu"],
                                   wd=HYPER["wd"], eps=HYPER["eps"], a=HYPER["a"], b=HYPER["b"],
                                   c=HYPER["c"], steps=HYPER["steps"])
        pos = sample_positions(spec)
        idx = tuple(pos[:, k] for k in range(3)) if len(spec.shape) == 3 else (pos[:, 1], pos[:, 2])
        out["tensor_index"].append(spec.index)
        out["positions"].append(pos)
        out["O"].append(O[idx])
        out["W"].append(W[idx])
        out["O_norm"].append(float(np.linalg.norm(O)))
        print(f"{spec.name} {spec.shape}: done at {time.time() - t0:.0f} s", flush=True)
        del td, B, O, W
    np.savez_compressed(os.path.join(HERE, f"fullsize_{name}.npz"),
                        tensor_index=np.array(out["tensor_index"], dtype=np.int64),
                        positions=np.stack(out["positions"]),
                        O=np.stack(out["O"]), W=np.stack(out["W"]),
                        O_norm=np.array(out["O_norm"]))
    print("wrote", name)


if __name__ == "__main__":
    main(sys.argv[1])
