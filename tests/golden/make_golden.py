"""Writes the stored expected values of tests/golden/ that the pages do not print.

Calls only ``oracle/`` (and the seeded shape list of the workloads, which holds no
arithmetic of the method).  Run from the repository root:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle import lpt_assign, newton_schulz  # noqa: E402
from matrix_optimizer_muon_amd.workloads import HYPER, workload  # noqa: E402


def quintic_rank1():
    # a unit rank-1 matrix with eps = 0 has one singular value 1, so its NS
    # output's nonzero entry is the k-fold scalar iterate p^k(1)
    G = np.zeros((3, 5)); G[1, 2] = 1.0
    vals = [float(newton_schulz(G, HYPER["a"], HYPER["b"], HYPER["c"], k, 0.0)[1, 2])
            for k in range(1, 6)]
    return {"note": "p^k(1) for the quintic (3.4445, -4.7750, 2.0315), k = 1..5, "
                    "written by tests/golden/make_golden.py from oracle.newton_schulz",
            "p_iterates_of_one": vals}


def llama_share():
    wl = workload("llama_d4096")
    rows = [t.shape[0] for t in wl.tensors]
    cols = [t.shape[1] for t in wl.tensors]
    res = lpt_assign(rows, cols, [1] * len(rows), [t.layer for t in wl.tensors], 8,
                     merge_below_elems=0, cost_kind=0, owner_slot=0)
    names = [wl.tensors[i].name for i in res["owner_order"]]
    return {"note": "global LPT of the 224 matrices of the 32-layer d=4096 model over 8 slots, "
                    "cost = numel, same-layer-distinct-slot rule; written by "
                    "tests/golden/make_golden.py from oracle.lpt_assign",
            "slot_of": res["slot_of"], "slot_load": res["slot_load"],
            "owner_slot": 0, "owner_order": res["owner_order"],
            "owner_names": names, "group_offsets": res["group_offsets"]}


if __name__ == "__main__":
    with open(os.path.join(HERE, "quintic_rank1.json"), "w") as f:
        json.dump(quintic_rank1(), f, indent=1)
    with open(os.path.join(HERE, "llama_d4096_slot0.json"), "w") as f:
        json.dump(llama_share(), f, indent=1)
    print("wrote golden files")
