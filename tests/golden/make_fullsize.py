"""Writes oracle reference data of the two largest workloads for the full-size GPU tests.

The fp64 oracle needs minutes per 4096-wide matrix and several minutes per
8192×28672 matrix, too long inside a GPU test, so this script runs it once on
the CPU and stores, for every stepped 2-D slice (each expert of a 3-D tensor is
its own slice, as the parameter-grouping page's last-two-dims rule makes it):

* tile samples: SAMPLES seeded positions inside EVERY 256×256 tile of the slice
  (storage layout, tiles in row-major order of the tile grid, the last row and
  column of tiles clipped to the slice), stored as uint8 offsets inside the
  tile, and the oracle's Newton–Schulz output O at them (float32);
* tile norms: ‖O_tile‖_F of every tile (float64);
* sketches: O·r (one value per row) and sᵀ·O (one per column) for seeded
  Gaussian vectors r (length cols) and s (length rows), float64 arithmetic,
  stored as float32; a wrong row or column of O changes its sketch entry;
* ‖O‖_F of the slice.

It calls only ``oracle/`` plus the seeded input generators (which hold no
arithmetic of the method); ``sketch_vectors`` and ``tile_positions`` below only
draw random numbers.  Run from the repository root:

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

from matrix_optimizer_muon_amd.workloads import HYPER, make_tensor, workload  # noqa: E402

SAMPLES = 16        # positions per 256×256 tile
TILE = 256


def stepped_tensors(name, lpt):
    """The stepped tensors of a workload: one owner slot's LPT share of the 224
    Llama matrices (``lpt`` is the partition function to use), else all."""
    wl = workload(name)
    if name == "llama_d4096":
        rows = [t.shape[0] for t in wl.tensors]
        cols = [t.shape[1] for t in wl.tensors]
        res = lpt(rows, cols, [1] * len(rows), [t.layer for t in wl.tensors], 8, owner_slot=0)
        return wl, [wl.tensors[int(i)] for i in res["owner_order"]]
    return wl, list(wl.tensors)


def tile_grid(rows, cols):
    return -(-rows // TILE), -(-cols // TILE)


def tile_positions(tensor_index, slice_index, rows, cols):
    """uint8 (n_tiles, SAMPLES) row and column offsets inside every tile."""
    tr, tc = tile_grid(rows, cols)
    rng = np.random.default_rng([77, tensor_index, slice_index])
    u = rng.random((tr * tc, SAMPLES, 2))
    ti = np.repeat(np.arange(tr), tc)
    tj = np.tile(np.arange(tc), tr)
    hr = np.minimum(TILE, rows - ti * TILE)[:, None]
    hc = np.minimum(TILE, cols - tj * TILE)[:, None]
    lr = np.floor(u[:, :, 0] * hr).astype(np.uint8)
    lc = np.floor(u[:, :, 1] * hc).astype(np.uint8)
    return lr, lc


def global_positions(rows, cols, lr, lc):
    """Slice-global (row, col) int64 arrays of the tile samples."""
    tr, tc = tile_grid(rows, cols)
    ti = np.repeat(np.arange(tr), tc)[:, None]
    tj = np.tile(np.arange(tc), tr)[:, None]
    return ti * TILE + lr.astype(np.int64), tj * TILE + lc.astype(np.int64)


def sketch_vectors(tensor_index, slice_index, rows, cols):
    """Seeded Gaussian r (cols) and s (rows), float64."""
    rng = np.random.default_rng([78, tensor_index, slice_index])
    return rng.standard_normal(cols), rng.standard_normal(rows)


def tile_norms(O):
    rows, cols = O.shape
    tr, tc = tile_grid(rows, cols)
    P = np.zeros((tr * TILE, tc * TILE))
    P[:rows, :cols] = O
    return np.sqrt((P.reshape(tr, TILE, tc, TILE) ** 2).sum(axis=(1, 3))).reshape(-1)


def main(name):
    import oracle
    wl, ts = stepped_tensors(name, oracle.lpt_assign)
    keys = ("slice_tensor", "slice_batch", "slice_rows", "slice_cols", "O_norm")
    meta = {k: [] for k in keys}
    samp_r, samp_c, samp_O, tnorm, sk_or, sk_so = [], [], [], [], [], []
    t0 = time.time()
    for spec in ts:
        td = make_tensor(wl, spec)
        _, O, _ = oracle.muon_step(td.grad, td.momentum, td.master, lr=HYPER["lr"], mu=HYPER["mu"],
                                   wd=HYPER["wd"], eps=HYPER["eps"], a=HYPER["a"], b=HYPER["b"],
                                   c=HYPER["c"], steps=HYPER["steps"])
        slices = O.reshape((-1,) + O.shape[-2:])
        for b, Ob in enumerate(slices):
            rows, cols = Ob.shape
            lr, lc = tile_positions(spec.index, b, rows, cols)
            gr, gc = global_positions(rows, cols, lr, lc)
            r, s = sketch_vectors(spec.index, b, rows, cols)
            meta["slice_tensor"].append(spec.index)
            meta["slice_batch"].append(b)
            meta["slice_rows"].append(rows)
            meta["slice_cols"].append(cols)
            meta["O_norm"].append(float(np.sqrt(np.sum(Ob * Ob))))
            samp_r.append(lr)
            samp_c.append(lc)
            samp_O.append(Ob[gr, gc].astype(np.float32))
            tnorm.append(tile_norms(Ob))
            sk_or.append((Ob @ r).astype(np.float32))
            sk_so.append((s @ Ob).astype(np.float32))
        print(f"{spec.name} {spec.shape}: done at {time.time() - t0:.0f} s", flush=True)
        del td, O, slices
    n_tiles = [len(x) for x in tnorm]
    out = {k: np.array(v) for k, v in meta.items()}
    out["tensor_index"] = np.array([t.index for t in ts], dtype=np.int64)
    out["tile_off"] = np.concatenate([[0], np.cumsum(n_tiles)]).astype(np.int64)
    out["row_off"] = np.concatenate([[0], np.cumsum(meta["slice_rows"])]).astype(np.int64)
    out["col_off"] = np.concatenate([[0], np.cumsum(meta["slice_cols"])]).astype(np.int64)
    out["samp_r"] = np.concatenate(samp_r)
    out["samp_c"] = np.concatenate(samp_c)
    out["samp_O"] = np.concatenate(samp_O)
    out["tile_norm"] = np.concatenate(tnorm)
    out["sketch_Or"] = np.concatenate(sk_or)
    out["sketch_sO"] = np.concatenate(sk_so)
    out["samples_per_tile"] = np.array(SAMPLES)
    np.savez_compressed(os.path.join(HERE, f"fullsize_{name}.npz"), **out)
    print("wrote", name, f"({len(meta['O_norm'])} slices, {out['tile_off'][-1]} tiles)")


if __name__ == "__main__":
    main(sys.argv[1])
