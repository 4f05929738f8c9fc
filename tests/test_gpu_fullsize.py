"""Full-size parity of the two largest workloads (needs an MI355X).

The fp64 oracle cannot step these workloads inside a test (minutes per matrix),
so ``tests/golden/make_fullsize.py`` ran it once on the CPU and stored, for
every stepped 2-D slice (each expert of the 3-D tensor is a slice): 16 seeded
samples of O inside every 256×256 tile, ‖O_tile‖_F of every tile, the
sketches O·r and sᵀ·O for seeded Gaussian r, s, and ‖O‖_F.  The GPU runs the
whole workload in one call, in the launch configuration ``bench.py`` times, on
the bf16 matrix-core path and on the fp32 path, and is compared per slice:

* every tile: the relative error over its 16 samples ≤ TILE_SAMPLES[prec] (a
  tile holding another tile's values, zeros or garbage is off by ~1), and its
  norm within TOL[prec] of the oracle's;
* every row and every column: the sketch entry within SKETCH_ENTRY[prec] of
  the sketch's RMS (a wrong row or column moves its entry);
* the whole slice: relative error of the two sketches, of all its samples and
  of ‖O‖_F ≤ TOL[prec] (2e-2 on the bf16 path, 1e-4 on the fp32 path);
* momentum (zero start): B' equals G exactly, every element;
* update: W' against (1 − lr·wd)·W − lr·O_gpu in fp64, every element, ≤ 1e-6.
"""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import matrix_optimizer_muon_amd as mm  # noqa: E402
from matrix_optimizer_muon_amd.workloads import HYPER, make_tensor  # noqa: E402

from golden.make_fullsize import TILE, global_positions, sketch_vectors, stepped_tensors  # noqa: E402

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

TOL = {"bf16": 2e-2, "f32": 1e-4}
TILE_SAMPLES = {"bf16": 0.1, "f32": 1e-3}
SKETCH_ENTRY = {"bf16": 0.1, "f32": 1e-3}

_cache = {}


def device_inputs(name):
    """Gradients and initial masters of the stepped tensors, on the GPU (kept
    for the second precision)."""
    if name in _cache:
        return _cache[name]
    _cache.clear()
    wl, ts = stepped_tensors(name, mm.lpt_assign)
    grads, masters = [], []
    for spec in ts:
        td = make_tensor(wl, spec)
        if td.grad_bits is not None:
            grads.append(torch.from_numpy(td.grad_bits.view(np.int16)).view(torch.bfloat16).cuda())
        else:
            grads.append(torch.from_numpy(td.grad).cuda())
        masters.append(torch.from_numpy(td.master).cuda())
        del td
    _cache[name] = (ts, grads, masters)
    return _cache[name]


def rel(x, y):
    return float(np.linalg.norm(x - y) / np.linalg.norm(y))


def check_slice(o, gold, k, prec):
    """Compare one slice's GPU output o (rows×cols fp32, on the GPU) with the
    stored oracle data of slice k; returns the slice's worst relative error."""
    rows, cols = int(gold["slice_rows"][k]), int(gold["slice_cols"][k])
    ti, tn = gold["tile_off"][k], gold["tile_off"][k + 1]
    lr, lc = gold["samp_r"][ti:tn], gold["samp_c"][ti:tn]
    gr, gc = global_positions(rows, cols, lr, lc)
    vals = o[torch.from_numpy(gr).cuda(), torch.from_numpy(gc).cuda()].double().cpu().numpy()
    ref = gold["samp_O"][ti:tn].astype(np.float64)
    tile_err = np.linalg.norm(vals - ref, axis=1) / np.linalg.norm(ref, axis=1)
    bad = np.nonzero(tile_err > TILE_SAMPLES[prec])[0]
    assert bad.size == 0, f"slice {k}: tiles {bad[:10].tolist()} off by {tile_err[bad[:10]].tolist()}"
    e_samples = rel(vals, ref)
    # tile norms
    tr, tc = -(-rows // TILE), -(-cols // TILE)
    pad = torch.zeros((tr * TILE, tc * TILE), dtype=torch.float64, device=o.device)
    pad[:rows, :cols] = o.double()
    norms = pad.view(tr, TILE, tc, TILE).pow(2).sum(dim=(1, 3)).sqrt().reshape(-1).cpu().numpy()
    tref = gold["tile_norm"][ti:tn]
    norm_err = np.abs(norms - tref) / tref
    assert norm_err.max() <= TOL[prec], (k, int(norm_err.argmax()), float(norm_err.max()))
    # sketches: one entry per row (O·r) and per column (sᵀ·O)
    r, s = sketch_vectors(int(gold["slice_tensor"][k]), int(gold["slice_batch"][k]), rows, cols)
    od = o.double()
    o_r = (od @ torch.from_numpy(r).cuda()).cpu().numpy()
    s_o = (torch.from_numpy(s).cuda() @ od).cpu().numpy()
    errs = [e_samples]
    for got, key, off in ((o_r, "sketch_Or", "row_off"), (s_o, "sketch_sO", "col_off")):
        a, b = gold[off][k], gold[off][k + 1]
        want = gold[key][a:b].astype(np.float64)
        rms = np.sqrt(np.mean(want * want))
        entry = np.abs(got - want) / rms
        assert entry.max() <= SKETCH_ENTRY[prec], (k, key, int(entry.argmax()), float(entry.max()))
        errs.append(rel(got, want))
    e_norm = abs(float(torch.linalg.vector_norm(od)) - gold["O_norm"][k]) / gold["O_norm"][k]
    errs.append(e_norm)
    assert max(errs) <= TOL[prec], (k, errs)
    return max(errs)


@pytest.mark.parametrize("precision", ["bf16", "f32"])
@pytest.mark.parametrize("name", ["llama_d4096", "mlp_moe_large"])
def test_fullsize_parity(name, precision):
    path = os.path.join(GOLDEN, f"fullsize_{name}.npz")
    gold = dict(np.load(path))
    assert int(gold["samples_per_tile"]) == 16
    ts, grads, masters0 = device_inputs(name)
    assert [t.index for t in ts] == gold["tensor_index"].tolist()
    moms = [torch.zeros(g.shape, dtype=torch.float32, device="cuda") for g in grads]
    masters = [w.clone() for w in masters0]
    outs = [torch.empty(g.shape, dtype=torch.float32, device="cuda") for g in grads]
    print(f"{name} {precision}: {len(ts)} tensors on the GPU, stepping", flush=True)
    mm.muon_step(grads, moms, masters, ns_outs=outs, precision=precision)
    torch.cuda.synchronize()
    lr, wd = HYPER["lr"], HYPER["wd"]
    k = 0
    worst = 0.0
    for spec, g, m, w0, w, o in zip(ts, grads, moms, masters0, masters, outs):
        assert torch.equal(m, g.float()), spec.name
        w_ref = (1 - lr * wd) * w0.double() - lr * o.double()
        e_w = float(torch.linalg.vector_norm(w.double() - w_ref) / torch.linalg.vector_norm(w_ref))
        assert e_w <= 1e-6, (spec.name, e_w)
        for b in range(o.shape[0] if o.dim() == 3 else 1):
            assert int(gold["slice_tensor"][k]) == spec.index and int(gold["slice_batch"][k]) == b
            worst = max(worst, check_slice(o[b] if o.dim() == 3 else o, gold, k, precision))
            k += 1
    assert k == len(gold["O_norm"])
    print(f"{name} {precision}: {k} slices, {int(gold['tile_off'][-1])} tiles checked; "
          f"worst slice error {worst:.2e}", flush=True)
    del moms, masters, outs
    torch.cuda.empty_cache()
