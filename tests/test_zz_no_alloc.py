"""The allocation-free step (dmuon_muon_step_noalloc) against the workspace step
(dmuon_muon_step), through the C ABI (needs an MI355X).

Two calls in a row share the GPU's static scratch, the second on a smaller
input; each must give the same bits as dmuon_muon_step on copies of the same
inputs, and stay within the oracle bounds (NS output ≤ 2e-2 on the bf16
path, ≤ 1e-4 on the fp32 path; momentum and update ≤ 1e-6).
"""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import matrix_optimizer_muon_amd as mm  # noqa: E402
from matrix_optimizer_muon_amd import _binding as B  # noqa: E402
from matrix_optimizer_muon_amd.workloads import HYPER, make_custom  # noqa: E402
import oracle  # noqa: E402

pytestmark = pytest.mark.gpu
Q5 = (HYPER["a"], HYPER["b"], HYPER["c"])
TOL = {"bf16": 2e-2, "f32": 1e-4}


def to_dev(td):
    if td.grad_bits is not None:
        g = torch.from_numpy(td.grad_bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    else:
        g = torch.from_numpy(td.grad.copy()).cuda()
    return (g, torch.from_numpy(td.momentum.copy()).cuda(), torch.from_numpy(td.master.copy()).cuda(),
            torch.empty(td.grad.shape, dtype=torch.float32, device="cuda"))


def rel(x, y):
    return float(np.linalg.norm(np.asarray(x, np.float64) - y) / np.linalg.norm(y))


@pytest.mark.parametrize("precision", ["bf16", "f32"])
def test_noalloc_matches_the_workspace_step(precision):
    first = [make_custom((600, 1000), "bf16", seed=(90, 0), scale=1e-3),
             make_custom((2, 520, 300), "f32", seed=(90, 1)),
             make_custom((257, 257), "f32", seed=(90, 2))]
    second = [make_custom((300, 200), "f32", seed=(90, 3))]          # smaller: the scratch keeps
    for tds in (first, second):                                      # the first call's contents
        ref = [to_dev(td) for td in tds]
        mm.muon_step([d[0] for d in ref], [d[1] for d in ref], [d[2] for d in ref],
                     ns_outs=[d[3] for d in ref], precision=precision)
        got = [to_dev(td) for td in tds]
        cfg = B.make_cfg(HYPER["lr"], HYPER["mu"], HYPER["wd"], HYPER["eps"], Q5, HYPER["steps"],
                         precision)
        arr, n = B.make_descs([d[0] for d in got], [d[1] for d in got], [d[2] for d in got],
                              [d[3] for d in got])
        B.check(B.lib().dmuon_muon_step_noalloc(arr, n, ctypes.byref(cfg),
                                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
        torch.cuda.synchronize()
        for td, r, g in zip(tds, ref, got):
            for k in (1, 2, 3):          # momentum, master, NS output
                assert torch.equal(r[k], g[k]), (td.spec.shape, k)
            Bo, Oo, _ = oracle.muon_step(td.grad, td.momentum, td.master, lr=HYPER["lr"], mu=HYPER["mu"],
                                         wd=HYPER["wd"], eps=HYPER["eps"], a=Q5[0], b=Q5[1], c=Q5[2],
                                         steps=HYPER["steps"])
            O = g[3].cpu().numpy()
            assert rel(O, Oo) <= TOL[precision]
            assert rel(g[1].cpu().numpy(), Bo) <= 1e-6
            assert rel(g[2].cpu().numpy(), oracle.decay_update(td.master, O, HYPER["lr"], HYPER["wd"])) <= 1e-6


@pytest.mark.parametrize("precision", ["bf16", "f32"])
def test_noalloc_captured_in_a_graph(precision):
    """Code under graph capture is one of the callers the allocation-free step
    is for: the step captured into a graph (its table copies are kernels, so
    every replay rewrites the scratch tables) and replayed twice, with eager
    work and synchronisations between the replays, gives the bits of two
    direct allocation-free steps."""
    tds = [make_custom((600, 1000), "bf16", seed=(92, 0), scale=1e-3),
           make_custom((2, 520, 300), "f32", seed=(92, 1))]

    def setup():
        devs = [to_dev(td) for td in tds]
        cfg = B.make_cfg(HYPER["lr"], HYPER["mu"], HYPER["wd"], HYPER["eps"], Q5, HYPER["steps"], precision)
        arr, n = B.make_descs([d[0] for d in devs], [d[1] for d in devs], [d[2] for d in devs],
                              [d[3] for d in devs])
        return devs, cfg, arr, n

    def call(cfg, arr, n):
        B.check(B.lib().dmuon_muon_step_noalloc(arr, n, ctypes.byref(cfg),
                                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))

    def snap(devs):
        return [[d[k].cpu().numpy() for k in (1, 2, 3)] for d in devs]

    devs, cfg, arr, n = setup()
    call(cfg, arr, n)
    torch.cuda.synchronize()
    want1 = snap(devs)
    call(cfg, arr, n)
    torch.cuda.synchronize()
    want2 = snap(devs)

    devs, cfg, arr, n = setup()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(cfg, arr, n)
    torch.cuda.synchronize()
    for want in (want1, want2):
        graph.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda") * 2.0       # eager work between the replays
        torch.cuda.synchronize()
        del junk
        for w, g in zip(want, snap(devs)):
            assert all(np.array_equal(a, b) for a, b in zip(w, g))
