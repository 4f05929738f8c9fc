"""Parity of the publish copy, the gradient-ingest scale and the ``adamw`` route (MI355X).

Bars:
* published bf16 parameter: bit-exact against the oracle's round-to-nearest-even
  cast of the GPU's own updated master (the cast is a function of W');
* gradient-ingest scale: momentum ≤ 1e-6, NS output ≤ 2e-2 (bf16) / 1e-4 (fp32),
  update ≤ 1e-6 against the fp64 oracle, as for the plain step;
* AdamW route: parameter, first and second moment each ≤ 1e-6 relative
  (Frobenius) against the fp64 oracle; the bf16 copy bit-exact as above.
The AdamW hyper-parameters reach the kernel as the fp32 values of the C ABI
(β₂ = 0.999 becomes 0.99900001…), so the oracle is given those same fp32 values;
with a fresh state the second moment is entirely (1 − β₂)·g², where the two
spellings of β₂ differ by 1.3e-5.
Shapes cover even and odd row lengths (the two store forms of the publish copy),
ragged tiles, 2-D and 3-D tensors, k = 0, numel not a multiple of the vector
width, unaligned tensors (scalar path) and zero-size tensors.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import matrix_optimizer_muon_amd as mm  # noqa: E402
from matrix_optimizer_muon_amd.workloads import (HYPER, make_adamw, make_adamw_custom,  # noqa: E402
                                                  make_custom, workload)
import oracle  # noqa: E402

pytestmark = pytest.mark.gpu

TOL_NS = {"bf16": 2e-2, "f32": 1e-4}
ADAM = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01)


def rel(x, y):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    d = np.linalg.norm(y)
    return np.linalg.norm(x - y) / (d if d > 0 else 1.0)


def grad_dev(td):
    if td.grad_bits is not None:
        return torch.from_numpy(td.grad_bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(td.grad.copy()).cuda()


def words(t):
    return t.cpu().numpy().view(np.uint16)


# --------------------------------------------------------------------------
# Muon route: publish copy and gradient-ingest scale
# --------------------------------------------------------------------------
MUON_SHAPES = [((300, 520), "bf16"), ((520, 301), "f32"), ((257, 255), "f32"),
               ((2, 130, 77), "bf16"), ((1, 9), "f32"), ((513, 1024), "bf16"), ((0, 6), "f32")]


def run_muon(tds, precision, steps, grad_scale=1.0, publish=True):
    g = [grad_dev(td) for td in tds]
    b = [torch.from_numpy(td.momentum.copy()).cuda() for td in tds]
    w = [torch.from_numpy(td.master.copy()).cuda() for td in tds]
    o = [torch.empty(td.grad.shape, dtype=torch.float32, device="cuda") for td in tds]
    pub = [torch.full(td.grad.shape, -1, dtype=torch.int16, device="cuda") for td in tds] if publish else None
    mm.muon_step(g, b, w, steps=steps, precision=precision, grad_scale=grad_scale, ns_outs=o,
                 param_outs=pub)
    torch.cuda.synchronize()
    return ([x.cpu().numpy() for x in b], [x.cpu().numpy() for x in o], [x.cpu().numpy() for x in w],
            None if pub is None else [words(x) for x in pub])


@pytest.mark.parametrize("precision", ["bf16", "f32"])
@pytest.mark.parametrize("steps", [5, 0])
def test_publish_copy_bit_exact(precision, steps):
    tds = [make_custom(sh, dt, seed=(71, i), scale=1e-3 if dt == "bf16" else 1.0)
           for i, (sh, dt) in enumerate(MUON_SHAPES)]
    B1, O, W1, P = run_muon(tds, precision, steps)
    for td, w, p, o in zip(tds, W1, P, O):
        assert p.shape == w.shape
        assert np.array_equal(p, oracle.publish_bf16(w)), td.spec.shape
        _, Oref, _ = oracle.muon_step(td.grad, td.momentum, td.master, lr=HYPER["lr"], mu=HYPER["mu"],
                                      wd=HYPER["wd"], eps=HYPER["eps"], a=HYPER["a"], b=HYPER["b"],
                                      c=HYPER["c"], steps=steps)
        if td.grad.size:
            assert rel(o, Oref) <= TOL_NS[precision], (td.spec.shape, rel(o, Oref))
            assert rel(w, oracle.decay_update(td.master, o, HYPER["lr"], HYPER["wd"])) <= 1e-6
    # the copy changes nothing else: the same call without it gives the same bits
    B2, O2, W2, _ = run_muon(tds, precision, steps, publish=False)
    for a, b in zip(W1 + O + B1, W2 + O2 + B2):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("precision", ["bf16", "f32"])
def test_grad_scale_parity(precision):
    s = 0.125
    tds = [make_custom((300, 700), "bf16", seed=(72, 0), scale=8e-3),
           make_custom((700, 300), "f32", seed=(72, 1), scale=8.0),
           make_custom((2, 200, 260), "f32", seed=(72, 2), scale=8.0)]
    B1, O, W1, _ = run_muon(tds, precision, 5, grad_scale=s, publish=False)
    for td, b, o, w in zip(tds, B1, O, W1):
        Bref, Oref, _ = oracle.muon_step(td.grad, td.momentum, td.master, lr=HYPER["lr"], mu=HYPER["mu"],
                                         wd=HYPER["wd"], eps=HYPER["eps"], a=HYPER["a"], b=HYPER["b"],
                                         c=HYPER["c"], steps=5, grad_scale=s)
        assert rel(b, Bref) <= 1e-6
        assert rel(o, Oref) <= TOL_NS[precision]
        assert rel(w, oracle.decay_update(td.master, o, HYPER["lr"], HYPER["wd"])) <= 1e-6


def test_grad_scale_one_is_the_plain_step():
    tds = [make_custom((300, 520), "bf16", seed=(73, 0), scale=1e-3)]
    a = run_muon(tds, "bf16", 5, grad_scale=1.0, publish=False)
    g = [grad_dev(td) for td in tds]
    b = [torch.from_numpy(td.momentum.copy()).cuda() for td in tds]
    w = [torch.from_numpy(td.master.copy()).cuda() for td in tds]
    mm.muon_step(g, b, w, precision="bf16")
    torch.cuda.synchronize()
    assert np.array_equal(a[0][0], b[0].cpu().numpy()) and np.array_equal(a[2][0], w[0].cpu().numpy())


# --------------------------------------------------------------------------
# adamw route
# --------------------------------------------------------------------------
def run_adamw(ads, step, grad_scale=1.0, offsets=None, publish=True, **hp):
    h = dict(ADAM, **hp)
    offsets = offsets or [0] * len(ads)

    def place(arr, off):
        # an `off`-element offset inside a larger buffer breaks 16-byte alignment
        buf = torch.zeros(arr.size + off, dtype=torch.float32, device="cuda")
        buf[off:] = torch.from_numpy(arr.reshape(-1).copy()).cuda()
        return buf[off:]

    p = [place(a.param, o) for a, o in zip(ads, offsets)]
    m = [place(a.exp_avg, o) for a, o in zip(ads, offsets)]
    v = [place(a.exp_avg_sq, o) for a, o in zip(ads, offsets)]
    g = []
    for a, o in zip(ads, offsets):
        if a.grad_bits is not None:
            buf = torch.zeros(a.grad.size + o, dtype=torch.int16, device="cuda")
            buf[o:] = torch.from_numpy(a.grad_bits.view(np.int16).reshape(-1).copy()).cuda()
            g.append(buf[o:].view(torch.bfloat16))
        else:
            g.append(place(a.grad, o))
    pub = None
    if publish:
        pub = []
        for a, o in zip(ads, offsets):
            buf = torch.full((a.param.size + o,), -1, dtype=torch.int16, device="cuda")
            pub.append(buf[o:])
    mm.adamw_step(p, g, m, v, step=step, lr=h["lr"], betas=(h["beta1"], h["beta2"]), eps=h["eps"],
                  weight_decay=h["wd"], grad_scale=grad_scale, param_outs=pub)
    torch.cuda.synchronize()
    return ([x.cpu().numpy() for x in p], [x.cpu().numpy() for x in m], [x.cpu().numpy() for x in v],
            None if pub is None else [words(x) for x in pub])


def f32(hp):
    """Hyper-parameters as the fp32 values the C ABI carries."""
    return {k: float(np.float32(v)) for k, v in hp.items()}


def check_adamw(ads, step, grad_scale=1.0, offsets=None, **hp):
    h = f32(dict(ADAM, **hp))
    grad_scale = float(np.float32(grad_scale))
    P, M, V, PUB = run_adamw(ads, step, grad_scale, offsets, **hp)
    for a, p, m, v, pub in zip(ads, P, M, V, PUB):
        pr, mr, vr = oracle.adamw_step(a.param, a.grad, a.exp_avg, a.exp_avg_sq, lr=h["lr"],
                                       beta1=h["beta1"], beta2=h["beta2"], eps=h["eps"], wd=h["wd"],
                                       step=step, grad_scale=grad_scale)
        if a.param.size == 0:
            continue
        assert rel(p, pr) <= 1e-6, (a.spec.shape, rel(p, pr))
        assert rel(m, mr) <= 1e-6, (a.spec.shape, rel(m, mr))
        assert rel(v, vr) <= 1e-6, (a.spec.shape, rel(v, vr))
        assert np.array_equal(pub, oracle.publish_bf16(p))
    return P, M, V


NUMELS = [1, 7, 8, 1000, 16384, 16385, 100003, 0]


@pytest.mark.parametrize("step", [1, 10])
def test_adamw_group_parity(step):
    ads = [make_adamw_custom(n, "bf16" if i % 2 else "f32", seed=(81, i)) for i, n in enumerate(NUMELS)]
    check_adamw(ads, step)


def test_adamw_fresh_state_and_scale():
    ads = [make_adamw_custom(n, "f32", seed=(82, i), scale=4e-3, fresh_state=True)
           for i, n in enumerate([33, 4096, 50000])]
    check_adamw(ads, 1, grad_scale=0.25)


def test_adamw_unaligned_tensors_take_the_scalar_path():
    ads = [make_adamw_custom(n, "bf16", seed=(83, i)) for i, n in enumerate([40000, 777, 16390])]
    check_adamw(ads, 3, offsets=[1, 3, 2])


def test_adamw_other_hyperparameters():
    ads = [make_adamw_custom(20000, "f32", seed=(84, 0))]
    check_adamw(ads, 5, lr=3e-2, beta1=0.5, beta2=0.9, eps=1e-6, wd=0.1)


def test_adamw_five_steps_track_the_oracle():
    a = make_adamw_custom(30000, "f32", seed=(85, 0), fresh_state=True)
    p = torch.from_numpy(a.param.copy()).cuda()
    m = torch.zeros_like(p)
    v = torch.zeros_like(p)
    pr, mr, vr = a.param.astype(np.float64), np.zeros(30000), np.zeros(30000)
    rng = np.random.default_rng(86)
    for k in range(1, 6):
        g = (rng.standard_normal(30000) * 1e-3).astype(np.float32)
        mm.adamw_step([p], [torch.from_numpy(g).cuda()], [m], [v], step=k)
        pr, mr, vr = oracle.adamw_step(pr, g, mr, vr, step=k, **f32(ADAM))
    torch.cuda.synchronize()
    assert rel(p.cpu().numpy(), pr) <= 1e-6
    assert rel(m.cpu().numpy(), mr) <= 1e-6
    assert rel(v.cpu().numpy(), vr) <= 1e-6


def test_adamw_deterministic():
    ads = [make_adamw_custom(50001, "bf16", seed=(87, 0))]
    a = run_adamw(ads, 4)
    b = run_adamw(ads, 4)
    for x, y in zip(a, b):
        for u, w in zip(x, y):
            assert np.array_equal(u, w)


@pytest.mark.parametrize("name", ["adamw_llama_norms", "adamw_stream"])
def test_adamw_workloads_full(name):
    wl = workload(name)
    ads = [make_adamw(wl, t) for t in wl.tensors]
    check_adamw(ads, 10)


def test_prepared_steps_in_a_training_loop():
    """The prepared Muon step (2-D weights) and AdamW step (1-D biases) driving
    a small bf16 MLP as a training loop would: gradients kept in place between
    iterations (zero_grad(set_to_none=False)), fp32 masters and state in
    caller tensors, the bf16 weights rewritten by the steps' published copies.
    After each iteration every bf16 weight is the round-to-nearest-even bf16 of
    its fp32 master, and the loss stays finite."""
    import matrix_optimizer_muon_amd as mm
    torch.manual_seed(0)
    model = torch.nn.Sequential(torch.nn.Linear(64, 300), torch.nn.ReLU(),
                                torch.nn.Linear(300, 40)).cuda().to(torch.bfloat16)
    x = torch.randn(256, 64, device="cuda").to(torch.bfloat16)
    y = torch.randn(256, 40, device="cuda")

    def backward():
        loss = torch.nn.functional.mse_loss(model(x).float(), y)
        loss.backward()
        return float(loss.detach())

    mats = [p for p in model.parameters() if p.dim() >= 2]
    vecs = [p for p in model.parameters() if p.dim() < 2]
    masters = [p.detach().float() for p in mats]
    momenta = [torch.zeros_like(w) for w in masters]
    v_master = [p.detach().float() for p in vecs]
    m1, m2 = [torch.zeros_like(w) for w in v_master], [torch.zeros_like(w) for w in v_master]
    start = [w.clone() for w in masters]
    backward()
    muon = mm.MuonStep([p.grad for p in mats], momenta, masters, lr=0.02, momentum=0.95,
                       weight_decay=0.01, param_outs=[p.data for p in mats])
    adamw = mm.AdamwStep(v_master, [p.grad for p in vecs], m1, m2, lr=1e-3, param_outs=[p.data for p in vecs])
    for it in range(1, 4):
        muon()
        adamw(it)
        torch.cuda.synchronize()
        for p, w in list(zip(mats, masters)) + list(zip(vecs, v_master)):
            assert torch.equal(p.data, w.to(torch.bfloat16)), (it, tuple(p.shape))
        model.zero_grad(set_to_none=False)
        loss = backward()
        assert np.isfinite(loss), it
    assert all(not torch.equal(a, b) for a, b in zip(start, masters))
