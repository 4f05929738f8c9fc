"""Pins of the oracle's publish cast, gradient-ingest scale and AdamW route step.

Each check ties the oracle to something other than its own code: a library
routine (torch's CPU bf16 conversion, torch.optim.AdamW run in float64), values
fixed by the bf16 format, or closed forms of the recurrences.
"""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")


def torch_bf16_bits(x32):
    return torch.from_numpy(np.ascontiguousarray(x32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_publish_matches_torch_rounding_over_magnitudes():
    rng = np.random.default_rng(5)
    mant = rng.standard_normal(200000)
    expo = rng.integers(-140, 128, 200000).astype(np.float64)
    with np.errstate(over="ignore"):
        x = (mant * np.exp2(expo)).astype(np.float32)
    x[:4] = [0.0, -0.0, np.inf, -np.inf]
    assert np.array_equal(oracle.publish_bf16(x), torch_bf16_bits(x))


def test_publish_format_values():
    one = np.float32(1.0)
    cases = {
        float(one): 0x3F80,
        1.0 + 2.0 ** -8: 0x3F80,            # exact half between 0x3F80 and 0x3F81: even wins
        1.0 + 3 * 2.0 ** -8: 0x3F82,        # exact half between 0x3F81 and 0x3F82: even wins
        1.0 + 2.0 ** -8 + 2.0 ** -20: 0x3F81,   # just above the half rounds up
        -2.0: 0xC000,
        float(np.finfo(np.float32).max): 0x7F80,   # carries into the exponent: +inf
        2.0 ** -133: 0x0001,                 # smallest bf16 subnormal, exact
        2.0 ** -135: 0x0000,                 # a quarter of it rounds to zero
        2.0 ** -126: 0x0080,                 # smallest normal
    }
    x = np.array(list(cases), dtype=np.float32)
    got = oracle.publish_bf16(x)
    assert [int(v) for v in got] == list(cases.values())
    nan = oracle.publish_bf16(np.array([np.nan], dtype=np.float32))[0]
    assert (int(nan) & 0x7F80) == 0x7F80 and (int(nan) & 0x7F) != 0


def test_grad_scale_closed_form():
    rng = np.random.default_rng(2)
    G = rng.standard_normal((6, 9))
    s, mu, t = 0.125, 0.95, 7
    B = np.zeros_like(G)
    for _ in range(t):
        B = oracle.momentum_update(B, G, mu, grad_scale=s)
    assert np.allclose(B, s * G * (1 - mu ** t) / (1 - mu), rtol=1e-13, atol=0)


def test_muon_step_with_scale_equals_prescaled_gradient():
    rng = np.random.default_rng(3)
    G = rng.standard_normal((12, 20))
    B = rng.standard_normal((12, 20))
    W = rng.standard_normal((12, 20))
    kw = dict(lr=0.02, mu=0.95, wd=0.01, eps=1e-7, a=3.4445, b=-4.7750, c=2.0315, steps=5)
    r1 = oracle.muon_step(G, B, W, grad_scale=0.25, **kw)
    r2 = oracle.muon_step(0.25 * G, B, W, **kw)
    for x, y in zip(r1, r2):
        assert np.allclose(x, y, rtol=1e-12, atol=1e-14)


ADAM = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01)


def test_adamw_first_step_closed_form():
    rng = np.random.default_rng(4)
    p0 = rng.standard_normal(1000) * 0.02
    g = rng.standard_normal(1000) * 1e-3
    z = np.zeros(1000)
    p1, m1, v1 = oracle.adamw_step(p0, g, z, z, step=1, **ADAM)
    lr, wd, eps = ADAM["lr"], ADAM["wd"], ADAM["eps"]
    # bias correction makes m̂ = g and v̂ = g² after one step from zero state
    assert np.allclose(p1, p0 * (1 - lr * wd) - lr * g / (np.abs(g) + eps), rtol=1e-12, atol=0)
    assert np.allclose(m1, (1 - ADAM["beta1"]) * g, rtol=1e-14, atol=0)
    assert np.allclose(v1, (1 - ADAM["beta2"]) * g * g, rtol=1e-14, atol=0)


def test_adamw_constant_gradient_closed_form():
    rng = np.random.default_rng(6)
    p0 = rng.standard_normal(500)
    g = rng.standard_normal(500)
    p, m, v = p0, np.zeros(500), np.zeros(500)
    t = 9
    for k in range(1, t + 1):
        p, m, v = oracle.adamw_step(p, g, m, v, step=k, **ADAM)
    lr, wd, eps = ADAM["lr"], ADAM["wd"], ADAM["eps"]
    q = 1 - lr * wd
    # with a constant gradient m̂ = g and v̂ = g² at every step
    step = lr * g / (np.abs(g) + eps)
    expect = p0 * q ** t - step * sum(q ** j for j in range(t))
    assert np.allclose(p, expect, rtol=1e-11, atol=1e-15)
    assert np.allclose(m, (1 - ADAM["beta1"] ** t) * g, rtol=1e-12, atol=0)
    assert np.allclose(v, (1 - ADAM["beta2"] ** t) * g * g, rtol=1e-12, atol=0)


def test_adamw_matches_torch_optim_in_float64():
    rng = np.random.default_rng(8)
    n = 3000
    p0 = rng.standard_normal(n) * 0.05
    grads = [rng.standard_normal(n) * 10.0 ** rng.integers(-4, 1) for _ in range(6)]
    tp = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.AdamW([tp], lr=ADAM["lr"], betas=(ADAM["beta1"], ADAM["beta2"]), eps=ADAM["eps"],
                            weight_decay=ADAM["wd"])
    p, m, v = p0, np.zeros(n), np.zeros(n)
    for k, g in enumerate(grads, start=1):
        tp.grad = torch.from_numpy(g.copy())
        opt.step()
        p, m, v = oracle.adamw_step(p, g, m, v, step=k, **ADAM)
    st = opt.state[tp]
    assert np.allclose(tp.detach().numpy(), p, rtol=1e-12, atol=1e-15)
    assert np.allclose(st["exp_avg"].numpy(), m, rtol=1e-12, atol=1e-18)
    assert np.allclose(st["exp_avg_sq"].numpy(), v, rtol=1e-12, atol=1e-22)


def test_adamw_zero_gradient_only_decays():
    p0 = np.linspace(-1, 1, 11)
    m0 = np.full(11, 0.5)
    v0 = np.full(11, 0.25)
    p, m, v = oracle.adamw_step(p0, np.zeros(11), m0, v0, step=3, **ADAM)
    assert np.allclose(m, ADAM["beta1"] * m0, rtol=1e-15, atol=0)
    assert np.allclose(v, ADAM["beta2"] * v0, rtol=1e-15, atol=0)
    lr = ADAM["lr"]
    m_hat = m / (1 - ADAM["beta1"] ** 3)
    v_hat = v / (1 - ADAM["beta2"] ** 3)
    assert np.allclose(p, p0 * (1 - lr * ADAM["wd"]) - lr * m_hat / (np.sqrt(v_hat) + ADAM["eps"]), rtol=1e-13, atol=0)


def test_adamw_rejects_step_zero():
    with pytest.raises(ValueError):
        oracle.adamw_step(np.zeros(2), np.zeros(2), np.zeros(2), np.zeros(2), step=0, **ADAM)
