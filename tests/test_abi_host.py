"""Host-side checks of libdmuon_ns that need no GPU.

* the library loads and exports every function that include/dmuon_ns.h declares;
* the C++ LPT equals the reference LPT of oracle/ (index work: bit-exact);
* argument validation rejects every bad call before anything is enqueued (the
  pointers used here are never dereferenced: validation makes no HIP call).
"""
import ctypes
import os
import re

import numpy as np
import pytest

from matrix_optimizer_muon_amd import _binding as B
from matrix_optimizer_muon_amd import lpt_assign
from oracle import lpt_assign as ref_lpt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "dmuon_ns.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dmuon_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_header_function():
    L = B.lib()
    names = header_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(L, name), name
    assert sorted(B.EXPORTED) == names
    assert L.dmuon_abi_version() == 5 == B.ABI_VERSION


# --------------------------------------------------------------------------
# LPT: C++ == reference
# --------------------------------------------------------------------------
def compare_lpt(rows, cols, batch, layer, R, merge=0, kind=0, owner=0):
    got = lpt_assign(rows, cols, batch, layer, R, merge_below_elems=merge, cost_kind=kind,
                     owner_slot=owner)
    want = ref_lpt(list(rows), list(cols), list(batch), list(layer), R, merge_below_elems=merge,
                   cost_kind=kind, owner_slot=owner)
    assert got["slot_of"].tolist() == want["slot_of"]
    assert got["slot_load"].tolist() == want["slot_load"]
    assert got["owner_order"].tolist() == want["owner_order"]
    assert got["group_offsets"].tolist() == want["group_offsets"]
    return got


@pytest.mark.parametrize("seed", range(30))
def test_lpt_matches_reference_random(seed):
    rng = np.random.default_rng([31, seed])
    n = int(rng.integers(1, 120))
    R = int(rng.integers(1, 12))
    rows = rng.choice([64, 128, 256, 512, 1000], n)
    cols = rng.choice([64, 128, 256, 512, 1000], n)
    batch = rng.integers(1, 4, n)
    layer = rng.integers(-1, max(1, n // 5), n)
    merge = int(rng.choice([0, 20000, 200000]))
    compare_lpt(rows, cols, batch, layer, R, merge=merge, kind=int(seed % 2),
                owner=int(rng.integers(0, R)))


def test_lpt_matches_reference_llama_d4096():
    from matrix_optimizer_muon_amd.workloads import workload
    wl = workload("llama_d4096")
    rows = [t.shape[0] for t in wl.tensors]
    cols = [t.shape[1] for t in wl.tensors]
    layer = [t.layer for t in wl.tensors]
    for owner in range(8):
        got = compare_lpt(rows, cols, [1] * 224, layer, 8, owner=owner)
    assert got["slot_load"].max() / got["slot_load"].mean() < 1.03


def test_lpt_empty_and_errors():
    got = lpt_assign(np.zeros(0), np.zeros(0), np.zeros(0), np.zeros(0), 4)
    assert got["slot_load"].tolist() == [0, 0, 0, 0]
    assert got["owner_order"].tolist() == []
    with pytest.raises(ValueError):
        lpt_assign([1], [1], [1], [0], 0)
    with pytest.raises(ValueError):
        lpt_assign([1], [1], [0], [0], 2)            # batch must be >= 1
    with pytest.raises(ValueError):
        lpt_assign([1], [1], [1], [0], 2, owner_slot=2)


# --------------------------------------------------------------------------
# validation of the GPU entry points (no GPU needed: all calls are rejected)
# --------------------------------------------------------------------------
FAKE = 0x7f0000000000       # a plausible device address, never dereferenced


def desc(ndim=2, shape=(8, 16), dtype=B.F32, base=FAKE, numel_bytes=1 << 20):
    t = B.Tensor()
    t.ndim = ndim
    for i, s in enumerate(shape[:3]):
        t.shape[i] = s
    t.grad_dtype = dtype
    t.grad = base
    t.momentum = base + numel_bytes
    t.master = base + 2 * numel_bytes
    t.ns_out = None
    t.param_out = None
    return t


def cfg(**kw):
    c = dict(lr=0.02, momentum=0.95, weight_decay=0.01, eps=1e-7, coeffs=(3.4445, -4.775, 2.0315),
             steps=5, precision="bf16", stream_groups=0)
    c.update(kw)
    return B.make_cfg(c["lr"], c["momentum"], c["weight_decay"], c["eps"], c["coeffs"],
                      c["steps"], c["precision"], 1.0, c["stream_groups"])


ENTRY = ("dmuon_muon_step", "dmuon_muon_step_prepare", "dmuon_muon_step_run")


def step(descs, c=None, ws=FAKE + (1 << 40), ws_bytes=1 << 40, side=None, n_side=0):
    """Call all three step entry points with the same arguments; they validate
    alike, so they must return the same code."""
    arr = (B.Tensor * max(len(descs), 1))(*descs)
    c = c or cfg()
    L = B.lib()
    rcs = []
    for name in ENTRY:
        args = [arr, len(descs), ctypes.byref(c), ctypes.c_void_p(ws), ws_bytes, None]
        if name != "dmuon_muon_step_prepare":
            args += [side, n_side]
        rcs.append(getattr(L, name)(*args))
    if n_side == 0 and side is None:
        assert len(set(rcs)) == 1, rcs
    return rcs[0] if len(set(rcs)) == 1 else rcs


def wsize(descs, c=None):
    arr = (B.Tensor * max(len(descs), 1))(*descs)
    out = ctypes.c_size_t(0)
    rc = B.lib().dmuon_muon_step_workspace_size(arr, len(descs), ctypes.byref(c or cfg()),
                                                ctypes.byref(out))
    return rc, out.value


def test_rejects_one_dim_tensor():
    assert step([desc(ndim=1, shape=(128,))]) == -2
    assert "2 dims" in B.lib().dmuon_last_error().decode()
    assert step([desc(ndim=4, shape=(2, 3, 4))]) == -2


def test_rejects_bad_arguments():
    assert step([desc(shape=(-1, 4))]) == -3
    assert step([desc(shape=(70000, 4))]) == -3
    assert step([desc(dtype=7)]) == -4
    assert step([desc()], cfg(precision="bf16"), ws=0) == -6
    assert step([desc()], ws=FAKE + (1 << 40) + 8) == -6          # misaligned
    assert step([desc()], ws_bytes=16) == -6                       # too small
    assert step([desc()], cfg(steps=65)) == -5
    assert step([desc()], cfg(steps=-1)) == -5
    assert step([desc()], cfg(eps=-1.0)) == -5
    assert step([desc()], cfg(lr=float("nan"))) == -5
    c = cfg()
    c.grad_scale = float("inf")
    assert step([desc()], c) == -5
    bad = desc()
    bad.master = None
    assert step([bad]) == -1
    c = cfg()
    c.prec = 5
    assert step([desc()], c) == -4
    assert step([desc()], cfg(stream_groups=5)) == -5
    assert step([desc()], cfg(stream_groups=-1)) == -5
    arr = (B.Tensor * 1)()
    assert B.lib().dmuon_muon_step(arr, -1, ctypes.byref(cfg()), None, 0, None, None, 0) == -3
    assert B.lib().dmuon_muon_step(None, 1, ctypes.byref(cfg()), None, 0, None, None, 0) == -1
    assert B.lib().dmuon_muon_step(arr, 1, None, None, 0, None, None, 0) == -1


def test_rejects_bad_side_streams():
    two = (ctypes.c_void_p * 2)(0x1000, None)
    one = (ctypes.c_void_p * 1)(0x1000)
    L = B.lib()
    arr = (B.Tensor * 1)(desc())
    for name in ("dmuon_muon_step", "dmuon_muon_step_run"):
        fn = getattr(L, name)
        base = [arr, 1, ctypes.byref(cfg()), ctypes.c_void_p(FAKE + (1 << 40)), 1 << 40, None]
        assert fn(*base, None, -1) == -5
        assert fn(*base, None, 1) == -1                 # array missing
        assert fn(*base, two, 2) == -1                   # NULL entry (the null stream)
        # a valid stream list passes validation; the call then fails only where it
        # would touch the GPU, after the forced failure point below
        os.environ["DMUON_TEST_FAIL_AT"] = "plan"
        try:
            assert fn(*base, one, 1) == -8
        finally:
            del os.environ["DMUON_TEST_FAIL_AT"]


def test_group_count():
    def groups(descs, c=None):
        arr = (B.Tensor * max(len(descs), 1))(*descs)
        out = ctypes.c_int32(-1)
        rc = B.lib().dmuon_muon_step_groups(arr, len(descs), ctypes.byref(c or cfg()), ctypes.byref(out))
        return rc, out.value
    small = [desc(shape=(512, 512), base=FAKE + (i << 24)) for i in range(6)]
    assert groups(small) == (0, 4)                       # under four rounds of tiles: 4 groups
    assert groups(small[:2]) == (0, 2)                   # never more than the tensors
    big = [desc(shape=(8192, 28672), base=FAKE + (i << 34)) for i in range(2)]
    assert groups(big) == (0, 1)                         # many rounds: one launch sequence
    assert groups(small, cfg(stream_groups=3)) == (0, 3)
    assert groups(small, cfg(stream_groups=1)) == (0, 1)
    assert groups([desc(shape=(0, 4))]) == (0, 0)
    assert groups(small, cfg(stream_groups=9))[0] == -5
    # the workspace depends on the group count (per-group tables)
    assert wsize(small, cfg(stream_groups=1))[1] != wsize(small, cfg(stream_groups=4))[1]


def test_rejects_aliasing():
    a = desc()
    a.master = a.momentum                                        # written twice
    assert step([a]) == -7
    a = desc()
    a.ns_out = a.grad                                            # writes over the gradient
    assert step([a]) == -7
    x, y = desc(base=FAKE), desc(base=FAKE + (1 << 20))          # y.grad == x.momentum
    assert step([x, y]) == -7
    x, y = desc(base=FAKE), desc(base=FAKE)                      # shared grads only: allowed
    y.momentum += 3 << 20
    y.master += 3 << 20
    rc, need = wsize([x, y])
    assert rc == 0 and need > 0
    # workspace overlapping a tensor
    assert step([desc()], ws=FAKE, ws_bytes=1 << 40) == -7
    # the published copy is a written buffer: it may not cover the gradient or the master
    a = desc()
    a.param_out = a.grad
    assert step([a]) == -7
    a = desc()
    a.param_out = a.master + 64
    assert step([a]) == -7
    a = desc()
    a.param_out = FAKE + (3 << 20)
    rc, need = wsize([a])
    assert rc == 0 and need > 0


def test_zero_size_is_noop_and_needs_no_workspace():
    assert step([desc(shape=(0, 16))], ws=0, ws_bytes=0) == 0
    assert step([desc(ndim=3, shape=(0, 4, 4))], ws=0, ws_bytes=0) == 0
    assert step([], ws=0, ws_bytes=0) == 0
    assert wsize([desc(shape=(5, 0))]) == (0, 0)


def test_workspace_size_properties():
    rc1, s_bf = wsize([desc(shape=(256, 512))], cfg(precision="bf16"))
    rc2, s_f = wsize([desc(shape=(256, 512))], cfg(precision="f32"))
    assert rc1 == rc2 == 0
    assert s_f > s_bf > 256 * 512 * 4
    rc3, s_t = wsize([desc(shape=(512, 256))], cfg(precision="bf16"))   # tall: same operands
    assert rc3 == 0 and s_t == s_bf
    rc4, s_b = wsize([desc(ndim=3, shape=(3, 256, 512))], cfg(precision="bf16"))
    assert rc4 == 0 and 2.5 * s_bf < s_b < 3.5 * s_bf
    out = ctypes.c_size_t(0)
    assert B.lib().dmuon_ns_batched_workspace_size(2, 100, 300, 0, 5, ctypes.byref(out)) == 0
    assert out.value > 0
    assert B.lib().dmuon_ns_batched_workspace_size(2, 100, 300, 9, 5, ctypes.byref(out)) == -4


def test_ns_batched_and_gemm_validation():
    L = B.lib()
    vp = ctypes.c_void_p
    args = dict(a=3.4445, b=-4.775, c=2.0315)
    assert L.dmuon_ns_batched(vp(FAKE), 0, vp(FAKE), 1, 4, 4, *args.values(), 5, 1e-7, 1, 0,
                              vp(0), 0, None) == -7                      # out overlaps x
    assert L.dmuon_ns_batched(vp(FAKE), 0, vp(FAKE + 4096), 1, 4, 4, *args.values(), 5, 1e-7, 1,
                              0, vp(0), 0, None) == -6
    assert L.dmuon_ns_batched(vp(FAKE), 0, vp(FAKE + 8), 1, 4, 4, *args.values(), 5, 1e-7, 1, 0,
                              vp(FAKE + (1 << 30)), 1 << 30, None) == -7
    assert L.dmuon_ns_batched(vp(FAKE), 3, vp(FAKE), 1, 4, 4, *args.values(), 5, 1e-7, 1, 0,
                              vp(0), 0, None) == -4
    assert L.dmuon_ns_batched(vp(FAKE), 0, vp(FAKE + 4096), 1, 4, 4, *args.values(), 5, 1e-7, 2, 0,
                              vp(0), 0, None) == -5
    assert L.dmuon_ns_batched(None, 0, None, 0, 4, 4, *args.values(), 5, 1e-7, 1, 0,
                              vp(0), 0, None) == 0
    assert L.dmuon_gemm_nt(vp(FAKE), vp(FAKE), vp(FAKE), 4, 4, 10, 32, 64, 4, 1, None) == -3
    assert L.dmuon_gemm_nt(vp(FAKE), vp(FAKE), vp(FAKE), 4, 4, 10, 64, 64, 4, 2, None) == -4


@pytest.mark.parametrize("where", ["plan", "table"])
def test_forced_failure_before_enqueue(monkeypatch, where):
    """'plan' fails after validation; 'table' fails the table copy before its
    first launch: neither makes a HIP call, so both run without a GPU."""
    monkeypatch.setenv("DMUON_TEST_FAIL_AT", where)
    L = B.lib()
    arr = (B.Tensor * 1)(desc())
    ws = ctypes.c_void_p(FAKE + (1 << 40))
    assert L.dmuon_muon_step(arr, 1, ctypes.byref(cfg()), ws, 1 << 40, None, None, 0) == -8
    assert f"DMUON_TEST_FAIL_AT={where}" in L.dmuon_last_error().decode()
    assert L.dmuon_muon_step_prepare(arr, 1, ctypes.byref(cfg()), ws, 1 << 40, None) == -8
    vp = ctypes.c_void_p
    assert L.dmuon_ns_batched(vp(FAKE), 0, vp(FAKE + 4096), 1, 4, 4, 3.4, -4.7, 2.0, 5, 1e-7, 1, 0,
                              ws, 1 << 40, None) == -8
    if where == "plan":   # run copies no table: it fails at 'plan' only
        assert L.dmuon_muon_step_run(arr, 1, ctypes.byref(cfg()), ws, 1 << 40, None, None, 0) == -8
    # an invalid call still reports its own error first
    assert L.dmuon_muon_step(arr, 1, ctypes.byref(cfg(steps=99)), ws, 1 << 40, None, None, 0) == -5
    monkeypatch.delenv("DMUON_TEST_FAIL_AT")


def test_noalloc_validation():
    """The allocation-free step validates like the others and refuses a step
    whose scratch would exceed the static 64 MiB before any HIP call."""
    L = B.lib()

    def noalloc(descs, c=None):
        arr = (B.Tensor * max(len(descs), 1))(*descs)
        return L.dmuon_muon_step_noalloc(arr, len(descs), ctypes.byref(c or cfg()), None)
    assert noalloc([desc(ndim=1, shape=(128,))]) == -2
    assert noalloc([desc()], cfg(stream_groups=2)) == -5
    a = desc()
    a.master = a.momentum
    assert noalloc([a]) == -7
    assert noalloc([desc(shape=(0, 7))]) == 0
    assert noalloc([desc(shape=(8192, 28672), numel_bytes=1 << 30)]) == -6
    assert "static scratch" in L.dmuon_last_error().decode()
    rc, need = wsize([desc(shape=(4096, 4096), numel_bytes=1 << 30)], cfg(stream_groups=1))
    assert rc == 0 and need > 64 << 20
    assert noalloc([desc(shape=(4096, 4096), numel_bytes=1 << 30)]) == -6
    os.environ["DMUON_TEST_FAIL_AT"] = "plan"
    try:
        assert noalloc([desc(shape=(256, 512))]) == -8      # fits: fails only at the forced point
    finally:
        del os.environ["DMUON_TEST_FAIL_AT"]


def test_python_wrappers_raise_value_error():
    with pytest.raises(ValueError):
        B.check(-2)
    with pytest.raises(RuntimeError):
        B.check(-8)


# --------------------------------------------------------------------------
# the adamw route
# --------------------------------------------------------------------------
def adesc(numel=1000, dtype=B.F32, base=FAKE, span=1 << 20):
    t = B.AdamwTensor()
    t.numel = numel
    t.grad_dtype = dtype
    t.reserved = 0
    t.grad = base
    t.param = base + span
    t.exp_avg = base + 2 * span
    t.exp_avg_sq = base + 3 * span
    t.param_out = None
    return t


def acfg(**kw):
    c = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, grad_scale=1.0, step=1)
    c.update(kw)
    return B.AdamwCfg(c["lr"], c["beta1"], c["beta2"], c["eps"], c["weight_decay"], c["grad_scale"],
                      c["step"])


def astep(descs, c=None, ws=FAKE + (1 << 40), ws_bytes=1 << 40):
    arr = (B.AdamwTensor * max(len(descs), 1))(*descs)
    return B.lib().dmuon_adamw_step(arr, len(descs), ctypes.byref(c or acfg()), ctypes.c_void_p(ws),
                                    ws_bytes, None)


def awsize(descs):
    arr = (B.AdamwTensor * max(len(descs), 1))(*descs)
    out = ctypes.c_size_t(0)
    rc = B.lib().dmuon_adamw_step_workspace_size(arr, len(descs), ctypes.byref(out))
    return rc, out.value


def test_adamw_validation():
    assert astep([adesc(numel=-1)]) == -3
    assert astep([adesc(dtype=9)]) == -4
    bad = adesc()
    bad.reserved = 1
    assert astep([bad]) == -3
    bad = adesc()
    bad.exp_avg_sq = None
    assert astep([bad]) == -1
    assert astep([adesc()], acfg(step=0)) == -5
    assert astep([adesc()], acfg(beta1=1.0)) == -5
    assert astep([adesc()], acfg(beta2=-0.1)) == -5
    assert astep([adesc()], acfg(eps=0.0)) == -5
    assert astep([adesc()], acfg(lr=-1.0)) == -5
    assert astep([adesc()], acfg(grad_scale=float("nan"))) == -5
    assert astep([adesc()], ws=0) == -6
    assert astep([adesc()], ws_bytes=8) == -6
    arr = (B.AdamwTensor * 1)()
    assert B.lib().dmuon_adamw_step(arr, 1, None, None, 0, None) == -1
    assert B.lib().dmuon_adamw_step(None, 1, ctypes.byref(acfg()), None, 0, None) == -1


def test_adamw_aliasing_and_sizes():
    a = adesc()
    a.exp_avg = a.param                       # written twice
    assert astep([a]) == -7
    a = adesc()
    a.param_out = a.grad
    assert astep([a]) == -7
    x, y = adesc(base=FAKE), adesc(base=FAKE + (1 << 20))   # y.grad == x.param
    assert astep([x, y]) == -7
    assert astep([adesc()], ws=FAKE, ws_bytes=1 << 40) == -7
    assert astep([adesc(numel=0)], ws=0, ws_bytes=0) == 0
    assert astep([], ws=0, ws_bytes=0) == 0
    assert awsize([adesc(numel=0)]) == (0, 0)
    rc1, s1 = awsize([adesc()])
    rc2, s2 = awsize([adesc(base=FAKE + (i << 24)) for i in range(40)])
    assert rc1 == rc2 == 0 and 0 < s1 < s2


@pytest.mark.parametrize("where", ["plan", "table"])
def test_adamw_forced_failure(monkeypatch, where):
    monkeypatch.setenv("DMUON_TEST_FAIL_AT", where)
    assert astep([adesc()]) == -8
    monkeypatch.delenv("DMUON_TEST_FAIL_AT")


def test_debug_slice_buffers_layout():
    """The per-phase test hook: host only, so it runs here on plausible
    addresses.  Every buffer it reports lies inside the workspace, the
    buffers of one slice do not overlap, consecutive slices sit one slice
    stride apart, the shape fields follow the orientation rule, and bad
    indices are rejected."""
    L = B.lib()
    descs = [desc(2, (300, 700), B.BF16, base=FAKE, numel_bytes=1 << 24),
             desc(3, (3, 520, 300), B.F32, base=FAKE + (1 << 30), numel_bytes=1 << 24)]
    arr = (B.Tensor * 2)(*descs)
    for prec in ("bf16", "f32"):
        for groups in (1, 2):
            c = cfg(precision=prec, stream_groups=groups)
            rc, need = wsize(descs, c)
            assert rc == 0 and need > 0
            ws = FAKE + (1 << 40)
            esz = 2 if prec == "bf16" else 4

            def get(t, s):
                out = B.DebugSlice()
                rc = L.dmuon_debug_slice_buffers(arr, 2, ctypes.byref(c), ctypes.c_void_p(ws), need, t, s,
                                                 ctypes.byref(out))
                return rc, out

            rc, d0 = get(0, 0)
            assert rc == 0
            assert (d0.m, d0.n, d0.wide, d0.elem_bytes) == (300, 700, 1, esz)
            assert d0.ld_m == 320
            rc, d1 = get(1, 1)
            rc2, d2 = get(1, 2)
            assert rc == 0 and rc2 == 0
            assert (d1.m, d1.n, d1.wide) == (300, 520, 0)
            if prec == "bf16":      # the tensor's own layout (tall: 520 rows of 300)
                assert (d0.x_rows, d0.x_oriented, d1.x_rows, d1.x_oriented) == (300, 0, 520, 0)
                assert d0.x_ld >= 700 and d0.x_ld % 64 == 0 and d1.x_ld >= 300 and d1.x_ld % 64 == 0
            else:                   # oriented X: m rows of n
                assert (d0.x_rows, d0.x_oriented, d1.x_rows, d1.x_oriented) == (300, 1, 300, 1)
                assert d0.x_ld >= 700 and d1.x_ld >= 520
            for d in (d0, d1, d2):
                regions = [(d.x_copy, d.x_rows * d.x_ld * esz), (d.a_prime, d.m * d.ld_m * esz),
                           (d.b_prime, d.m * d.ld_m * esz), (d.scalars, 4 * 8)]
                for lo, size in regions:
                    assert ws <= lo and lo + size <= ws + need
                regions.sort()
                for (lo, size), (lo2, _) in zip(regions, regions[1:]):
                    assert lo + size <= lo2
            assert d2.a_prime - d1.a_prime == d1.m * d1.ld_m * esz
            assert d2.x_copy - d1.x_copy == d1.x_rows * d1.x_ld * esz
            assert d2.scalars - d1.scalars == 80 * 4
            assert get(2, 0)[0] == -3 and get(1, 3)[0] == -3 and get(0, 1)[0] == -3 and get(-1, 0)[0] == -3
            rc = L.dmuon_debug_slice_buffers(arr, 2, ctypes.byref(c), ctypes.c_void_p(ws), need, 0, 0, None)
            assert rc == -1
            rc = L.dmuon_debug_slice_buffers(arr, 2, ctypes.byref(c), ctypes.c_void_p(ws), need - 256, 0, 0,
                                             ctypes.byref(B.DebugSlice()))
            assert rc == -6


def test_workspace_regions_of_all_slices_are_disjoint():
    """The planner's workspace layout, on 30 seeded random tensor sets (2-D and
    3-D, wide and tall, ragged, both precisions, 1–4 groups): every slice's
    operand copy, A′, B′ and scalars lie inside the workspace, and no two of
    these regions, of the same or of different slices and tensors, overlap."""
    L = B.lib()
    rng = np.random.default_rng(12345)
    for case in range(30):
        n = int(rng.integers(1, 6))
        descs = []
        for k in range(n):
            rows, cols = int(rng.integers(1, 1500)), int(rng.integers(1, 1500))
            ndim = 3 if rng.random() < 0.4 else 2
            batch = int(rng.integers(1, 4))
            shape = (batch, rows, cols) if ndim == 3 else (rows, cols)
            descs.append(desc(ndim, shape, B.BF16 if rng.random() < 0.5 else B.F32,
                              base=FAKE + k * (1 << 32), numel_bytes=1 << 30))
        prec = "bf16" if rng.random() < 0.5 else "f32"
        c = cfg(precision=prec, stream_groups=int(rng.integers(1, 5)))
        rc, need = wsize(descs, c)
        assert rc == 0 and need > 0
        ws = FAKE + (1 << 44)
        esz = 2 if prec == "bf16" else 4
        arr = (B.Tensor * n)(*descs)
        regions = []
        for t, dsc in enumerate(descs):
            for s in range(dsc.shape[0] if dsc.ndim == 3 else 1):
                d = B.DebugSlice()
                assert L.dmuon_debug_slice_buffers(arr, n, ctypes.byref(c), ctypes.c_void_p(ws), need, t, s,
                                                   ctypes.byref(d)) == 0
                regions += [(d.x_copy, d.x_rows * d.x_ld * esz), (d.a_prime, d.m * d.ld_m * esz),
                            (d.b_prime, d.m * d.ld_m * esz), (d.scalars, 80 * 4)]
        regions.sort()
        for lo, size in regions:
            assert ws <= lo and lo + size <= ws + need, case
        for (lo, size), (lo2, _) in zip(regions, regions[1:]):
            assert lo + size <= lo2, case
