"""Each phase of the step checked alone in fp64 on its own GPU inputs (needs an MI355X).

A prepared step with k = 1 leaves the first iteration's intermediates in its
workspace, and ``dmuon_debug_slice_buffers`` reports where: the operand copy
the Gram read, A′ = inv²·X Xᵀ − d₀·I, B′ = (b + 2c·d₀)·A′ + c·A′² and the
scalars inv, d₀.  The NS output of that step is X₁ = inv·(α·B + B′·X) with
α = a + b·d₀ + c·d₀².  Each quantity is recomputed in fp64 from the GPU's own
inputs to that phase, so a mistake in one kernel cannot hide behind the
others.  Bounds follow from the arithmetic:
* the bf16 copy of B is round-to-nearest-even of the GPU's fp32 momentum, bit
  for bit, with zeros in the row padding; the fp32 path's oriented copy is B;
* inv and d₀ are fp32 sums: ≤ 1e-5 relative;
* A′ and B′ on the bf16 path are one bf16 rounding of an fp32-accumulated
  value: within one bf16 unit in the last place (2⁻⁷ relative) plus 1e-5 of
  the largest value the fp32 sums held (for A′ the unshifted Gram, whose
  diagonal ≈ d₀ the shift cancels); both triangles hold the same values; on
  the fp32 path within 1e-5 of that scale;
* X₁: α·X reaches the bf16 matrix cores as α₁ + α₂ (two bf16 values, 2⁻¹⁷
  relative), the rest is fp32: ≤ 2e-5 relative Frobenius and 1e-4 of the
  largest entry elementwise.
"""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import matrix_optimizer_muon_amd as mm  # noqa: E402
from matrix_optimizer_muon_amd import _binding as B  # noqa: E402
from matrix_optimizer_muon_amd.workloads import (HYPER, bf16_bits_to_f32, f32_to_bf16_bits,  # noqa: E402
                                                  make_custom)

pytestmark = pytest.mark.gpu

A_, B_, C_ = HYPER["a"], HYPER["b"], HYPER["c"]


def to_dev(td):
    if td.grad_bits is not None:
        g = torch.from_numpy(td.grad_bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    else:
        g = torch.from_numpy(td.grad.copy()).cuda()
    return g, torch.from_numpy(td.momentum.copy()).cuda(), torch.from_numpy(td.master.copy()).cuda()


def read(ws, addr, count, dtype):
    """count elements of dtype at device address addr inside the workspace tensor."""
    off = addr - ws.data_ptr()
    nbytes = count * np.dtype(dtype).itemsize
    assert 0 <= off and off + nbytes <= ws.numel()
    return ws[off:off + nbytes].cpu().numpy().view(dtype)


def close_bf16(got, ref, scale):
    """Within one bf16 ulp of the reference (2⁻⁷ relative) plus 1e-5 of the
    scale of the fp32 sums it came from."""
    return np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-5 * scale


@pytest.mark.parametrize("precision", ["bf16", "f32"])
def test_each_phase_against_fp64(precision):
    tds = [make_custom((300, 700), "bf16", seed=(79, 0), scale=1e-3),      # wide, bf16 gradient
           make_custom((2, 600, 280), "f32", seed=(79, 1)),                # tall, batched
           make_custom((1100, 1500), "bf16", seed=(79, 2), scale=1e-3)]    # 5×6 ragged tiles
    devs = [to_dev(td) for td in tds]
    outs = [torch.zeros(td.grad.shape, dtype=torch.float32, device="cuda") for td in tds]
    st = mm.MuonStep([d[0] for d in devs], [d[1] for d in devs], [d[2] for d in devs], ns_outs=outs,
                     steps=1, precision=precision, stream_groups=1)
    st()
    torch.cuda.synchronize()
    ws = st.workspace
    esz = 2 if precision == "bf16" else 4
    for t, s in ((0, 0), (1, 1), (2, 0)):
        d = B.DebugSlice()
        B.check(B.lib().dmuon_debug_slice_buffers(st._m.arr, st._m.n, ctypes.byref(st.cfg),
                                                  ctypes.c_void_p(ws.data_ptr()), ws.numel(), t, s,
                                                  ctypes.byref(d)))
        m, n, wide = d.m, d.n, d.wide
        Bs = devs[t][1].cpu().numpy()
        Bs = Bs[s] if Bs.ndim == 3 else Bs                  # the GPU's new momentum, tensor layout
        Bo = (Bs if wide else Bs.T).astype(np.float64)      # oriented m×n
        label = f"tensor {t} slice {s} {Bs.shape} {precision}"

        # ingest: the operand copy
        xc = read(ws, d.x_copy, d.x_rows * d.x_ld, np.uint16 if esz == 2 else np.float32).reshape(d.x_rows, d.x_ld)
        if esz == 2:
            assert np.array_equal(xc[:, :Bs.shape[1]], f32_to_bf16_bits(Bs)), label
            assert not xc[:, Bs.shape[1]:].any(), label
            hi = bf16_bits_to_f32(xc[:, :Bs.shape[1]]).astype(np.float64)
            Xop = hi if wide else hi.T
        else:
            assert np.array_equal(xc[:, :n], (Bs if wide else Bs.T)), label
            assert not xc[:, n:].any(), label
            Xop = Bo

        # norm finalize
        inv, d0 = (float(v) for v in read(ws, d.scalars, 2, np.float32))
        nrm = np.linalg.norm(Bs.astype(np.float64))
        assert abs(inv - 1.0 / (nrm + HYPER["eps"])) <= 1e-5 * inv, label
        assert abs(d0 - nrm ** 2 * inv ** 2 / m) <= 1e-5 * d0, label

        def mat(addr):
            v = read(ws, addr, m * d.ld_m, np.uint16 if esz == 2 else np.float32).reshape(m, d.ld_m)[:, :m]
            return bf16_bits_to_f32(v).astype(np.float64) if esz == 2 else v.astype(np.float64)

        # Gram: A′ = inv²·X Xᵀ − d₀·I on the copy the Gram read
        Ap = mat(d.a_prime)
        A_ref = inv * inv * (Xop @ Xop.T) - d0 * np.eye(m)
        # square: B′ = (b + 2c·d₀)·A′ + c·A′² on the GPU's A′
        Bp = mat(d.b_prime)
        B_ref = (B_ + 2 * C_ * d0) * Ap + C_ * (Ap @ Ap)
        # the fp32 sums are those of the unshifted Gram inv²·X Xᵀ (diagonal ≈ d₀),
        # which the shift then mostly cancels on the diagonal
        scale_a = np.abs(A_ref + d0 * np.eye(m)).max()
        scale_b = np.abs(B_ref).max()
        if esz == 2:
            assert np.array_equal(Ap, Ap.T) and np.array_equal(Bp, Bp.T), label
            assert close_bf16(Ap, A_ref, scale_a).all(), (label, np.abs(Ap - A_ref).max())
            assert close_bf16(Bp, B_ref, scale_b).all(), (label, np.abs(Bp - B_ref).max())
        else:
            assert np.abs(Ap - A_ref).max() <= 1e-5 * scale_a, (label, np.abs(Ap - A_ref).max(), scale_a)
            assert np.abs(Bp - B_ref).max() <= 1e-5 * scale_b, (label, np.abs(Bp - B_ref).max(), scale_b)

        # apply (the last one, k = 1): X₁ = inv·(α·B + B′·X) is the NS output
        alpha = A_ + B_ * d0 + C_ * d0 * d0
        X1_ref = inv * (alpha * Bo + Bp @ Xop)
        O = outs[t].cpu().numpy()
        O = (O[s] if O.ndim == 3 else O).astype(np.float64)
        X1 = O if wide else O.T
        e = np.linalg.norm(X1 - X1_ref) / np.linalg.norm(X1_ref)
        print(f"{label}: copy exact, inv/d0 ok, A' ok, B' ok, X1 rel {e:.2e}", flush=True)
        assert e <= 2e-5, (label, e)
        assert np.abs(X1 - X1_ref).max() <= 1e-4 * np.abs(X1_ref).max(), label
