"""The matrix-core ceiling probe on the GPU: it performs the instructions it
claims (the sum of every wave's accumulators equals the sum over all output
entries of its products, computed here in fp64 from the same operand
generator and the documented operand lane layouts), zero operands give zeros,
and the bench's ceiling measurement returns a plausible rate."""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

pytestmark = pytest.mark.gpu


def mix32(x):
    x = x.astype(np.uint64) & 0xFFFFFFFF
    x ^= x >> 16
    x = (x * 0x7FEB352D) & 0xFFFFFFFF
    x ^= x >> 15
    x = (x * 0x846CA68B) & 0xFFFFFFFF
    x ^= x >> 16
    return x


def operands(keys):
    """bf16 operand registers (8 values per lane) of the given keys, as float64."""
    h = mix32((keys[:, None].astype(np.uint64) * 8 + np.arange(8, dtype=np.uint64)[None, :]) & 0xFFFFFFFF)
    bits = (h & 0x807F) | ((120 + (h >> 8) % 14) << 7)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def wave_sums(shape, blocks, iters, absolute=False):
    """Σ over every accumulator entry of each wave after `iters` rounds (with
    absolute=True, the same sum of |products|, the scale of its rounding error).
    For a product of an (rows × K) and a (K × cols) fragment the sum of all
    outputs is Σ_k (Σ_rows a[·, k]) (Σ_cols b[k, ·]); lane l holds
    k = 8·(l // rows) + e of row / column l % rows (rows = 32 for 32×32×16, 16 for
    16×16×32)."""
    t = np.arange(blocks * 256, dtype=np.uint64)
    rows = shape
    kgrp = (np.arange(64) // rows)
    out = []
    for w in range(blocks * 4):
        lanes = t[w * 64:(w + 1) * 64]
        A = [operands(lanes * 16 + i) for i in range(4)]
        B = [operands(lanes * 16 + 8 + i) for i in range(4)]
        if absolute:
            A, B = [np.abs(a) for a in A], [np.abs(b) for b in B]
        # column sums per k: k = 8·group + e
        SA = [np.concatenate([a[kgrp == g].sum(0) for g in range(64 // rows)]) for a in A]
        SB = [np.concatenate([b[kgrp == g].sum(0) for g in range(64 // rows)]) for b in B]
        s = 0.0
        n_acc = 8 if shape == 32 else 16
        for u in range(4):
            for i in range(n_acc):
                q = (i + u) & 3 if shape == 32 else ((i >> 2) + u) & 3
                s += float(SA[i & 3] @ SB[q])
        out.append(s * (iters // 4))
    return np.array(out)


@pytest.mark.parametrize("shape", [32, 16])
def test_probe_accumulates_what_it_claims(shape):
    import torch
    from matrix_optimizer_muon_amd import probe
    blocks, iters = 2, 4
    sink = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda")
    probe.probe_mfma(shape, probe.RANDOM, blocks, iters, sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = sink.double().cpu().numpy().reshape(blocks * 4, 64).sum(1)
    want = wave_sums(shape, blocks, iters)
    # fp32 accumulation: ≤ 64 products per accumulator entry, then a 128-term sum
    # per lane, so the error stays below ~200 unit roundoffs of Σ|products|
    tol = 200 * 2.0 ** -24 * wave_sums(shape, blocks, iters, absolute=True)
    assert np.all(np.isfinite(got))
    assert np.all(np.abs(got - want) <= tol), (got - want, tol)
    probe.probe_mfma(shape, probe.ZERO, blocks, iters, sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.count_nonzero(sink).item() == 0


def test_bench_mfma_ceiling_is_plausible():
    import bench
    c = bench.mfma_ceiling(32, 0, seconds=0.5, settle=0.2)
    assert c["instruction"] == "v_mfma_f32_32x32x16_bf16" and c["operands"] == "random bf16"
    assert 200.0 < c["tflops"] < 2600.0, c
    assert c["launches"] >= 4
