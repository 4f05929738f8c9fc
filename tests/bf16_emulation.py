"""numpy emulation of the bf16 matrix-core path's numerics (test helper, CPU).

It models what the HIP kernels round and where, not how they tile or order
their sums:
* matrix-core operands are bf16 (round to nearest even) and products
  accumulate in fp32 (numpy sgemm);
* the diagonal shift: A = d·I + A' with d = ‖X‖²_F / m, so that
  aX + bAX + cA²X = (a + bd + cd²)·X + [(b + 2cd)·A' + c·A'²]·X; A' and B'
  are stored as bf16;
* the start X₀ = inv·B is never formed: the first Gram scales its accumulator
  by inv² and the first apply multiplies (α·B + B'·bf16(B)) by inv;
* the iterate is computed in fp32; between iterations it is kept as its bf16
  copy hi (the next operand) plus lo = X − hi stored as signed bytes with one
  shared exponent per 16 values of a column (``iterate="hilo8"``, the
  library's storage), or rounded to nearest even to its top ``iterate_bits``
  bits (``iterate="bits"``);
* d_{t+1} is the fp32 sum of squares of the fp32 iterate, over m.

``shift=False`` or ``iterate="bits", iterate_bits=16`` (a bf16 iterate) give
the weaker schemes the design was chosen over; the tests use them as controls.
"""
import numpy as np

from matrix_optimizer_muon_amd.workloads import bf16_bits_to_f32, f32_to_bf16_bits


def bf16(x):
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def round_bits(x, bits):
    """Round fp32 to its top ``bits`` bits, to nearest even (bits ≤ 32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if bits >= 32:
        return x.copy()
    drop = 32 - bits
    u = x.view(np.uint32).astype(np.uint64)
    half = (1 << (drop - 1)) - 1
    u = (u + half + ((u >> drop) & 1)) >> drop << drop
    return (u & 0xFFFFFFFF).astype(np.uint32).view(np.float32)


def hilo8(X, block=16):
    """hi = bf16(X) plus lo = X − hi quantised to signed bytes q with a shared
    power-of-two scale per block of 16 values down a column: with mx the
    block's largest |lo|, lo ≈ q·2^(E − 7), 2^(E−1) ≤ mx < 2^E, |q| ≤ 127."""
    X = np.asarray(X, dtype=np.float32)
    hi = bf16(X)
    lo = (X - hi).astype(np.float32)
    m, n = lo.shape
    pad = (-m) % block
    L = np.pad(lo, ((0, pad), (0, 0))).reshape(-1, block, n)
    mx = np.abs(L).max(axis=1, keepdims=True)
    e = np.where(mx > 0, np.floor(np.log2(np.where(mx > 0, mx, 1.0))) + 1, 0)
    q = np.clip(np.rint(L * 2.0 ** (7 - e)), -127, 127)
    lo_q = (q * 2.0 ** (e - 7)).astype(np.float32).reshape(-1, n)[:m]
    return hi + lo_q


def ns_bf16_path(B, a, b, c, steps, eps, iterate="hilo8", iterate_bits=24, shift=True):
    """k Newton–Schulz iterations of one 2-D slice B (fp32) as the bf16 path
    computes them; returns the fp32 output in B's orientation."""
    B = np.asarray(B, dtype=np.float32)
    tall = B.shape[0] > B.shape[1]
    if tall:
        B = np.ascontiguousarray(B.T)
    m = B.shape[0]
    f = np.float32
    ss = np.sum(B.astype(np.float32) ** 2, dtype=np.float32)
    inv = f(1.0) / (np.sqrt(ss) + f(eps))
    X = B                      # unscaled start; inv rides on the first Gram and apply
    d = f(ss * inv * inv / f(m)) if shift else f(0.0)
    scale = inv
    I = np.eye(m, dtype=np.float32)
    for _ in range(steps):
        Xb = bf16(X)
        acc = Xb @ Xb.T
        Ap = bf16(scale * scale * acc - d * I)
        Bp = bf16(f(b + 2 * c * d) * Ap + f(c) * (Ap @ Ap.T))
        alpha = f(a + b * d + c * d * d)
        Xn = scale * (alpha * X + Bp @ Xb)
        d = f(np.sum(Xn * Xn, dtype=np.float32) / f(m)) if shift else f(0.0)
        X = hilo8(Xn) if iterate == "hilo8" else round_bits(Xn, iterate_bits)
        scale = f(1.0)
    X = Xn                     # the last iterate leaves the apply unrounded
    return np.ascontiguousarray(X.T) if tall else X
