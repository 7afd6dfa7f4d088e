"""Would the trailing products keep the codes if they ran as bf16 products?

A CPU-only study (not collected by pytest; run it as a script).  The lazy
trailing update V[:, i2:] -= E U[i:i2, i2:] ("Part 3: Adaptive Rounding:
GPTQ", 'Observation 2: Lazy Batch Updates') is a dense product.  Splitting
each fp32 operand into x_hi = bf16(x) and x_lo = bf16(x - x_hi) and taking
E U ~ E_hi U_hi + E_hi U_lo + E_lo U_hi keeps about 16 bits of every term,
so three bf16 products could replace one fp32 product on the matrix cores.
This runs the oracle's blocked sweep (B = 128, 4-bit, group 128, on inputs of
the attention-projection recipe) once in fp64 and once with every flush
product computed that way (the other variants: fp32 products, and a
six-product split with three parts per operand), and reports the identical
fraction and the distance of each diverged row's first mismatch from a
rounding boundary in steps (the bar allows decisions within 1e-4 steps).

  python tests/bf16x3_flush_study.py 1024 4096 f32 x3

Measured (1024 x 4096, 16384 tokens): f32 1.000000 identical; x3 0.999765,
11 of 1024 rows diverged, every first mismatch within 3.6e-6 steps of a
boundary.  (256 x 2048: x3 1 row, 1.0e-6 steps; x6 identical.)
"""
import os
import sys
import time

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import oracle as O  # noqa: E402
import synth  # noqa: E402


def bf16(x):
    """Round to bfloat16 (nearest, ties to even), returned as fp64."""
    a = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((a + 0x7FFF + ((a >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def split(x, parts):
    out, r = [], np.asarray(x, np.float64)
    for _ in range(parts):
        h = bf16(r)
        out.append(h)
        r = r - h
    return out


def product(A, B, mode):
    if mode == "f64":
        return A @ B
    if mode == "f32":
        return (A.astype(np.float32) @ B.astype(np.float32)).astype(np.float64)
    if mode == "x3":
        Ah, Al = split(A, 2)
        Bh, Bl = split(B, 2)
        return Ah @ Bh + Ah @ Bl + Al @ Bh
    if mode == "x6":
        A0, A1, A2 = split(A, 3)
        B0, B1, B2 = split(B, 3)
        return A0 @ B0 + A0 @ B1 + A1 @ B0 + A0 @ B2 + A1 @ B1 + A2 @ B0
    raise ValueError(mode)


def sweep(W, U, bits, group, B, mode):
    """The blocked sweep of the oracle (readings R3-R8) with the flush
    product taken by `product`."""
    V = W.copy()
    m, n = V.shape
    maxq = 2 ** bits - 1
    q = np.zeros((m, n), np.int64)
    T = np.zeros((m, n))
    E = np.zeros((m, n))
    S = np.zeros((m, n // group))
    Z = np.zeros((m, n // group))
    for i in range(0, n, B):
        i2 = min(i + B, n)
        for p in range(i, i2):
            if p % group == 0:
                S[:, p // group], Z[:, p // group] = O.quant_params(V[:, p:p + group], bits)
            s, z = S[:, p // group], Z[:, p // group]
            T[:, p] = V[:, p] / s
            q[:, p] = np.clip(np.rint(T[:, p]) + z, 0, maxq)
            e = (V[:, p] - s * (q[:, p] - z)) / U[p, p]
            E[:, p] = e
            V[:, p + 1:i2] -= np.outer(e, U[p, p + 1:i2])
        if i2 < n:
            V[:, i2:] -= product(E[:, i:i2], U[i:i2, i2:], mode)
    return q, T


def main():
    m, n = int(sys.argv[1]), int(sys.argv[2])
    modes = sys.argv[3:] or ["f32", "x3"]
    bits, group, B = 4, 128, 128
    W, X = synth.small_layer(m, n, 4 * n, seed=3, law="lognormal", w_dtype="f16", x_dtype="f16",
                             outlier_frac=0.001, outlier_channels=8)
    H = O.hessian([X.astype(np.float64)])
    U, _ = O.inverse_cholesky_upper(O.damp(H, 0.01)[0])
    U = U.astype(np.float32).astype(np.float64)
    Wd = W.astype(np.float64)
    t0 = time.time()
    qr, Tr = sweep(Wd, U, bits, group, B, "f64")
    print(f"reference sweep {time.time() - t0:.1f} s", flush=True)
    for mode in modes:
        qm, _ = sweep(Wd, U, bits, group, B, mode)
        diff = qm != qr
        rows = np.where(diff.any(axis=1))[0]
        first = np.array([O.boundary_distance(Tr[r, np.argmax(diff[r]):np.argmax(diff[r]) + 1])[0] for r in rows])
        worst = first.max() if len(first) else 0.0
        print(f"{mode}: identical {1 - diff.mean():.6f}, rows diverged {len(rows)}/{m}, first mismatch at most "
              f"{worst:.2e} steps from a boundary ({int((first > 1e-4).sum())} beyond 1e-4)", flush=True)


if __name__ == "__main__":
    main()
