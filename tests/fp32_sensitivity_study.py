"""How many codes can ANY fp32 pipeline keep identical to the fp64 oracle?

A CPU-only study (not collected by pytest; run it as a script).  GPTQ's
sweep is chaotic along a row: when a pre-rounding value sits closer to a
rounding boundary than the arithmetic's error, the two precisions may round
it to the two sides, and every later code of that row is computed from a
different history ("Part 3: Adaptive Rounding: GPTQ", 'Algorithm GPTQ' and
'Observation 3: The Cholesky Reformulation', which points at accumulated
floating-point error).  So the identical fraction depends on how large the
arithmetic's error is, not only on whether the arithmetic is right.

For one layer configuration this runs the fp64 oracle as the reference and
then variants that each introduce one kind of error of the size an fp32 GPU
pipeline introduces, and reports the identical fraction of each against the
reference on the same sampled rows:

  h32       H summed in fp32 (fp16 x fp16 products are exact in fp32), then
            the fp64 factor and sweep
  prep32    the factor computed in fp32 (LAPACK spotrf / spotri / spotrf on
            the reference H rounded to fp32), then the fp64 sweep
  pert:e    the reference factor with every entry multiplied by
            (1 + e N(0, 1)), then the fp64 sweep
  sweep32   the reference factor rounded to fp32 and the blocked sweep run in
            fp32 arithmetic
  all32     h32 + prep32 + sweep32
  gpu_u     (optional, --gpu-u file.npy) a factor computed elsewhere, e.g.
            by the GPU library, from the fp32 H, then the fp64 sweep

Usage:
    python tests/fp32_sensitivity_study.py --workload block7b --job 3 --rows 1024

Prints one line per variant and a JSON summary (--json PATH).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
from scipy.linalg import lapack

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import oracle as O  # noqa: E402
import synth  # noqa: E402


def hessian_fp32(X: np.ndarray, chunk: int = 2048) -> np.ndarray:
    """2 X^T X with every chunk's product and the running sum in fp32."""
    n = X.shape[1]
    H = np.zeros((n, n), dtype=np.float32)
    for c in range(0, X.shape[0], chunk):
        x = X[c:c + chunk].astype(np.float32)
        H += x.T @ x
    return H * np.float32(2.0)


def hessian_fp64(X: np.ndarray, chunk: int = 2048) -> np.ndarray:
    return O.hessian(X[c:c + chunk] for c in range(0, X.shape[0], chunk))


def factor_fp32(Hd32: np.ndarray) -> np.ndarray:
    """Upper U with Hd^-1 = U^T U by the three LAPACK steps, all in fp32."""
    L, info = lapack.spotrf(Hd32, lower=1, clean=1)
    assert info == 0, info
    G, info = lapack.spotri(L, lower=1)
    assert info == 0, info
    G = np.tril(G) + np.tril(G, -1).T
    U, info = lapack.spotrf(G, lower=0, clean=1)
    assert info == 0, info
    return np.triu(U)


def sweep_fp32(W: np.ndarray, U: np.ndarray, bits: int, group: int, block: int) -> dict:
    """The blocked sweep with fp32 values and fp32 arithmetic throughout
    (scale applied as a product with 1/s, as a GPU kernel would)."""
    V = np.array(W, dtype=np.float32)
    U = np.asarray(U, dtype=np.float32)
    m, n = V.shape
    G = O.n_groups(n, group)
    maxq = np.float32((1 << bits) - 1)
    q = np.zeros((m, n), dtype=np.int64)
    S = np.zeros((m, G), dtype=np.float32)
    Z = np.zeros((m, G), dtype=np.float32)
    E = np.zeros((m, block), dtype=np.float32)

    def params(vals):
        lo = np.minimum(vals.min(axis=1), np.float32(0))
        hi = np.maximum(vals.max(axis=1), np.float32(0))
        empty = hi == lo
        hi = np.where(empty, np.float32(1), hi)
        lo = np.where(empty, np.float32(0), lo)
        s = ((hi - lo) / maxq).astype(np.float32)
        z = np.rint(-lo / s).astype(np.float32)
        return s, z

    if group <= 0:
        S[:, 0], Z[:, 0] = params(V)
    for i in range(0, n, block):
        i2 = min(i + block, n)
        for p in range(i, i2):
            if group > 0 and p % group == 0:
                S[:, p // group], Z[:, p // group] = params(V[:, p:min(p + group, n)])
            gi = 0 if group <= 0 else p // group
            s, z = S[:, gi], Z[:, gi]
            inv_s = (np.float32(1) / s).astype(np.float32)
            qz = np.clip(np.rint(V[:, p] * inv_s), -z, maxq - z).astype(np.float32)
            q[:, p] = (qz + z).astype(np.int64)
            err = (V[:, p] - s * qz).astype(np.float32)
            e = (err / U[p, p]).astype(np.float32)
            E[:, p - i] = e
            V[:, p + 1:i2] -= np.outer(e, U[p, p + 1:i2]).astype(np.float32)
        if i2 < n:
            V[:, i2:] -= (E[:, :i2 - i] @ U[i:i2, i2:]).astype(np.float32)
    return {"q": q, "s": S.astype(np.float64), "z": Z.astype(np.float64)}


def compare(q: np.ndarray, ref: dict, group: int) -> dict:
    mism = q != ref["q"]
    rows = np.where(mism.any(axis=1))[0]
    gidx = np.zeros(q.shape[1], dtype=np.int64) if group <= 0 else np.arange(q.shape[1]) // group
    firsts = []
    for r in rows:
        p = int(np.argmax(mism[r]))
        d = min(float(O.boundary_distance(np.array([ref["t"][r, p]]))[0]),
                float(O.boundary_distance(np.array([ref["tz"][r, gidx[p]]]))[0]))
        firsts.append(d)
    return {"same_frac": 1.0 - float(mism.mean()), "rows_diverged": int(len(rows)),
            "mismatches": int(mism.sum()),
            "first_dist_max": max(firsts) if firsts else 0.0}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="block7b")
    ap.add_argument("--job", type=int, default=3)
    ap.add_argument("--rows", type=int, default=1024)
    ap.add_argument("--tokens", type=int, default=0, help="override the token count (0 = the workload's)")
    ap.add_argument("--eps", default="1e-7,3e-7,1e-6,3e-6")
    ap.add_argument("--gpu-u", default="", help="optional .npy factor to evaluate with the fp64 sweep")
    ap.add_argument("--json", default="")
    args = ap.parse_args()

    wl = synth.workloads()[args.workload]
    job = wl.jobs[args.job]
    xs = job.x
    if args.tokens:
        xs = synth.XSpec(xs.name, xs.n, args.tokens, xs.law, xs.dtype, xs.outlier_channels, xs.outlier_mult,
                         xs.corr_sigma)
    t0 = time.time()
    W = synth.stacked_weight(job, wl.seed, wl.wid)
    m, n = W.shape
    rng = np.random.default_rng(2024)
    rows = np.sort(rng.choice(m, size=min(args.rows, m), replace=False))
    Wr = W[rows].astype(np.float64)
    del W
    X = synth.x_full(xs, wl.seed, wl.wid)
    print(f"[{args.workload}/{args.job}] W {m}x{n} (rows sampled {len(rows)}) X {X.shape[0]}x{n} "
          f"bits {job.bits} group {job.group}; inputs {time.time() - t0:.1f}s", flush=True)

    H64 = hessian_fp64(X)
    H32 = hessian_fp32(X)
    del X
    print(f"  H fp64 / fp32 done {time.time() - t0:.1f}s; fp32 H rel err "
          f"{np.linalg.norm(H32 - H64) / np.linalg.norm(H64):.3e}", flush=True)
    Hd, lam = O.damp(H64, job.damp)
    U64, info = O.inverse_cholesky_upper(Hd)
    assert info == 0
    ev = np.linalg.eigvalsh(Hd)
    kappa = float(ev[-1] / ev[0])
    print(f"  reference factor {time.time() - t0:.1f}s; cond(H_d) {kappa:.3e}", flush=True)
    ref = O.gptq_quantize(Wr, U64, job.bits, job.group, job.block)
    out = {"workload": args.workload, "job": args.job, "m": m, "n": n, "rows": len(rows),
           "tokens": int(xs.tokens), "cond_Hd": kappa, "variants": {}}

    def report(name, q, extra=None):
        c = compare(q, ref, job.group)
        if extra:
            c.update(extra)
        out["variants"][name] = c
        ex = "".join(f" {k} {v:.3e}" for k, v in (extra or {}).items())
        print(f"  {name:10s} identical {c['same_frac']:.6f}  rows diverged {c['rows_diverged']:4d}/{len(rows)}"
              f"  first-mismatch boundary distance max {c['first_dist_max']:.2e}{ex}  ({time.time() - t0:.0f}s)",
              flush=True)

    # fp32 Hessian, fp64 rest
    Hd32in, _ = O.damp(H32.astype(np.float64), job.damp)
    U_h32, info = O.inverse_cholesky_upper(Hd32in)
    assert info == 0
    report("h32", O.gptq_quantize(Wr, U_h32, job.bits, job.group, job.block)["q"],
           {"u_rel": float(np.linalg.norm(U_h32 - U64) / np.linalg.norm(U64))})
    del U_h32, Hd32in
    # fp32 factor from the reference H
    Hd_r32 = Hd.astype(np.float32)
    U_p32 = factor_fp32(Hd_r32).astype(np.float64)
    U_same, _ = O.inverse_cholesky_upper(Hd_r32.astype(np.float64))
    report("prep32", O.gptq_quantize(Wr, U_p32, job.bits, job.group, job.block)["q"],
           {"u_rel": float(np.linalg.norm(U_p32 - U_same) / np.linalg.norm(U_same))})
    del U_same
    # perturbed factor
    for e in [float(x) for x in args.eps.split(",") if x]:
        Up = U64 * (1.0 + e * rng.standard_normal(U64.shape))
        report(f"pert:{e:g}", O.gptq_quantize(Wr, np.triu(Up), job.bits, job.group, job.block)["q"])
        del Up
    # fp32 sweep
    report("sweep32", sweep_fp32(Wr, U64.astype(np.float32), job.bits, job.group, job.block)["q"])
    # all fp32
    Hd_a, _ = O.damp(H32.astype(np.float64), job.damp)
    U_a = factor_fp32(Hd_a.astype(np.float32))
    report("all32", sweep_fp32(Wr, U_a, job.bits, job.group, job.block)["q"])
    if args.gpu_u:
        Ug = np.load(args.gpu_u).astype(np.float64)
        report("gpu_u", O.gptq_quantize(Wr, Ug, job.bits, job.group, job.block)["q"],
               {"u_rel": float(np.linalg.norm(Ug - U64) / np.linalg.norm(U64))})
    if args.json:
        with open(args.json, "w") as f:
            json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
