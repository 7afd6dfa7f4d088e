"""Comparison helpers between GPU outputs and the fp64 oracle.

Tolerances:
  * H: ||H_gpu - H_oracle||_F / ||H_oracle||_F <= 1e-5.
  * Codes and zero points: bit-exact along one history.  Where the oracle's
    pre-rounding value (v/s, or the zero point -x_lo/s of a group) lies
    within 1e-4 steps of a rounding boundary, the fp32 kernel and the fp64
    oracle may round to the two sides of it; both are correct roundings, and
    every later value of that row depends on which one was taken.  So the
    oracle's sweep is run again on the same inputs taking the GPU's choice at
    such near-ties (and nowhere else); every code and zero point must then be
    identical.  Before that, the first run's identical fraction must be at
    least MIN_SAME = 0.999 (the fraction of codes the sweep may change at
    near-ties and through what follows from them).
  * Scales: relative 1e-5 on every group of the followed run.
  * Layer loss ||(W - What) X||^2 (one fp64 evaluator for both sides): within
    1e-3 relative.
"""
from __future__ import annotations

import sys
from typing import Dict

import numpy as np

import oracle as O

H_RTOL = 1e-5
TIE = 1e-4
MIN_SAME = 0.999
SCALE_RTOL = 1e-5
LOSS_RTOL = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def h_rel_err(H_gpu: np.ndarray, H_ref: np.ndarray) -> float:
    return float(np.linalg.norm(H_gpu.astype(np.float64) - H_ref) / np.linalg.norm(H_ref))


def group_index(n: int, group: int) -> np.ndarray:
    return np.zeros(n, dtype=np.int64) if group <= 0 else np.arange(n) // group


def compare_codes(q_gpu: np.ndarray, s_gpu: np.ndarray, z_gpu: np.ndarray, ref: Dict[str, np.ndarray],
                  group: int) -> Dict[str, float]:
    q_o, t, tz = ref["q"], ref["t"], ref["tz"]
    m, n = q_o.shape
    gidx = group_index(n, group)
    mism = q_gpu != q_o
    rows = np.where(mism.any(axis=1))[0]
    first = np.full(m, n, dtype=np.int64)
    unexcused = []
    for r in rows:
        p = int(np.argmax(mism[r]))
        first[r] = p
        near = O.boundary_distance(np.array([t[r, p]]))[0] < TIE or \
            O.boundary_distance(np.array([tz[r, gidx[p]]]))[0] < TIE
        if not near:
            unexcused.append((int(r), p, float(t[r, p]), int(q_gpu[r, p]), int(q_o[r, p])))
    # scales of groups starting at or before the first mismatch
    G = s_gpu.shape[1]
    gstart = np.zeros(G, dtype=np.int64) if group <= 0 else np.arange(G) * group
    ok_mask = gstart[None, :] <= first[:, None]
    srel = np.abs(s_gpu.astype(np.float64) - ref["s"]) / np.abs(ref["s"])
    zdiff = (z_gpu.astype(np.int64) != ref["z"].astype(np.int64))
    return {
        "same_frac": 1.0 - float(mism.mean()),
        "rows_diverged": int(len(rows)),
        "unexcused": unexcused,
        "scale_rel_max": float(srel[ok_mask].max()) if ok_mask.any() else 0.0,
        "zero_mismatch": int(zdiff[ok_mask].sum()),
    }


def assert_codes(rep: Dict[str, float], label: str = "", min_same: float = MIN_SAME) -> None:
    assert not rep["unexcused"], f"{label}: first mismatch not at a near-tie: {rep['unexcused'][:5]}"
    assert rep["same_frac"] >= min_same, f"{label}: only {rep['same_frac']:.5f} of codes identical"
    assert rep["scale_rel_max"] <= SCALE_RTOL, f"{label}: scale rel err {rep['scale_rel_max']:.3e}"


def loss_rel(W: np.ndarray, H: np.ndarray, q_gpu, s_gpu, z_gpu, ref, group) -> float:
    Wh_gpu = O.dequant_from(q_gpu, s_gpu, z_gpu, group)
    l_gpu = O.layer_loss(W, Wh_gpu, H)
    l_ora = O.layer_loss(W, ref["What"], H)
    if l_ora == 0.0:  # exactly representable weights: both sides must be (numerically) lossless
        scale = float(np.sum((np.asarray(W, np.float64) @ H) * W)) or 1.0
        return abs(l_gpu) / scale
    return abs(l_gpu - l_ora) / l_ora


def follow_check(q_gpu: np.ndarray, s_gpu: np.ndarray, z_gpu: np.ndarray, W: np.ndarray, U: np.ndarray,
                 bits: int, group: int, block, label: str = "") -> Dict[str, np.ndarray]:
    """The oracle's sweep on the same W and U, taking the GPU's rounding at
    near-ties only (within TIE steps of a boundary); every code and zero point
    must then match and every scale agree to SCALE_RTOL.  Returns that run."""
    ref = O.gptq_quantize(W, U, bits, group, block, follow=(q_gpu, z_gpu), tie=TIE)
    bad = np.argwhere(q_gpu != ref["q"])
    zbad = np.argwhere(z_gpu.astype(np.int64) != ref["z"].astype(np.int64))
    srel = float(np.max(np.abs(s_gpu.astype(np.float64) - ref["s"]) / np.abs(ref["s"]))) if ref["s"].size else 0.0
    say(f"  {label} followed {ref['followed']} near-tie decisions; codes differing after that {len(bad)}, "
        f"zero points {len(zbad)}, scale rel {srel:.2e}")
    if len(bad):
        r, c = bad[0]
        raise AssertionError(f"{label}: {len(bad)} codes differ away from near-ties; first at row {r} col {c}: "
                             f"gpu {q_gpu[r, c]} oracle {ref['q'][r, c]} (t = {ref['t'][r, c]:.6f})")
    assert not len(zbad), f"{label}: {len(zbad)} zero points differ away from near-ties, first {zbad[0]}"
    assert srel <= SCALE_RTOL, f"{label}: scale rel err {srel:.3e}"
    return ref
