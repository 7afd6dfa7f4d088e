"""Plain fp64 CPU oracle for GPTQ layer-wise second-order weight quantization.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct
reference that the GPU library is checked against.  Only the test suite, the
smoke check and the CPU-baseline leg of the benchmark may import it; the
library itself never does, and this module imports nothing from the library.

Everything is float64 numpy/scipy, written to be read against the pages that
describe the method.  Short names used in the citations below:

  [OBQ]     "Part 2: Adaptive Rounding: Optimal Brain Quantizer (OBQ)"
            (feed.roma.co.ke)
  [GPTQ]    "Part 3: Adaptive Rounding: GPTQ" (hello-fri-end.github.io)
  [SOQ]     the English blog post on GPTQ second-order quantization
            (hungho77.github.io, /hung/blog/gptq-second-order-quantization/)
  [SOQ-vi]  the Vietnamese edition of that post (/hung/vi/blog/...)
  [OptRot]  "OptRot: Mitigating Weight Outliers via Data-Free Rotations for
            Post-Training Quantization" (abstract and Figure 1)

Beyond the per-layer path, dequant_matmul is the runtime consumer of the
packed layer (weights unpacked and dequantized next to 16-bit activations),
hadamard_rotate is the fixed rotation applied before GPTQ that [OptRot]
uses as its baseline, and quantize_transformer_stack / quantize_mlp_stack
are the network-level loop
([GPTQ] "Algorithm GPTQ": one layer at a time, each layer's calibration
inputs taken from the network as quantized so far; [SOQ] "Calibration for a
multimodal or VLA backbone": later blocks see activations already changed by
the earlier quantized blocks).

Readings taken where the pages are silent or disagree (each is also listed in
the design notes):

  R1  H = 2 X X^T, unnormalised ([SOQ] "The objective is layer output";
      [SOQ-vi] "Objective").  Codes do not depend on this scale because the
      damping is relative.
  R2  lambda = damp * mean(diag H) of the undamped H, added once to every
      diagonal entry ([SOQ] "3. Cholesky reformulation").
  R3  The factor read row by row is the UPPER U with H_d^{-1} = U^T U; row p of
      U covers columns >= p, which is what compensating later columns needs
      ([GPTQ] "Observation 3"; [SOQ-vi] writes the flush as E R[B, B:]).
  R4  Signs: e_p = (v_p - what_p) / U_pp and V <- V - e U[p, :].  This is the
      loss-minimising update of [GPTQ] "Observation 3" / [OBQ] "Generalized
      Weight Update" written with U; the flush in [GPTQ] "Algorithm GPTQ"
      stores the opposite sign in E, which taken literally pushes weights the
      wrong way.
  R5  Quantizer ([GPTQ] summary table "Asymmetric uniform"; [SOQ]
      "Group-wise quantization"): x_lo = min(0, min v), x_hi = max(0, max v),
      s = (x_hi - x_lo) / maxq, z = rint(-x_lo / s), q = clip(rint(v/s) + z,
      0, maxq), what = s (q - z).  A group whose values are all zero (empty
      range) uses x_hi = 1 (s = 1/maxq, z = 0), so its codes are exact zeros.
  R6  Rounding is round-half-to-even (IEEE rint).
  R7  Group parameters are taken when the sweep reaches the group's first
      column, from the current (already compensated) values of that group;
      per-row parameters (group <= 0) come from the original row.
  R8  Columns are swept left to right ([GPTQ] "Observation 1").
  R9  Block size and group size must nest (group % block == 0 or
      block % group == 0); the last block and group may be short.
  R12 The fixed rotation is R = blockdiag(H_b, ..., H_b) / sqrt(b), H_b the
      Sylvester-ordered Hadamard matrix of order b (a power of two dividing
      the row length); rows are rotated as M <- M R.  With W' = W R and
      X' = X R the layer output is unchanged (X' W'^T = X W^T, R orthogonal),
      so R folds into the previous layer and costs nothing at run time
      ([OptRot] Figure 1, "fusible" rotations); H' = 2 X'^T X' = R^T H R.
      Weight incoherence (the quantity [OptRot] Theorem 3.1 bounds the error
      with) is read as mu_W = sqrt(m n) max |W_ij| / ||W||_F.
  R13 The network the loop runs through is a stack of transformer blocks
      shaped like a 7B model's, without normalisation (the pages fix neither
      the block nor its norms):
        x <- x + W_o attn(W_q x, W_k x, W_v x)
        x <- x + W_down (silu(W_gate x) * (W_up x)),  silu(v) = v / (1 + e^-v)
      attn is causal multi-head softmax attention over sequences of
      consecutive tokens, head h the columns [h dh, (h+1) dh), scores scaled
      by 1/sqrt(dh).  q, k and v share one Hessian (same input) and are swept
      as one stacked layer, as are gate and up; o and down get their own from
      the attention output and the hidden activations.  quantize_mlp_stack is
      the same loop over MLP blocks alone.
  R16 Activation precision in the network loop: the GPU network stores every
      activation in fp16 (each a single rounding of an fp32 result), so the
      oracle network can round the same values at the same points
      (act_dtype="f16"); its arithmetic between the roundings stays fp64.
  R14 OBQ's greedy order ([OBQ] "Greedy Search"; the loss-increase formula
      there is lost from the text): the score of an unquantized weight p is
      dL_p = (what_p - w_p)^2 / [H^-1]_pp with what_p its rounding on the grid
      (OBS's factor 1/2 dropped: it moves no argmin), H^-1 = U^T U from the
      same upper factor the fixed-order sweep reads, and equal scores go to
      the smaller column index.  Because the order jumps across groups, every
      group's (or the row's) grid is fixed once from the ORIGINAL weights,
      before any compensation (R7 cannot apply: a group has no "first column
      reached").
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, Optional, Tuple

import numpy as np
import scipy.linalg
from scipy.linalg import lapack


# ----------------------------------------------------------------------------- Hessian and damping

def hessian(chunks: Iterable[np.ndarray]) -> np.ndarray:
    """H = 2 X X^T with X the [n x tokens] calibration inputs, given here as
    token-major chunks [tokens_c x n] ([SOQ] "The objective is layer output":
    the Hessian of ||WX - What X||^2 is 2XX^T; [OBQ] "Goal": the input
    covariance stands in for the true Hessian).  fp64, both triangles."""
    H = None
    for c in chunks:
        c = np.asarray(c, dtype=np.float64)
        G = c.T @ c
        H = G if H is None else H + G
    return 2.0 * H


def damp(H: np.ndarray, rel: float) -> Tuple[np.ndarray, float]:
    """H_d = H + lambda I with lambda = rel * mean(diag H) ([SOQ] "3. Cholesky
    reformulation": about one percent of the average Hessian diagonal;
    [GPTQ] "Algorithm GPTQ": H = XX^T + lambda I)."""
    lam = float(rel) * float(np.mean(np.diag(H)))
    Hd = np.array(H, dtype=np.float64, copy=True)
    Hd[np.diag_indices_from(Hd)] += lam
    return Hd, lam


# ----------------------------------------------------------------------------- inverse-Hessian factor

def inverse_cholesky_upper(Hd: np.ndarray) -> Tuple[Optional[np.ndarray], int]:
    """U upper-triangular with H_d^{-1} = U^T U ([GPTQ] "Observation 3": factor
    the inverse once, then read its rows; reading R3).

    Steps as stated: Cholesky of H_d, the inverse from that factor, then the
    Cholesky of the inverse.  Returns (U, 0), or (None, k) when the k-th
    (1-based) leading minor of H_d is not positive definite."""
    L, info = lapack.dpotrf(np.asarray(Hd, dtype=np.float64), lower=1, clean=1)
    if info != 0:
        return None, int(info)
    G, info = lapack.dpotri(L, lower=1)
    if info != 0:
        return None, int(info)
    G = np.tril(G) + np.tril(G, -1).T
    U, info = lapack.dpotrf(G, lower=0, clean=1)
    if info != 0:
        return None, int(info)
    return np.triu(U), 0


# ----------------------------------------------------------------------------- quantizer

def maxq_of(bits: int) -> int:
    return (1 << int(bits)) - 1


def quant_params(v: np.ndarray, bits: int) -> Tuple[np.ndarray, np.ndarray]:
    """Asymmetric min/max scale and integer zero point per row of v [rows x k]
    (reading R5).  Returns s [rows] (float64) and z [rows] (float64 holding
    integers)."""
    v = np.asarray(v, dtype=np.float64)
    maxq = maxq_of(bits)
    lo = np.minimum(v.min(axis=1), 0.0)
    hi = np.maximum(v.max(axis=1), 0.0)
    empty = hi == lo
    hi = np.where(empty, 1.0, hi)
    lo = np.where(empty, 0.0, lo)
    s = (hi - lo) / maxq
    z = np.rint(-lo / s)
    return s, z


def quantize(v: np.ndarray, s: np.ndarray, z: np.ndarray, bits: int) -> np.ndarray:
    """q = clip(rint(v/s) + z, 0, maxq) (reading R5, R6); integer codes."""
    t = np.asarray(v, dtype=np.float64) / s
    return np.clip(np.rint(t) + z, 0, maxq_of(bits)).astype(np.int64)


def dequantize(q: np.ndarray, s: np.ndarray, z: np.ndarray) -> np.ndarray:
    return s * (np.asarray(q, dtype=np.float64) - z)


def n_groups(n: int, group: int) -> int:
    return 1 if group <= 0 else (n + group - 1) // group


def check_schedule(n: int, group: int, block: int) -> None:
    if block < 1:
        raise ValueError("block must be >= 1")
    if group > 0 and not (group % block == 0 or block % group == 0):
        raise ValueError("group and block sizes must nest (reading R9)")


# ----------------------------------------------------------------------------- the sweep

def gptq_quantize(W: np.ndarray, U: np.ndarray, bits: int, group: int, block: Optional[int],
                  follow: Optional[Tuple[np.ndarray, np.ndarray]] = None, tie: float = 0.0) -> Dict[str, np.ndarray]:
    """GPTQ's column sweep over one layer ([GPTQ] "Algorithm GPTQ"; [SOQ-vi]
    "Lazy batch update").

    block=None runs the definition: after each column every later column is
    compensated at once.  block=B runs the pages' lazy schedule: within a
    block of B columns the compensation touches only the block, and the
    accumulated scaled errors E are flushed to all later columns by one
    matrix product V[:, i2:] -= E U[i:i2, i2:] when the block ends.  Both give
    the same result up to the order of floating-point sums.

    Per column p (readings R3-R8):
      at a group start: (s, z) from the current V[:, p:p+group]
      q = clip(rint(V_p / s) + z, 0, maxq);  what = s (q - z)
      e = (V_p - what) / U_pp                   (the scaled error kept in E)
      V[:, later] -= e U[p, later]              ([OBQ] "Generalized Weight Update":
                                                 delta_rem = delta_p (H^-1)_{p,rem}/(H^-1)_pp,
                                                 read from row p of U)

    follow = (q_other, z_other), tie = d compares against a sweep that rounds
    in another precision: wherever this sweep's own pre-rounding value (V_p/s,
    or -x_lo/s for a zero point) lies within d steps of a rounding boundary
    and the other side's code or zero point is one of the two roundings next
    to that boundary, this sweep takes the other side's choice (both are
    correct roundings of a value the two precisions place on different sides
    of the boundary; every later column of the row depends on which one was
    taken).  Nothing else changes; "followed" counts the decisions taken over
    that differ from this sweep's own.

    Returns q [m x n] int64, s and z [m x G], E [m x n], What [m x n],
    t [m x n] = V_p / s (pre-rounding value in steps) and tz [m x G] = -x_lo/s
    (pre-rounding zero point), err_sq [m] = sum_p e_p^2, followed (int)."""
    V = np.array(W, dtype=np.float64, copy=True)
    m, n = V.shape
    if U.shape != (n, n):
        raise ValueError("U must be n x n")
    B = n if block is None else int(block)
    if block is not None:
        check_schedule(n, group, B)
    G = n_groups(n, group)
    q = np.zeros((m, n), dtype=np.int64)
    E = np.zeros((m, n))
    T = np.zeros((m, n))
    S = np.zeros((m, G))
    Z = np.zeros((m, G))
    TZ = np.zeros((m, G))
    maxq = maxq_of(bits)
    if follow is not None:
        fq = np.asarray(follow[0]).astype(np.int64)
        fz = np.asarray(follow[1]).astype(np.int64)
        if fq.shape != (m, n) or fz.shape != (m, G):
            raise ValueError("follow codes must be m x n and zero points m x G")
    followed = 0

    def take_over(own: np.ndarray, pre: np.ndarray, below: np.ndarray, above: np.ndarray,
                  other: np.ndarray) -> np.ndarray:
        """own decision, or the other side's where pre is a near-tie and the
        other side chose one of the two roundings next to it (below, above)."""
        nonlocal followed
        near = boundary_distance(pre) < tie
        ok = near & ((other == below) | (other == above)) & (other != own)
        followed += int(ok.sum())
        return np.where(ok, other, own)

    def take_params(p: int, g_idx: int, vals: np.ndarray):
        s, z = quant_params(vals, bits)
        lo = np.minimum(vals.min(axis=1), 0.0)
        TZ[:, g_idx] = -lo / s
        if follow is not None:
            fl = np.floor(TZ[:, g_idx]).astype(np.int64)
            z = take_over(z.astype(np.int64), TZ[:, g_idx], fl, fl + 1, fz[:, g_idx]).astype(np.float64)
        S[:, g_idx], Z[:, g_idx] = s, z

    if group <= 0:
        take_params(0, 0, V)
    for i in range(0, n, B):
        i2 = min(i + B, n)
        for p in range(i, i2):
            if group > 0 and p % group == 0:
                take_params(p, p // group, V[:, p:min(p + group, n)])
            gi = 0 if group <= 0 else p // group
            s, z = S[:, gi], Z[:, gi]
            T[:, p] = V[:, p] / s
            q[:, p] = np.clip(np.rint(T[:, p]) + z, 0, maxq).astype(np.int64)
            if follow is not None:
                below = np.clip(np.floor(T[:, p]) + z, 0, maxq).astype(np.int64)
                above = np.clip(np.floor(T[:, p]) + 1 + z, 0, maxq).astype(np.int64)
                q[:, p] = take_over(q[:, p], T[:, p], below, above, fq[:, p])
            what = s * (q[:, p] - z)
            e = (V[:, p] - what) / U[p, p]
            E[:, p] = e
            end = n if block is None else i2
            V[:, p + 1:end] -= np.outer(e, U[p, p + 1:end])
        if block is not None and i2 < n:
            V[:, i2:] -= E[:, i:i2] @ U[i:i2, i2:]
    gidx = np.zeros(n, dtype=np.int64) if group <= 0 else np.arange(n) // group
    What = S[:, gidx] * (q - Z[:, gidx])
    return {"q": q, "s": S, "z": Z, "E": E, "What": What, "t": T, "tz": TZ,
            "err_sq": np.sum(E * E, axis=1), "followed": followed}


def obs_step(v_row: np.ndarray, U: np.ndarray, p: int, what_p: float) -> np.ndarray:
    """One compensation step on a single row: fix column p to what_p and move
    the later columns by the optimal amount ([OBQ] "Generalized Weight
    Update"), using row p of U (reading R3/R4).  Returns the new row."""
    v = np.array(v_row, dtype=np.float64, copy=True)
    e = (v[p] - what_p) / U[p, p]
    v[p] = what_p
    v[p + 1:] -= e * U[p, p + 1:]
    return v


# ----------------------------------------------------------------------------- two slower routes to the same sweep (cross-checks)

def gptq_quantize_obs(W: np.ndarray, Hd: np.ndarray, bits: int, group: int) -> Dict[str, np.ndarray]:
    """The same fixed-order sweep driven by an explicit inverse Hessian and its
    rank-one downdate after each column ([OBQ] "The OBS / GPTQ Trick";
    [GPTQ] "Observation 3": H^-1_{-p} = H^-1 - H^-1_{:,p} H^-1_{p,:} / (H^-1)_pp),
    with the update delta_rem = delta_p (H^-1)_{p,rem} / (H^-1)_pp.
    O(n^3); for small n only."""
    V = np.array(W, dtype=np.float64, copy=True)
    m, n = V.shape
    Hinv = np.linalg.inv(np.asarray(Hd, dtype=np.float64))
    q = np.zeros((m, n), dtype=np.int64)
    G = n_groups(n, group)
    S = np.zeros((m, G))
    Z = np.zeros((m, G))
    if group <= 0:
        S[:, 0], Z[:, 0] = quant_params(V, bits)
    for p in range(n):
        if group > 0 and p % group == 0:
            S[:, p // group], Z[:, p // group] = quant_params(V[:, p:p + group], bits)
        gi = 0 if group <= 0 else p // group
        q[:, p] = quantize(V[:, p], S[:, gi], Z[:, gi], bits)
        delta = dequantize(q[:, p], S[:, gi], Z[:, gi]) - V[:, p]     # what_p - w_p
        V[:, p + 1:] += np.outer(delta, Hinv[p, p + 1:] / Hinv[p, p])
        V[:, p] += delta
        Hinv = Hinv - np.outer(Hinv[:, p], Hinv[p, :]) / Hinv[p, p]
    return {"q": q, "s": S, "z": Z, "V": V}


def gptq_quantize_naive(W: np.ndarray, Hd: np.ndarray, bits: int, group: int) -> Dict[str, np.ndarray]:
    """The same sweep re-inverting the Hessian of the not-yet-quantized
    columns at every step (the naive procedure of [OBQ] "The OBS / GPTQ
    Trick").  O(n^4); for tiny n only."""
    V = np.array(W, dtype=np.float64, copy=True)
    m, n = V.shape
    q = np.zeros((m, n), dtype=np.int64)
    G = n_groups(n, group)
    S = np.zeros((m, G))
    Z = np.zeros((m, G))
    if group <= 0:
        S[:, 0], Z[:, 0] = quant_params(V, bits)
    for p in range(n):
        if group > 0 and p % group == 0:
            S[:, p // group], Z[:, p // group] = quant_params(V[:, p:p + group], bits)
        gi = 0 if group <= 0 else p // group
        q[:, p] = quantize(V[:, p], S[:, gi], Z[:, gi], bits)
        delta = dequantize(q[:, p], S[:, gi], Z[:, gi]) - V[:, p]
        Ginv = np.linalg.inv(np.asarray(Hd, dtype=np.float64)[p:, p:])
        V[:, p + 1:] += np.outer(delta, Ginv[0, 1:] / Ginv[0, 0])
        V[:, p] += delta
    return {"q": q, "s": S, "z": Z, "V": V}


def obq_greedy(W: np.ndarray, U: np.ndarray, bits: int, group: int,
               follow: Optional[Tuple[Optional[np.ndarray], Optional[np.ndarray], Optional[np.ndarray]]] = None,
               tie: float = 0.0, order_tie: Optional[float] = None) -> Dict[str, np.ndarray]:
    """OBQ's greedy-order quantization of each row ([OBQ] "Greedy Search",
    "The OBS / GPTQ Trick", "Generalized Weight Update"; reading R14).

    Each row runs on its own copy of H^-1 = U^T U.  At every step, among the
    row's unquantized weights, the one whose rounding adds the least to the
    proxy loss, dL_p = (what_p - w_p)^2 / [H^-1]_pp, is quantized; the rest
    move by (what_p - w_p) [H^-1]_{p,rem} / [H^-1]_pp, and the row's H^-1
    loses weight p by the rank-one downdate H^-1 - H^-1_{:,p} H^-1_{p,:} /
    [H^-1]_pp.  The grid of every group is fixed from the original row.

    follow = (q_other, z_other, order_other) (each may be None) and tie,
    order_tie compare against a run in another precision: a rounding or zero
    point within `tie` steps of a boundary takes the other side's adjacent
    choice (as in gptq_quantize); at a step where the other side quantized
    column g and g is still unquantized here, g is taken instead of this run's
    own pick k when sqrt(dL_g) <= sqrt(dL_k) + order_tie (s_g / sqrt([H^-1]_gg)
    + s_k / sqrt([H^-1]_kk)), i.e. when the two scores agree to order_tie grid
    steps in sqrt-loss units.  order_tie defaults to tie.

    Returns q [m x n] int64 codes, s, z [m x G], order [m x n] (column
    quantized at each step), loss [m] = sum of the chosen dL, What [m x n],
    followed (decisions taken over that differ from this run's own),
    order_margin (largest followed sqrt-loss gap in the units above)."""
    W = np.asarray(W, dtype=np.float64)
    m, n = W.shape
    U = np.asarray(U, dtype=np.float64)
    if U.shape != (n, n):
        raise ValueError("U must be n x n")
    Hinv0 = U.T @ U
    G = n_groups(n, group)
    gcol = np.zeros(n, dtype=np.int64) if group <= 0 else np.arange(n) // group
    maxq = maxq_of(bits)
    S = np.zeros((m, G))
    Z = np.zeros((m, G))
    otie = tie if order_tie is None else order_tie
    fq = fz = fo = None
    if follow is not None:
        fq, fz, fo = follow
    followed = 0
    margin = 0.0
    for g in range(G):
        cols = np.arange(n) if group <= 0 else np.arange(g * group, min((g + 1) * group, n))
        s, z = quant_params(W[:, cols], bits)
        if fz is not None:
            tz = -np.minimum(W[:, cols].min(axis=1), 0.0) / s
            near = boundary_distance(tz) < tie
            other = np.asarray(fz)[:, g].astype(np.int64)
            fl = np.floor(tz).astype(np.int64)
            ok = near & ((other == fl) | (other == fl + 1)) & (other != z)
            followed += int(ok.sum())
            z = np.where(ok, other, z)
        S[:, g], Z[:, g] = s, z
    q = np.zeros((m, n), dtype=np.int64)
    order = np.zeros((m, n), dtype=np.int64)
    loss = np.zeros(m)
    for r in range(m):
        w = W[r].copy()
        Hi = Hinv0.copy()
        active = np.ones(n, dtype=bool)
        sr, zr = S[r, gcol], Z[r, gcol]
        for step in range(n):
            idx = np.flatnonzero(active)
            d = np.diag(Hi)[idx]
            qc = np.clip(np.rint(w[idx] / sr[idx]) + zr[idx], 0, maxq)
            err = sr[idx] * (qc - zr[idx]) - w[idx]
            score = err * err / d
            k = int(np.argmin(score))           # first minimum: smallest column
            if fo is not None and active[fo[r, step]]:
                kg = int(np.searchsorted(idx, fo[r, step]))
                rho = np.sqrt(score)
                unit = sr[idx] / np.sqrt(d)
                gap = (rho[kg] - rho[k]) / (unit[kg] + unit[k])
                if kg != k and gap <= otie:
                    followed += 1
                    margin = max(margin, gap)
                    k = kg
            p = int(idx[k])
            code = int(qc[k])
            if fq is not None:
                t = w[p] / sr[p]
                other = int(fq[r, p])
                lo_c = int(np.clip(np.floor(t) + zr[p], 0, maxq))
                hi_c = int(np.clip(np.floor(t) + 1 + zr[p], 0, maxq))
                if boundary_distance(np.array([t]))[0] < tie and other in (lo_c, hi_c) and other != code:
                    followed += 1
                    code = other
            what = sr[p] * (code - zr[p])
            delta = what - w[p]
            loss[r] += delta * delta / Hi[p, p]
            q[r, p] = code
            order[r, step] = p
            rem = active.copy()
            rem[p] = False
            w[rem] += delta * Hi[p, rem] / Hi[p, p]
            w[p] = what
            Hi = Hi - np.outer(Hi[:, p], Hi[p, :]) / Hi[p, p]
            active[p] = False
    What = S[:, gcol] * (q - Z[:, gcol])
    return {"q": q, "s": S, "z": Z, "order": order, "loss": loss, "What": What, "followed": followed,
            "order_margin": margin}


# ----------------------------------------------------------------------------- comparators and measures

def rtn(W: np.ndarray, bits: int, group: int) -> Dict[str, np.ndarray]:
    """Round-to-nearest with the same quantizer and parameters taken from the
    original weights, no compensation ([SOQ] "GPTQ in the method landscape")."""
    W = np.asarray(W, dtype=np.float64)
    m, n = W.shape
    G = n_groups(n, group)
    S = np.zeros((m, G))
    Z = np.zeros((m, G))
    if group <= 0:
        S[:, 0], Z[:, 0] = quant_params(W, bits)
    else:
        for g in range(G):
            S[:, g], Z[:, g] = quant_params(W[:, g * group:(g + 1) * group], bits)
    gidx = np.zeros(n, dtype=np.int64) if group <= 0 else np.arange(n) // group
    q = np.clip(np.rint(W / S[:, gidx]) + Z[:, gidx], 0, maxq_of(bits)).astype(np.int64)
    return {"q": q, "s": S, "z": Z, "What": S[:, gidx] * (q - Z[:, gidx])}


def dequant_from(q: np.ndarray, s: np.ndarray, z: np.ndarray, group: int) -> np.ndarray:
    n = q.shape[1]
    gidx = np.zeros(n, dtype=np.int64) if group <= 0 else np.arange(n) // group
    return np.asarray(s, np.float64)[:, gidx] * (q.astype(np.float64) - np.asarray(z, np.float64)[:, gidx])


def layer_loss(W: np.ndarray, What: np.ndarray, H: np.ndarray) -> float:
    """||W X - What X||_F^2 ([SOQ] "The objective is layer output"), evaluated
    as 1/2 tr(dW H dW^T) with the undamped H = 2 X X^T."""
    D = np.asarray(W, dtype=np.float64) - np.asarray(What, dtype=np.float64)
    return 0.5 * float(np.sum((D @ np.asarray(H, dtype=np.float64)) * D))


def layer_loss_direct(W: np.ndarray, What: np.ndarray, X_tokens: np.ndarray) -> float:
    """||(W - What) X||_F^2 with X given token-major [tokens x n]."""
    D = np.asarray(W, dtype=np.float64) - np.asarray(What, dtype=np.float64)
    Y = np.asarray(X_tokens, dtype=np.float64) @ D.T
    return float(np.sum(Y * Y))


# ----------------------------------------------------------------------------- packed code layout

def packed_words(n: int, bits: int) -> int:
    return (n * bits + 31) // 32


def pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """Per row, a little-endian bit-stream of b-bit codes: code j occupies bits
    [j*b, (j+1)*b) counted from bit 0 of the row's first uint32 word; a code
    may straddle two words."""
    q = np.asarray(q, dtype=np.uint64)
    m, n = q.shape
    W = packed_words(n, bits)
    acc = np.zeros((m, W + 1), dtype=np.uint64)
    for j in range(n):
        bit = j * bits
        w, off = divmod(bit, 32)
        acc[:, w] |= (q[:, j] << np.uint64(off))
    lo = acc & np.uint64(0xFFFFFFFF)
    carry = acc >> np.uint64(32)
    lo[:, 1:] |= carry[:, :-1]
    return lo[:, :W].astype(np.uint32)


def unpack_codes(words: np.ndarray, bits: int, n: int) -> np.ndarray:
    """Inverse of pack_codes: [m x words] uint32 -> [m x n] int64 codes."""
    words = np.asarray(words, dtype=np.uint64)
    m = words.shape[0]
    ext = np.concatenate([words, np.zeros((m, 1), dtype=np.uint64)], axis=1)
    mask = np.uint64((1 << bits) - 1)
    out = np.zeros((m, n), dtype=np.int64)
    for j in range(n):
        bit = j * bits
        w, off = divmod(bit, 32)
        both = ext[:, w] | (ext[:, w + 1] << np.uint64(32))
        out[:, j] = ((both >> np.uint64(off)) & mask).astype(np.int64)
    return out


# ----------------------------------------------------------------------------- runtime use of the packed layer

def dequant_matmul(X: np.ndarray, words: np.ndarray, s: np.ndarray, z: np.ndarray, bits: int, group: int,
                   n: int) -> np.ndarray:
    """Y = X What^T, [tokens x m], for a packed layer.

    The weight-only path keeps activations in 16-bit floats; at run time the
    packed b-bit weights are unpacked and dequantized, What = s (q - z) (R5),
    and multiplied with the activations ([SOQ] "What the original results
    established": speed comes from moving fewer weight bytes and unpacking
    them efficiently; [SOQ-vi] closing paragraph: the artifact still needs a
    packed INT4 kernel for the target device).  X [tokens x n] is taken
    exactly as given; words, s, z are the layer outputs of quantize_layer.
    fp64 throughout."""
    q = unpack_codes(words, bits, n)
    What = dequant_from(q, s, z, group)
    return np.asarray(X, dtype=np.float64) @ What.T


# ----------------------------------------------------------------------------- whole layer

def quantize_layer_from_x(W: np.ndarray, x_chunks: Iterable[np.ndarray], bits: int, group: int, block: int,
                          rel_damp: float = 0.01) -> Dict[str, object]:
    """The per-layer pipeline of [GPTQ] "Algorithm GPTQ" for one layer:
    H from X, damping, the inverse factor, then the blocked sweep."""
    H = hessian(x_chunks)
    Hd, lam = damp(H, rel_damp)
    U, info = inverse_cholesky_upper(Hd)
    if info != 0:
        raise np.linalg.LinAlgError(f"damped Hessian not positive definite at column {info}")
    out = gptq_quantize(W, U, bits, group, block)
    out.update({"H": H, "lam": lam, "U": U})
    return out


def boundary_distance(t: np.ndarray) -> np.ndarray:
    """Distance (in quantization steps) of a pre-rounding value to the nearest
    rounding boundary k + 1/2."""
    return np.abs(t - (np.floor(t) + 0.5))


# ----------------------------------------------------------------------------- fixed rotation before GPTQ

def hadamard_matrix(b: int) -> np.ndarray:
    """Sylvester-ordered Hadamard matrix of order b (a power of two):
    H_1 = [1], H_2k = [[H_k, H_k], [H_k, -H_k]] (reading R12)."""
    if b < 1 or b & (b - 1):
        raise ValueError("order must be a power of two")
    Hm = np.ones((1, 1))
    while Hm.shape[0] < b:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    return Hm


def default_rotation_block(n: int) -> int:
    """The largest power of two dividing n, at most 4096."""
    b = 1
    while n % (2 * b) == 0 and 2 * b <= 4096:
        b *= 2
    return b


def hadamard_rotate(M: np.ndarray, block: int = 0) -> np.ndarray:
    """M R with R = blockdiag(H_b, ..., H_b) / sqrt(b) over the columns of M
    (reading R12; [OptRot] abstract and Figure 1: a fixed, fusible rotation
    applied before GPTQ to spread weight outliers).  block <= 0 takes the
    largest power of two dividing the row length (at most 4096)."""
    M = np.asarray(M, dtype=np.float64)
    rows, n = M.shape
    b = default_rotation_block(n) if block <= 0 else int(block)
    if b & (b - 1) or n % b:
        raise ValueError("block must be a power of two dividing the row length")
    R = hadamard_matrix(b) / math.sqrt(b)
    return (M.reshape(rows, n // b, b) @ R).reshape(rows, n)


def weight_incoherence(W: np.ndarray) -> float:
    """mu_W = sqrt(m n) max |W_ij| / ||W||_F (reading R12)."""
    W = np.asarray(W, dtype=np.float64)
    return float(math.sqrt(W.size) * np.max(np.abs(W)) / np.linalg.norm(W))


# ----------------------------------------------------------------------------- the network-level loop

def silu(v: np.ndarray) -> np.ndarray:
    """v / (1 + e^-v) (reading R13)."""
    v = np.asarray(v, dtype=np.float64)
    return v / (1.0 + np.exp(-v))


def swiglu(G: np.ndarray, Uo: np.ndarray) -> np.ndarray:
    """silu(G) * Uo, the hidden activations of an MLP block (reading R13)."""
    return silu(G) * np.asarray(Uo, dtype=np.float64)


def quantize_mlp_stack(blocks, X0: np.ndarray, bits: int, group: int, block: int, damp_rel: float):
    """Quantize a stack of MLP blocks one layer at a time, each layer's
    calibration inputs computed by the network as quantized so far ([GPTQ]
    "Algorithm GPTQ"; [SOQ] "Calibration for a multimodal or VLA backbone";
    the block of reading R13).  blocks: list of (W_gate [f x d], W_up [f x d],
    W_down [d x f]).  Per block: H from X, gate and up quantized with its
    factor; A = swiglu(X What_gate^T, X What_up^T); H from A, down quantized;
    X <- X + A What_down^T.  Returns a list of dicts (the three sweeps' outputs
    plus the block's inputs X and A) and the final X."""
    X = np.asarray(X0, dtype=np.float64)
    out = []
    for Wg, Wu, Wd in blocks:
        H = hessian([X])
        U, info = inverse_cholesky_upper(damp(H, damp_rel)[0])
        if info:
            raise ValueError("block input Hessian not positive definite")
        rg = gptq_quantize(np.asarray(Wg, np.float64), U, bits, group, block)
        ru = gptq_quantize(np.asarray(Wu, np.float64), U, bits, group, block)
        A = swiglu(X @ rg["What"].T, X @ ru["What"].T)
        H2 = hessian([A])
        U2, info = inverse_cholesky_upper(damp(H2, damp_rel)[0])
        if info:
            raise ValueError("hidden-activation Hessian not positive definite")
        rd = gptq_quantize(np.asarray(Wd, np.float64), U2, bits, group, block)
        out.append({"gate": rg, "up": ru, "down": rd, "X": X, "A": A, "U": U, "U2": U2})
        X = X + A @ rd["What"].T
    return out, X


# ----------------------------------------------------------------------------- transformer blocks

def attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, seq_len: int, heads: int) -> np.ndarray:
    """Causal multi-head softmax attention (reading R13): for every sequence of
    seq_len consecutive tokens and every head h (columns [h dh, (h+1) dh)),
    O_i = sum_{j <= i} softmax_j(Q_i . K_j / sqrt(dh)) V_j.  fp64."""
    Q, K, V = (np.asarray(a, dtype=np.float64) for a in (Q, K, V))
    T, dm = Q.shape
    dh = dm // heads
    O = np.zeros_like(Q)
    mask = np.tril(np.ones((seq_len, seq_len), dtype=bool))
    for s0 in range(0, T, seq_len):
        for h in range(heads):
            c = slice(h * dh, (h + 1) * dh)
            S = Q[s0:s0 + seq_len, c] @ K[s0:s0 + seq_len, c].T / math.sqrt(dh)
            S = np.where(mask, S, -np.inf)
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            O[s0:s0 + seq_len, c] = P @ V[s0:s0 + seq_len, c]
    return O


def attention_error_bound(Q, K, V, O, seq_len: int, heads: int) -> np.ndarray:
    """Per-element bound on how far an fp32 computation of attention(Q, K, V)
    can be from O (exact products of 16-bit inputs; an fp32 dot product of dh
    terms errs by at most (dh + 16) 2^-24 sum_d |q_d k_d| / sqrt(dh) in a
    score, which moves output i by at most sum_j p_ij d_ij |v_j - O_i|; the
    exponentials, the normalisation and the weighted sum add a few relative
    2^-24 of sum_j p_ij |v_j|)."""
    Q, K, V, O = (np.asarray(a, dtype=np.float64) for a in (Q, K, V, O))
    T, dm = Q.shape
    dh = dm // heads
    B = np.zeros_like(Q)
    mask = np.tril(np.ones((seq_len, seq_len), dtype=bool))
    for s0 in range(0, T, seq_len):
        for h in range(heads):
            c = slice(h * dh, (h + 1) * dh)
            S = Q[s0:s0 + seq_len, c] @ K[s0:s0 + seq_len, c].T / math.sqrt(dh)
            S = np.where(mask, S, -np.inf)
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            Dsc = (dh + 16) * 2.0 ** -24 * (np.abs(Q[s0:s0 + seq_len, c]) @ np.abs(K[s0:s0 + seq_len, c]).T) \
                / math.sqrt(dh)
            PD = P * Dsc
            Va = np.abs(V[s0:s0 + seq_len, c])
            B[s0:s0 + seq_len, c] = PD @ Va + PD.sum(axis=1, keepdims=True) * np.abs(O[s0:s0 + seq_len, c]) \
                + 2.0 ** -21 * (P @ Va)
    return B + 2.0 ** -40


def round_activations(y: np.ndarray, act_dtype: Optional[str], other: Optional[np.ndarray] = None,
                      tol: Optional[np.ndarray] = None) -> Tuple[np.ndarray, int]:
    """Round fp64 values to the activation dtype (reading R16; round to
    nearest even), or keep them when act_dtype is None.  other, tol compare
    against a network that computes the values in another precision, with an
    error of at most tol: where the other side stored the rounding of some
    value within tol of y (fp16(y - tol) <= other <= fp16(y + tol); rounding
    is monotone), its value is taken (it is a correct rounding of a result the
    other precision may produce; everything downstream depends on it).
    Returns (values, number of values taken over that differ from the own
    rounding)."""
    y = np.asarray(y, dtype=np.float64)
    if act_dtype is None:
        return y, 0
    if act_dtype != "f16":
        raise ValueError("only fp16 activations are modelled")
    own = y.astype(np.float16)
    if other is None:
        return own.astype(np.float64), 0
    g = np.asarray(other).astype(np.float16)
    t = np.asarray(tol, dtype=np.float64)
    lo = (y - t).astype(np.float16)
    hi = (y + t).astype(np.float16)
    ok = (g >= lo) & (g <= hi) & (g != own)
    return np.where(ok, g, own).astype(np.float64), int(ok.sum())


def _matmul_tol(X: np.ndarray, What: np.ndarray) -> np.ndarray:
    """Bound on an fp32 computation of X What^T with exact products: a sum of K
    terms, each rounding relative 2^-24 of a partial sum of at most sum |x w|."""
    K = X.shape[1]
    return 2.0 ** -24 * (K + 64) * (np.abs(X) @ np.abs(What).T)


def quantize_transformer_stack(blocks, X0: np.ndarray, seq_len: int, heads: int, bits: int, group: int,
                               block: int, damp_rel: float, act_dtype: Optional[str] = None,
                               follow=None, tie: float = 0.0):
    """The network-level loop over transformer blocks (reading R13; [GPTQ]
    "Algorithm GPTQ": one layer at a time, each layer's calibration inputs
    computed by the network as quantized so far).  blocks: list of (W_q, W_k,
    W_v, W_o, W_gate, W_up, W_down).  Per block: H of x, q/k/v swept as one
    stacked layer with its factor; QKV = x What_qkv^T; A = attention; H of A,
    o swept; x += A What_o^T; H of x, gate/up swept together; A2 = swiglu; H of
    A2, down swept; x += A2 What_down^T.

    act_dtype="f16" rounds every activation where a 16-bit network stores it
    (reading R16).  follow (one dict per block with that network's "QKV", "A",
    "Yo", "X_mid", "GU", "A2", "Yd", "X_out" and the (q, z) of its four sweeps
    "qkv", "o", "gate_up", "down") and tie compare against such a network: its
    codes and zero points are taken at near-ties (gptq_quantize's follow) and
    its activations where they are roundings of a value within the error
    bound of an fp32 computation of that value (round_activations).  Returns
    (per-block dicts, final x)."""
    X, _ = round_activations(X0, act_dtype)
    out = []
    for b, (Wq, Wk, Wv, Wo, Wg, Wu, Wd) in enumerate(blocks):
        fb = follow[b] if follow is not None else {}
        rec = {"X": X, "followed_act": 0}

        def act(name, y, tol):
            v, k = round_activations(y, act_dtype, fb.get(name), tol)
            rec["followed_act"] += k
            rec[name] = v
            return v

        def sweep(W, Xin, name):
            H = hessian([Xin])
            U, info = inverse_cholesky_upper(damp(H, damp_rel)[0])
            if info:
                raise ValueError(f"{name}: Hessian not positive definite")
            fq = fb.get(name)
            r = gptq_quantize(np.asarray(W, np.float64), U, bits, group, block, follow=fq,
                              tie=tie if fq is not None else 0.0)
            rec[name] = r
            rec["U_" + name] = U
            return r

        d = X.shape[1]
        r = sweep(np.concatenate([Wq, Wk, Wv], axis=0), X, "qkv")
        QKV = act("QKV", X @ r["What"].T, _matmul_tol(X, r["What"]))
        Q, K_, V = QKV[:, :d], QKV[:, d:2 * d], QKV[:, 2 * d:]
        A0 = attention(Q, K_, V, seq_len, heads)
        A = act("A", A0, attention_error_bound(Q, K_, V, A0, seq_len, heads))
        r = sweep(Wo, A, "o")
        Yo = act("Yo", A @ r["What"].T, _matmul_tol(A, r["What"]))
        Xm = act("X_mid", X + Yo, 2.0 ** -23 * np.abs(X + Yo))
        r = sweep(np.concatenate([Wg, Wu], axis=0), Xm, "gate_up")
        GU = act("GU", Xm @ r["What"].T, _matmul_tol(Xm, r["What"]))
        f = np.asarray(Wg).shape[0]
        A2y = swiglu(GU[:, :f], GU[:, f:])
        A2 = act("A2", A2y, 2.0 ** -20 * np.abs(A2y) + 2.0 ** -40)
        r = sweep(Wd, A2, "down")
        Yd = act("Yd", A2 @ r["What"].T, _matmul_tol(A2, r["What"]))
        X = act("X_out", Xm + Yd, 2.0 ** -23 * np.abs(Xm + Yd))
        out.append(rec)
    return out, X
