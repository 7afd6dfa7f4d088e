"""Pins of the oracle's OBQ greedy-order variant (obq_greedy; [OBQ] "Greedy
Search", "The OBS / GPTQ Trick", "Generalized Weight Update"; reading R14).

The strongest pin re-derives every greedy decision from the definition on the
page: at each step, quantize the weight whose rounding increases the proxy
loss the least, the remaining weights re-optimized by solving the constrained
quadratic outright (no rank-one downdates, no OBS formulas)."""
import numpy as np
import pytest

import oracle as O


def _problem(m, n, seed, tokens=None, corr=0.7):
    """Rows of W and a correlated damped Hessian (tokens x n inputs with a
    shared component, so that compensation matters)."""
    rng = np.random.default_rng(seed)
    T = tokens or 4 * n
    base = rng.standard_normal((T, 1))
    X = corr * base + rng.standard_normal((T, n)) * np.linspace(0.5, 2.0, n)
    H = O.hessian([X])
    Hd, _ = O.damp(H, 0.01)
    U, info = O.inverse_cholesky_upper(Hd)
    assert info == 0
    W = rng.normal(0, 1.0, (m, n))
    return W, Hd, U


def _brute_greedy(w0, Hd, s_cols, z_cols, maxq):
    """Greedy order from its definition: f(v) = (v - w0)^T Hd (v - w0); with
    the quantized set Q fixed, the free weights sit at the constrained
    minimum; the next weight is the free one whose rounding (of its value at
    that minimum) raises the constrained minimum of f the least."""
    n = w0.size
    fixed = {}

    def optimum(fx):
        v = w0.copy()
        Q = sorted(fx)
        F = [j for j in range(n) if j not in fx]
        if Q:
            v[Q] = [fx[j] for j in Q]
            if F:
                v[F] = w0[F] - np.linalg.solve(Hd[np.ix_(F, F)], Hd[np.ix_(F, Q)] @ (v[Q] - w0[Q]))
        dv = v - w0
        return v, float(dv @ Hd @ dv)

    order, codes = [], np.zeros(n, dtype=np.int64)
    v, f0 = optimum(fixed)
    for _ in range(n):
        best = None
        for p in range(n):
            if p in fixed:
                continue
            c = int(np.clip(np.rint(v[p] / s_cols[p]) + z_cols[p], 0, maxq))
            val = s_cols[p] * (c - z_cols[p])
            _, f1 = optimum({**fixed, p: val})
            if best is None or f1 - f0 < best[0] - 1e-12 * max(1.0, abs(best[0])):
                best = (f1 - f0, p, c, val)
        _, p, c, val = best
        fixed[p] = val
        order.append(p)
        codes[p] = c
        v, f0 = optimum(fixed)
    return np.array(order), codes, f0


@pytest.mark.parametrize("n,group,bits,seed", [(5, 0, 3, 0), (6, 3, 2, 1), (7, 4, 4, 2), (6, 0, 2, 3)])
def test_greedy_matches_definition_by_brute_force(n, group, bits, seed):
    W, Hd, U = _problem(4, n, seed)
    res = O.obq_greedy(W, U, bits, group)
    gcol = np.zeros(n, dtype=np.int64) if group <= 0 else np.arange(n) // group
    for r in range(W.shape[0]):
        order, codes, f = _brute_greedy(W[r], Hd, res["s"][r, gcol], res["z"][r, gcol], O.maxq_of(bits))
        np.testing.assert_array_equal(res["order"][r], order)
        np.testing.assert_array_equal(res["q"][r], codes)
        assert res["loss"][r] == pytest.approx(f, rel=1e-9, abs=1e-12)


@pytest.mark.parametrize("n,group", [(24, 0), (32, 8), (40, 16)])
def test_loss_increments_sum_to_the_quadratic_form(n, group):
    """sum of the chosen dL_p = (w - what)^T H_d (w - what) per row: each
    step's OBS increase is exact, so the increments telescope."""
    W, Hd, U = _problem(6, n, 10 + n)
    res = O.obq_greedy(W, U, 4, group)
    D = W - res["What"]
    quad = np.einsum("ij,jk,ik->i", D, Hd, D)
    np.testing.assert_allclose(res["loss"], quad, rtol=1e-9)


def test_identity_hessian_is_rtn_in_error_order():
    """H^-1 = I: no weight moves, so the codes are round-to-nearest on the
    original grid and the order sorts the rounding errors (ties to the smaller
    column)."""
    rng = np.random.default_rng(5)
    W = rng.normal(0, 1, (5, 19))
    res = O.obq_greedy(W, np.eye(19), 3, 0)
    ref = O.rtn(W, 3, 0)
    np.testing.assert_array_equal(res["q"], ref["q"])
    err = (res["What"] - W) ** 2
    for r in range(5):
        np.testing.assert_array_equal(res["order"][r], np.lexsort((np.arange(19), err[r])))
    np.testing.assert_allclose(res["loss"], err.sum(axis=1), rtol=1e-12)


def test_fixed_order_reduces_to_the_obs_sweep():
    """Forcing the left-to-right order (per-row grid from the original row in
    both) gives exactly the fixed-order OBS sweep's codes."""
    W, Hd, U = _problem(8, 20, 7)
    forced = np.tile(np.arange(20), (8, 1))
    res = O.obq_greedy(W, U, 4, 0, follow=(None, None, forced), order_tie=np.inf)
    ref = O.gptq_quantize_obs(W, Hd, 4, 0)
    np.testing.assert_array_equal(res["order"], forced)
    np.testing.assert_array_equal(res["q"], ref["q"])
    np.testing.assert_allclose(res["s"], ref["s"], rtol=1e-15)


def test_first_pick_is_the_smallest_score_on_the_original_row():
    W, Hd, U = _problem(6, 16, 8)
    res = O.obq_greedy(W, U, 4, 0)
    Hinv = np.linalg.inv(Hd)
    s, z = res["s"][:, 0:1], res["z"][:, 0:1]
    what = s * (np.clip(np.rint(W / s) + z, 0, 15) - z)
    score = (what - W) ** 2 / np.diag(Hinv)
    np.testing.assert_array_equal(res["order"][:, 0], np.argmin(score, axis=1))


def test_order_is_a_permutation_and_grid_is_from_the_original_row():
    W, Hd, U = _problem(5, 24, 9)
    res = O.obq_greedy(W, U, 3, 8)
    for r in range(5):
        np.testing.assert_array_equal(np.sort(res["order"][r]), np.arange(24))
    s, z = O.quant_params(W[:, 8:16], 3)
    np.testing.assert_allclose(res["s"][:, 1], s, rtol=1e-15)
    np.testing.assert_array_equal(res["z"][:, 1], z)
    assert res["q"].min() >= 0 and res["q"].max() <= 7


def test_greedy_beats_fixed_order_on_a_correlated_layer():
    """The reason OBQ orders greedily: on a layer with strongly coupled
    inputs its proxy loss is below the fixed-order sweep's on the same grid
    (sum over rows; this seeded case has a clear margin)."""
    W, Hd, U = _problem(32, 48, 11, corr=2.0)
    g = O.obq_greedy(W, U, 3, 0)
    f = O.gptq_quantize_obs(W, Hd, 3, 0)
    Sg = np.repeat(f["s"], 48, axis=1)
    D = W - Sg * (f["q"] - np.repeat(f["z"], 48, axis=1))
    fixed_loss = np.einsum("ij,jk,ik->i", D, Hd, D).sum()
    assert g["loss"].sum() < fixed_loss


def test_follow_own_order_changes_nothing():
    W, Hd, U = _problem(4, 20, 12)
    a = O.obq_greedy(W, U, 4, 5)
    b = O.obq_greedy(W, U, 4, 5, follow=(a["q"], a["z"], a["order"]), tie=1e-4)
    assert b["followed"] == 0
    np.testing.assert_array_equal(a["q"], b["q"])
    np.testing.assert_array_equal(a["order"], b["order"])


def test_follow_takes_an_order_only_within_the_tolerance():
    """A swapped pair of picks is followed only when their scores agree to
    the given tolerance, and the followed run stays a valid greedy run from
    that point (loss identity still holds)."""
    W, Hd, U = _problem(3, 16, 13)
    a = O.obq_greedy(W, U, 4, 0)
    o = a["order"].copy()
    o[:, [0, 1]] = o[:, [1, 0]]
    strict = O.obq_greedy(W, U, 4, 0, follow=(None, None, o), order_tie=0.0)
    np.testing.assert_array_equal(strict["order"], a["order"])
    loose = O.obq_greedy(W, U, 4, 0, follow=(None, None, o), order_tie=10.0)
    np.testing.assert_array_equal(loose["order"][:, 0], o[:, 0])
    assert loose["followed"] >= 3
    D = W - loose["What"]
    np.testing.assert_allclose(loose["loss"], np.einsum("ij,jk,ik->i", D, Hd, D), rtol=1e-9)
