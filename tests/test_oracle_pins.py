"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test ties the oracle to something other than itself: hand-derived worked
examples (tests/golden), closed forms, an independent least-squares solve,
special cases that reduce to round-to-nearest, and exact algebraic identities.
A plausible mistake anywhere in the oracle (a dropped term, a flipped sign, a
transposed factor, a wrong group boundary) fails at least one of them.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import synth
from conftest import GOLDEN


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_layer(m, n, tokens, seed, corr=0.3):
    rng = np.random.default_rng(seed)
    W = rng.normal(0, 0.02, (m, n))
    M = np.eye(n) + corr * rng.normal(size=(n, n)) / np.sqrt(n)
    X = rng.normal(size=(tokens, n)) @ M.T * rng.lognormal(0, 0.5, n)
    return W, X


def _prep(X, rel=0.01):
    H = O.hessian([X])
    Hd, lam = O.damp(H, rel)
    U, info = O.inverse_cholesky_upper(Hd)
    assert info == 0
    return H, Hd, lam, U


# ----------------------------------------------------------------------------- worked examples (golden)

def test_golden_three_weight_compensation():
    g = _load("obq_three_weight.json")
    H = np.array(g["H"], dtype=float)
    U, info = O.inverse_cholesky_upper(H)
    assert info == 0
    w = np.array(g["w"])
    new = O.obs_step(w, U, 0, w[0] + g["dw1"])
    exp = [float(Fraction(a, b)) for a, b in zip(g["expected_dw_rest"]["num"], g["expected_dw_rest"]["den"])]
    np.testing.assert_allclose(new[1:] - w[1:], exp, rtol=1e-13, atol=1e-15)
    assert new[0] == w[0] + g["dw1"]


def test_golden_quantizer():
    g = _load("quantizer_worked.json")
    for c in g["cases"]:
        v = np.array([c["v"]])
        s, z = O.quant_params(v, c["bits"])
        s_exp = c["s"] if "s" in c else c["s_num"] / c["s_den"]
        np.testing.assert_allclose(s, [s_exp], rtol=1e-15)
        assert z[0] == c["z"]
        q = O.quantize(v, s[:, None], z[:, None], c["bits"])
        assert q[0].tolist() == c["q"]
        if "what" in c:
            np.testing.assert_allclose(O.dequantize(q, s[:, None], z[:, None])[0], c["what"], atol=1e-15)


def test_golden_inverse_factor_2x2():
    g = _load("inverse_factor_2x2.json")
    U, info = O.inverse_cholesky_upper(np.array(g["H"], dtype=float))
    assert info == 0
    exp = np.array(g["U_squared_signed"])
    np.testing.assert_allclose(np.sign(U) * U * U, exp, rtol=1e-14, atol=1e-16)


def test_golden_packing():
    g = _load("packed_3bit.json")
    q = np.array([g["codes"]])
    words = O.pack_codes(q, g["bits"])
    assert words[0].tolist() == g["words"]
    assert O.unpack_codes(words, g["bits"], q.shape[1]).tolist() == q.tolist()


def test_damping_closed_form():
    H = np.array([[1.0, 0.5, 0.0, 0.1], [0.5, 2.0, 0.3, 0.0], [0.0, 0.3, 3.0, 0.2], [0.1, 0.0, 0.2, 6.0]])
    Hd, lam = O.damp(H, 0.01)
    assert lam == pytest.approx(0.03, rel=1e-15)           # 1 % of mean(1, 2, 3, 6) = 3
    np.testing.assert_array_equal(Hd - np.diag(np.diag(Hd)), H - np.diag(np.diag(H)))
    np.testing.assert_allclose(np.diag(Hd), [1.03, 2.03, 3.03, 6.03], rtol=1e-15)


# ----------------------------------------------------------------------------- Hessian

def test_hessian_quadratic_form():
    """a^T H a = 2 ||X^T a||^2 for any a: H is the Hessian of the layer objective."""
    rng = np.random.default_rng(1)
    X = rng.normal(size=(300, 17))
    H = O.hessian([X[:100], X[100:250], X[250:]])
    np.testing.assert_array_equal(H, H.T)
    for _ in range(5):
        a = rng.normal(size=17)
        assert a @ H @ a == pytest.approx(2.0 * np.sum((X @ a) ** 2), rel=1e-12)
    # a column of zeros gives a zero row and column
    X[:, 3] = 0
    H = O.hessian([X])
    assert np.all(H[3] == 0) and np.all(H[:, 3] == 0)


def test_hessian_exact_on_fp16_inputs():
    """fp16 x fp16 products are exact in fp64: H equals an exact integer-scaled sum."""
    W, X = synth.small_layer(4, 24, 512, seed=3, law="lognormal", x_dtype="f16")
    H = O.hessian([X])
    Xi = X.astype(np.float64) * 2.0 ** 24          # fp16 values times 2^24 are integers here
    Xi = Xi.astype(object)
    for (i, j) in [(0, 0), (3, 7), (23, 11)]:
        exact = 2 * sum(int(Xi[t, i]) * int(Xi[t, j]) for t in range(X.shape[0]))
        assert H[i, j] == pytest.approx(float(exact) / 2.0 ** 48, rel=1e-15)


# ----------------------------------------------------------------------------- the inverse factor

def test_inverse_factor_routes():
    """U^T U = H_d^-1, and U equals the reversal route J chol(J H_d J)^-1 J."""
    _, X = _rand_layer(4, 40, 400, 2)
    _, Hd, _, U = _prep(X)
    n = Hd.shape[0]
    np.testing.assert_array_equal(U, np.triu(U))
    assert np.all(np.diag(U) > 0)
    np.testing.assert_allclose(U.T @ U @ Hd, np.eye(n), atol=1e-9)
    J = np.eye(n)[::-1]
    Lr = np.linalg.cholesky(J @ Hd @ J)
    U2 = J @ np.linalg.inv(Lr) @ J
    np.testing.assert_allclose(U, U2, rtol=1e-9, atol=1e-12 * np.abs(U).max())


def test_inverse_factor_reports_pivot():
    n = 6
    U, info = O.inverse_cholesky_upper(np.zeros((n, n)))
    assert U is None and info == 1
    H = np.eye(n)
    H[3, 3] = -1.0
    U, info = O.inverse_cholesky_upper(H)
    assert U is None and info == 4


# ----------------------------------------------------------------------------- the sweep against independent least squares

@pytest.mark.parametrize("n", [3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("rel", [0.0, 0.01])
def test_sweep_is_least_squares_optimal(n, rel):
    """After columns 0..p-1 are fixed to their quantized values, the value the
    sweep rounds at column p is the p-th entry of the minimiser of
    ||(w - w')X||^2 + (lambda/2)||w - w'||^2 over the free columns
    (the OBQ compensation, [OBQ] 'Linear System' / 'Generalized Weight Update'),
    solved here by numpy.linalg.lstsq with no Cholesky factor involved."""
    rng = np.random.default_rng(100 + n)
    m, T = 3, 64
    W = rng.normal(0, 1.0, (m, n))
    X = rng.normal(size=(T, n)) @ (np.eye(n) + 0.5 * rng.normal(size=(n, n)))
    H = O.hessian([X])
    Hd, lam = O.damp(H, rel)
    U, info = O.inverse_cholesky_upper(Hd)
    assert info == 0
    res = O.gptq_quantize(W, U, bits=2, group=0, block=None)
    Xt = X.T                                     # [n x T], the pages' X
    Xaug = np.concatenate([Xt, np.sqrt(lam / 2.0) * np.eye(n)], axis=1) if lam > 0 else Xt
    for r in range(m):
        for p in range(n):
            fixed_delta = W[r, :p] - res["What"][r, :p]
            rhs = -(Xaug[:p].T @ fixed_delta) if p else np.zeros(Xaug.shape[1])
            d_free, *_ = np.linalg.lstsq(Xaug[p:].T, rhs, rcond=None)
            v_opt = W[r, p:] - d_free
            v_sweep = res["t"][r, p] * res["s"][r, 0]
            assert v_sweep == pytest.approx(v_opt[0], rel=1e-9, abs=1e-12)


@pytest.mark.parametrize("group", [0, 4])
def test_three_routes_agree(group):
    """Cholesky rows, OBS rank-one downdates and naive re-inversion ([OBQ] 'The
    OBS / GPTQ Trick'; [GPTQ] 'Observation 3') give the same sweep."""
    W, X = _rand_layer(5, 12, 200, 4)
    H, Hd, lam, U = _prep(X)
    a = O.gptq_quantize(W, U, 3, group, block=None)
    b = O.gptq_quantize_obs(W, Hd, 3, group)
    c = O.gptq_quantize_naive(W, Hd, 3, group)
    assert np.array_equal(a["q"], b["q"]) and np.array_equal(a["q"], c["q"])
    np.testing.assert_allclose(a["What"], b["V"], atol=1e-12)
    np.testing.assert_allclose(a["What"], c["V"], atol=1e-12)
    np.testing.assert_allclose(a["s"], b["s"], rtol=1e-12)


# ----------------------------------------------------------------------------- special cases

@pytest.mark.parametrize("bits,group", [(4, 0), (4, 16), (3, 8), (2, 0)])
def test_diagonal_hessian_is_rtn(bits, group):
    """Uncorrelated inputs (diagonal H) leave nothing to compensate: the sweep
    reduces exactly to round-to-nearest ([SOQ] 'The objective is layer output')."""
    rng = np.random.default_rng(7)
    m, n = 9, 48
    W = rng.normal(0, 0.02, (m, n))
    H = np.diag(rng.lognormal(0, 1, n)) * 1000.0
    Hd, _ = O.damp(H, 0.01)
    U, info = O.inverse_cholesky_upper(Hd)
    assert info == 0
    assert np.count_nonzero(U - np.diag(np.diag(U))) == 0
    g = O.gptq_quantize(W, U, bits, group, block=16)
    r = O.rtn(W, bits, group)
    assert np.array_equal(g["q"], r["q"])
    np.testing.assert_array_equal(g["s"], r["s"])
    np.testing.assert_array_equal(g["z"], r["z"])


def test_single_column_and_on_grid_weights():
    rng = np.random.default_rng(8)
    W = rng.normal(0, 0.02, (6, 1))
    U = np.array([[0.3]])
    g = O.gptq_quantize(W, U, 4, 0, block=1)
    assert np.array_equal(g["q"], O.rtn(W, 4, 0)["q"])
    # weights already on the grid come back unchanged, with zero error
    _, X = _rand_layer(4, 32, 300, 9)
    _, _, _, U = _prep(X)
    q = rng.integers(0, 16, (4, 32))
    q[:, 0], q[:, 1] = 0, 15                 # pin the row range to the full grid
    s = np.array([0.01, 0.02, 0.005, 0.03])
    z = np.array([3.0, 8.0, 0.0, 15.0])
    Wg = s[:, None] * (q - z[:, None])
    g = O.gptq_quantize(Wg, U, 4, 0, block=8)
    assert np.array_equal(g["q"], q)
    assert np.max(np.abs(g["E"])) < 1e-12
    np.testing.assert_allclose(g["What"], Wg, atol=1e-15)


def test_zero_rows_and_groups():
    _, X = _rand_layer(3, 32, 300, 10)
    _, _, _, U = _prep(X)
    W = np.zeros((3, 32))
    W[1, 16:] = 0.01 * np.arange(16)
    g = O.gptq_quantize(W, U, 4, 16, block=16)
    assert np.all(g["q"][0] == 0) and np.all(g["What"][0] == 0)
    assert np.all(g["s"][0] == 1.0 / 15) and np.all(g["z"][0] == 0)


# ----------------------------------------------------------------------------- schedule invariance and exact identities

@pytest.mark.parametrize("group,blocks", [(0, [1, 2, 32, 128, 200]), (32, [1, 2, 8, 32, 64, 128]), (128, [1, 32, 64, 128])])
def test_block_size_invariance(group, blocks):
    """The lazy block schedule is an exact reformulation ([GPTQ] 'Observation 2',
    [SOQ-vi] 'Lazy batch update'): every B gives the definition's codes; only
    sub-1e-9 near-ties may differ by fp64 summation order."""
    W, X = _rand_layer(16, 200, 800, 11)
    _, _, _, U = _prep(X)
    ref = O.gptq_quantize(W, U, 4, group, block=None)
    for B in blocks:
        if group > 0 and not (group % B == 0 or B % group == 0):
            continue
        g = O.gptq_quantize(W, U, 4, group, block=B)
        diff = g["q"] != ref["q"]
        if diff.any():
            assert np.all(O.boundary_distance(ref["t"][diff]) < 1e-9)
        np.testing.assert_allclose(g["What"][~diff.any(1)], ref["What"][~diff.any(1)], atol=1e-12)


def test_loss_identities():
    """W - What = E U, tr(dW H_d dW^T) = ||E||^2 and
    ||dW X||^2 = (||E||^2 - lambda ||dW||^2)/2 (derived from [GPTQ]
    'Observation 3' with H_d^-1 = U^T U; per column this is OBQ's
    loss increase e_p^2/2 of [OBQ] 'Greedy Search')."""
    W, X = _rand_layer(12, 96, 600, 12)
    H, Hd, lam, U = _prep(X)
    g = O.gptq_quantize(W, U, 3, 32, block=32)
    dW = W - g["What"]
    np.testing.assert_allclose(dW, g["E"] @ U, atol=1e-13)
    E2 = np.sum(g["E"] ** 2)
    assert np.trace(dW @ Hd @ dW.T) == pytest.approx(E2, rel=1e-10)
    L = O.layer_loss(W, g["What"], H)
    assert L == pytest.approx(0.5 * (E2 - lam * np.sum(dW ** 2)), rel=1e-9)
    assert L == pytest.approx(O.layer_loss_direct(W, g["What"], X), rel=1e-10)
    np.testing.assert_allclose(g["err_sq"], np.sum(g["E"] ** 2, axis=1), rtol=1e-15)


def test_hessian_scale_invariance():
    """H -> 4H (a power of two, so every IEEE step scales exactly) leaves codes
    and scales bitwise unchanged: the damping is relative to H."""
    W, X = _rand_layer(8, 64, 400, 13)
    H = O.hessian([X])
    outs = []
    for c in (1.0, 4.0):
        Hd, _ = O.damp(c * H, 0.01)
        U, _ = O.inverse_cholesky_upper(Hd)
        outs.append(O.gptq_quantize(W, U, 4, 16, block=16))
    assert np.array_equal(outs[0]["q"], outs[1]["q"])
    np.testing.assert_array_equal(outs[0]["s"], outs[1]["s"])
    np.testing.assert_array_equal(outs[0]["E"] * 2.0, outs[1]["E"])


def test_row_independence():
    """Rows are independent subproblems sharing one U ([OBQ] 'From Layer Error
    to Row-wise Weight Errors'; [GPTQ] 'Observation 1')."""
    W, X = _rand_layer(10, 48, 300, 14)
    _, _, _, U = _prep(X)
    a = O.gptq_quantize(W, U, 4, 16, block=16)
    perm = np.random.default_rng(0).permutation(10)
    b = O.gptq_quantize(W[perm], U, 4, 16, block=16)
    assert np.array_equal(a["q"][perm], b["q"])
    c = O.gptq_quantize(W[3:5], U, 4, 16, block=16)
    assert np.array_equal(a["q"][3:5], c["q"])


@pytest.mark.parametrize("bits,group", [(4, 0), (4, 32), (3, 16), (3, 0)])
def test_gptq_beats_rtn(bits, group):
    wl = synth.workloads()["tiny"]
    job = wl.jobs[0]
    W = synth.stacked_weight(job, wl.seed, wl.wid).astype(np.float64)
    X = synth.x_full(job.x, wl.seed, wl.wid).astype(np.float64)
    H, Hd, lam, U = _prep(X)
    g = O.gptq_quantize(W, U, bits, group, block=32 if group in (0, 32) else 16)
    r = O.rtn(W, bits, group)
    assert O.layer_loss(W, g["What"], H) < O.layer_loss(W, r["What"], H)


def test_schedule_validation():
    with pytest.raises(ValueError):
        O.check_schedule(64, 48, 32)
    O.check_schedule(64, 64, 32)
    O.check_schedule(64, 16, 32)
    O.check_schedule(64, 0, 7)


def test_pack_roundtrip_all_widths():
    rng = np.random.default_rng(15)
    for bits in range(2, 9):
        for n in (1, 7, 31, 32, 33, 100):
            q = rng.integers(0, 1 << bits, (3, n))
            w = O.pack_codes(q, bits)
            assert w.shape == (3, O.packed_words(n, bits))
            assert np.array_equal(O.unpack_codes(w, bits, n), q)


# ----------------------------------------------------------------------------- the packed layer at run time

def test_dequant_matmul_zero_point_codes_give_zero():
    """Codes equal to their group's zero point dequantize to 0: Y = 0."""
    rng = np.random.default_rng(21)
    m, n, group, bits = 5, 256, 64, 4
    z = rng.integers(0, 16, (m, n // group))
    q = np.repeat(z, group, axis=1)
    s = rng.uniform(0.01, 0.1, (m, n // group))
    X = rng.normal(size=(3, n))
    assert np.array_equal(O.dequant_matmul(X, O.pack_codes(q, bits), s, z, bits, group, n), np.zeros((3, m)))


def test_dequant_matmul_single_code_selects_its_column():
    """One code one step above its zero point, all others at it: Y[:, r] is
    s[r, g(c)] X[:, c] for that column c only (bit order, column index, group
    index and the X W^T orientation all matter)."""
    rng = np.random.default_rng(22)
    m, n, bits = 4, 96, 3
    for group in (0, 32):
        G = O.n_groups(n, group)
        z = rng.integers(0, 4, (m, G))
        s = rng.uniform(0.5, 2.0, (m, G))
        X = rng.normal(size=(2, n))
        for r, c in ((0, 0), (1, 31), (2, 32), (3, 95), (1, 50)):
            g = 0 if group <= 0 else c // group
            q = np.repeat(z, n if group <= 0 else group, axis=1)[:, :n].copy()
            q[r, c] += 1
            Y = O.dequant_matmul(X, O.pack_codes(q, bits), s, z, bits, group, n)
            want = np.zeros((2, m))
            want[:, r] = s[r, g] * X[:, c]
            assert np.allclose(Y, want, rtol=0, atol=1e-15), (group, r, c)


def test_dequant_matmul_matches_rtn_layer():
    """Round-to-nearest quantization of W, packed, then run: equals X What^T
    with What as the quantizer itself produced it."""
    rng = np.random.default_rng(23)
    m, n = 6, 384
    X = rng.normal(size=(4, n))
    W = rng.normal(0, 0.02, (m, n))
    for bits, group in ((4, 128), (4, 0), (3, 64), (8, 128)):
        r = O.rtn(W, bits, group)
        Y = O.dequant_matmul(X, O.pack_codes(r["q"], bits), r["s"], r["z"], bits, group, n)
        assert np.allclose(Y, X @ r["What"].T, rtol=1e-13, atol=1e-15)


# ----------------------------------------------------------------------------- following another sweep at near-ties

def test_follow_own_result_changes_nothing():
    """Following the sweep's own codes and zero points is the plain sweep."""
    W, X = _rand_layer(10, 96, 500, 31)
    _, _, _, U = _prep(X)
    a = O.gptq_quantize(W, U, 3, 32, block=32)
    b = O.gptq_quantize(W, U, 3, 32, block=32, follow=(a["q"], a["z"]), tie=0.5)
    assert b["followed"] == 0
    for k in ("q", "s", "z", "E", "What"):
        np.testing.assert_array_equal(a[k], b[k])


def test_follow_takes_only_adjacent_roundings_at_near_ties():
    """Round-to-nearest layer (diagonal U), one value 1e-6 steps past the
    boundary 2.5: the other side's 'below' rounding is taken within the tie
    band, not outside it, and never a non-adjacent code or a code away from
    a tie.  Row [-1, 2, x], 4 bits: s = 3/15, z = rint(1/s) = 5
    ([SOQ-vi] asymmetric min/max grid)."""
    s = 3.0 / 15.0
    W = np.array([[-1.0, 2.0, s * (2.5 + 1e-6)]])
    U = np.eye(3)
    own = O.gptq_quantize(W, U, 4, 0, None)
    assert own["z"][0, 0] == 5 and list(own["q"][0]) == [0, 15, 8]
    z = own["z"].astype(np.int64)
    below = np.array([[0, 15, 7]])
    r = O.gptq_quantize(W, U, 4, 0, None, follow=(below, z), tie=1e-4)
    assert r["followed"] == 1 and r["q"][0, 2] == 7
    assert r["What"][0, 2] == pytest.approx(s * 2)
    assert O.gptq_quantize(W, U, 4, 0, None, follow=(below, z), tie=1e-7)["followed"] == 0
    for other in ([[0, 15, 9]], [[1, 15, 8]], [[0, 14, 8]]):   # not adjacent / not at a tie
        r = O.gptq_quantize(W, U, 4, 0, None, follow=(np.array(other), z), tie=1e-4)
        assert r["followed"] == 0 and list(r["q"][0]) == [0, 15, 8]
    # zero point at a near-tie: -lo/s = 5 + 0.5 + 1e-6 -> own 6, the other side's 5 is taken
    lo = -(5.5 + 1e-6) * s
    W2 = np.array([[lo, lo + 15 * s, 0.0]])
    own2 = O.gptq_quantize(W2, U, 4, 0, None)
    assert own2["z"][0, 0] == 6
    r2 = O.gptq_quantize(W2, U, 4, 0, None, follow=(own2["q"], np.array([[5]])), tie=1e-4)
    assert r2["z"][0, 0] == 5 and r2["followed"] >= 1
    assert O.gptq_quantize(W2, U, 4, 0, None, follow=(own2["q"], np.array([[4]])), tie=1e-4)["z"][0, 0] == 6


def test_follow_flip_is_compensated():
    """A decision taken over at column p changes that code only, and the
    later columns are compensated for it: W - What = E U still holds
    (the identity of [GPTQ] 'Observation 3' with H_d^-1 = U^T U), codes
    before p are unchanged, and the sweep stays a valid quantizer run."""
    W, X = _rand_layer(6, 64, 400, 32)
    _, _, _, U = _prep(X)
    a = O.gptq_quantize(W, U, 4, 0, None)
    r, p = 2, 17
    t = a["t"][r, p]
    other = a["q"].copy()
    # the rounding on the other side of the nearest boundary
    other[r, p] = int(np.clip(np.floor(t) + a["z"][r, 0] + (1 if np.rint(t) == np.floor(t) else 0), 0, 15))
    b = O.gptq_quantize(W, U, 4, 0, None, follow=(other, a["z"]), tie=1.0)   # every boundary counts as near
    assert b["q"][r, p] == other[r, p] != a["q"][r, p]
    np.testing.assert_array_equal(b["q"][r, :p], a["q"][r, :p])
    np.testing.assert_array_equal(np.delete(b["q"], r, axis=0), np.delete(a["q"], r, axis=0))
    np.testing.assert_allclose(W - b["What"], b["E"] @ U, atol=1e-13)
    assert not np.allclose(b["E"][r, p + 1:], a["E"][r, p + 1:])
