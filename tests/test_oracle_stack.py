"""Pins of the oracle's network-level loop (quantize_mlp_stack; reading R13:
MLP blocks x <- x + W_down (silu(W_gate x) * (W_up x)); [GPTQ] "Algorithm
GPTQ": each layer's calibration inputs come from the network as quantized so
far)."""
import math

import numpy as np
import pytest

import oracle as O


def test_silu_closed_forms():
    assert O.silu(np.array([0.0]))[0] == 0.0
    # silu(v) - silu(-v) = v, and silu(v) -> v for large v, -> 0 for very negative v
    v = np.linspace(-6, 6, 25)
    np.testing.assert_allclose(O.silu(v) - O.silu(-v), v, atol=1e-14)
    assert O.silu(np.array([40.0]))[0] == pytest.approx(40.0, rel=1e-15)
    assert abs(O.silu(np.array([-40.0]))[0]) < 1e-15
    assert O.silu(np.array([1.0]))[0] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    np.testing.assert_allclose(O.swiglu(np.array([[2.0, -1.0]]), np.array([[3.0, 5.0]])),
                               [[3.0 * 2.0 / (1 + math.exp(-2.0)), 5.0 * -1.0 / (1 + math.exp(1.0))]], rtol=1e-15)


def _stack(d, f, L, seed):
    rng = np.random.default_rng(seed)
    return [(rng.normal(0, 0.05, (f, d)), rng.normal(0, 0.05, (f, d)), rng.normal(0, 0.05, (d, f)))
            for _ in range(L)]


def test_each_layer_sees_the_quantized_network():
    """Block l's input is block l-1's output computed with the quantized
    weights (not the original ones), and each layer's result is exactly the
    single-layer sweep on that input."""
    d, f, T, L = 32, 48, 400, 3
    blocks = _stack(d, f, L, 1)
    X0 = np.random.default_rng(2).standard_normal((T, d))
    res, XL = O.quantize_mlp_stack(blocks, X0, 4, 16, 16, 0.01)
    X = X0
    for (Wg, Wu, Wd), r in zip(blocks, res):
        np.testing.assert_array_equal(r["X"], X)
        ref = O.quantize_layer_from_x(Wg, [X], 4, 16, 16, 0.01)
        np.testing.assert_array_equal(r["gate"]["q"], ref["q"])
        A = O.swiglu(X @ r["gate"]["What"].T, X @ r["up"]["What"].T)
        np.testing.assert_array_equal(r["A"], A)
        refd = O.quantize_layer_from_x(Wd, [A], 4, 16, 16, 0.01)
        np.testing.assert_array_equal(r["down"]["q"], refd["q"])
        X = X + A @ r["down"]["What"].T
    np.testing.assert_array_equal(XL, X)
    # the quantized network's inputs differ from the float network's after block 0
    Xf = X0 + O.swiglu(X0 @ blocks[0][0].T, X0 @ blocks[0][1].T) @ blocks[0][2].T
    assert not np.allclose(res[1]["X"], Xf, rtol=1e-6)


def test_exact_weights_pass_through():
    """Weights already on their quantization grid are reproduced exactly, so
    the quantized stack computes the float stack."""
    d, f, T = 16, 32, 200
    rng = np.random.default_rng(5)
    def on_grid(m, n):  # 4-bit per-row grid with scale 0.01 and zero 8, row min and max on the grid ends
        q = rng.integers(0, 16, (m, n))
        q[:, 0], q[:, 1] = 0, 15
        return 0.01 * (q - 8)
    blocks = [(on_grid(f, d), on_grid(f, d), on_grid(d, f))]
    X0 = rng.standard_normal((T, d))
    res, XL = O.quantize_mlp_stack(blocks, X0, 4, 0, 16, 0.01)
    Wg, Wu, Wd = blocks[0]
    np.testing.assert_allclose(res[0]["gate"]["What"], Wg, atol=1e-12)
    np.testing.assert_allclose(XL, X0 + O.swiglu(X0 @ Wg.T, X0 @ Wu.T) @ Wd.T, atol=1e-9)


# ----------------------------------------------------------------------------- transformer blocks

def _attention_by_loops(Q, K, V, seq_len, heads):
    """Causal softmax attention written query by query, key by key."""
    T, dm = Q.shape
    dh = dm // heads
    O = np.zeros((T, dm))
    for i in range(T):
        s0 = (i // seq_len) * seq_len
        for h in range(heads):
            c0 = h * dh
            sc = [sum(Q[i, c0 + e] * K[j, c0 + e] for e in range(dh)) / math.sqrt(dh) for j in range(s0, i + 1)]
            mx = max(sc)
            w = [math.exp(x - mx) for x in sc]
            tot = sum(w)
            for e in range(dh):
                O[i, c0 + e] = sum(wj * V[s0 + jj, c0 + e] for jj, wj in enumerate(w)) / tot
    return O


def test_attention_matches_loops():
    rng = np.random.default_rng(11)
    T, seq, heads, dh = 12, 6, 2, 3
    Q, K, V = (rng.standard_normal((T, heads * dh)) for _ in range(3))
    np.testing.assert_allclose(O.attention(Q, K, V, seq, heads), _attention_by_loops(Q, K, V, seq, heads),
                               rtol=1e-12, atol=1e-13)


def test_attention_special_cases():
    rng = np.random.default_rng(12)
    T, seq, heads, dh = 16, 8, 2, 4
    Q, K, V = (rng.standard_normal((T, heads * dh)) for _ in range(3))
    Oa = O.attention(Q, K, V, seq, heads)
    # the first token of every sequence sees only itself
    np.testing.assert_allclose(Oa[[0, 8]], V[[0, 8]], atol=1e-14)
    # equal keys: every visible key gets the same weight, a running mean of V
    Oe = O.attention(Q, np.ones_like(K), V, seq, heads)
    for i in range(T):
        s0 = (i // seq) * seq
        np.testing.assert_allclose(Oe[i], V[s0:i + 1].mean(axis=0), atol=1e-13)
    # one dominant score selects its value; heads are independent of each other
    K2 = K.copy()
    K2[3, :dh] = 60.0 * Q[7, :dh] / np.linalg.norm(Q[7, :dh])
    np.testing.assert_allclose(O.attention(Q, K2, V, seq, heads)[7, :dh], V[3, :dh], atol=1e-6)
    np.testing.assert_array_equal(O.attention(Q, K2, V, seq, heads)[:, dh:], Oa[:, dh:])


def test_attention_error_bound_covers_fp32():
    """An fp32 evaluation of the same attention stays inside the bound."""
    rng = np.random.default_rng(13)
    T, seq, heads, dh = 128, 64, 2, 64
    Q, K, V = ((rng.standard_normal((T, heads * dh)) * 2).astype(np.float16).astype(np.float64) for _ in range(3))
    O64 = O.attention(Q, K, V, seq, heads)
    Q32, K32, V32 = (a.astype(np.float32) for a in (Q, K, V))
    O32 = np.zeros_like(O64)
    mask = np.tril(np.ones((seq, seq), dtype=bool))
    for s0 in range(0, T, seq):
        for h in range(heads):
            c = slice(h * dh, (h + 1) * dh)
            S = (Q32[s0:s0 + seq, c] @ K32[s0:s0 + seq, c].T) / np.float32(math.sqrt(dh))
            S = np.where(mask, S, np.float32(-np.inf))
            P = np.exp(S - S.max(axis=1, keepdims=True)).astype(np.float32)
            O32[s0:s0 + seq, c] = (P @ V32[s0:s0 + seq, c]) / P.sum(axis=1, keepdims=True)
    B = O.attention_error_bound(Q, K, V, O64, seq, heads)
    assert np.all(np.abs(O32 - O64) <= B)


def test_round_activations_follow():
    y = np.array([1.0, 1.0 + 2 ** -11, 1.0 + 2 ** -11 + 1e-9, 0.3, -2.5])
    own, k = O.round_activations(y, "f16")
    np.testing.assert_array_equal(own, y.astype(np.float16).astype(np.float64))
    assert k == 0
    # 1 + 2^-11 is the midpoint of 1 and 1 + 2^-10: round to even gives 1; the other side's 1 + 2^-10 is taken
    other = own.copy()
    other[1] = 1.0 + 2 ** -10
    other[2] = 1.0             # the value just above the midpoint rounds up on its own: 1 is also adjacent
    other[3] = 0.25            # not a rounding of anything within the tolerance of 0.3: never taken
    got, k = O.round_activations(y, "f16", other, np.full(5, 1e-8))
    assert k == 2
    assert got[1] == 1.0 + 2 ** -10 and got[2] == 1.0 and got[3] == own[3]
    # outside the tolerance nothing is taken
    got, k = O.round_activations(y, "f16", other, np.full(5, 1e-12))
    assert k == 1 and got[2] == own[2] and got[1] == 1.0 + 2 ** -10
    # a wide tolerance (a result of cancelling sums) admits roundings two steps away, not three
    y2 = np.array([2.0 ** -12 * 1.5])
    ulp = 2.0 ** -22
    far2 = np.array([y2[0] + 2 * ulp])
    far3 = np.array([y2[0] + 3 * ulp])
    assert O.round_activations(y2, "f16", far2, np.array([2.2 * ulp]))[1] == 1
    assert O.round_activations(y2, "f16", far3, np.array([2.2 * ulp]))[1] == 0
    # fp64 activations pass through
    assert O.round_activations(y, None)[0] is not None and np.array_equal(O.round_activations(y, None)[0], y)


def _tblocks(d, f, L, seed):
    rng = np.random.default_rng(seed)
    return [tuple(rng.normal(0, 0.05, shp) for shp in [(d, d)] * 4 + [(f, d), (f, d), (d, f)]) for _ in range(L)]


@pytest.mark.parametrize("act", [None, "f16"])
def test_transformer_stack_each_layer_sees_the_quantized_network(act):
    d, f, T, L, seq, heads = 16, 24, 256, 2, 64, 2
    blocks = _tblocks(d, f, L, 3)
    X0 = np.random.default_rng(4).standard_normal((T, d))
    res, XL = O.quantize_transformer_stack(blocks, X0, seq, heads, 4, 16, 16, 0.01, act_dtype=act)
    rnd = (lambda a: a.astype(np.float16).astype(np.float64)) if act else (lambda a: a)
    X = rnd(X0)
    for (Wq, Wk, Wv, Wo, Wg, Wu, Wd), r in zip(blocks, res):
        np.testing.assert_array_equal(r["X"], X)
        ref = O.quantize_layer_from_x(np.concatenate([Wq, Wk, Wv]), [X], 4, 16, 16, 0.01)
        np.testing.assert_array_equal(r["qkv"]["q"], ref["q"])
        QKV = rnd(X @ r["qkv"]["What"].T)
        np.testing.assert_array_equal(r["QKV"], QKV)
        A = rnd(O.attention(QKV[:, :d], QKV[:, d:2 * d], QKV[:, 2 * d:], seq, heads))
        np.testing.assert_array_equal(r["A"], A)
        np.testing.assert_array_equal(r["o"]["q"], O.quantize_layer_from_x(Wo, [A], 4, 16, 16, 0.01)["q"])
        Xm = rnd(X + rnd(A @ r["o"]["What"].T))
        GU = rnd(Xm @ r["gate_up"]["What"].T)
        A2 = rnd(O.swiglu(GU[:, :f], GU[:, f:]))
        np.testing.assert_array_equal(r["A2"], A2)
        X = rnd(Xm + rnd(A2 @ r["down"]["What"].T))
        assert r["followed_act"] == 0
    np.testing.assert_array_equal(XL, X)


def test_transformer_stack_following_itself_changes_nothing():
    d, f, T, L, seq, heads = 16, 24, 128, 2, 64, 2
    blocks = _tblocks(d, f, L, 5)
    X0 = np.random.default_rng(6).standard_normal((T, d))
    res, XL = O.quantize_transformer_stack(blocks, X0, seq, heads, 3, 0, 16, 0.01, act_dtype="f16")
    fol = [{**{k: r[k] for k in ("QKV", "A", "Yo", "X_mid", "GU", "A2", "Yd", "X_out")},
            **{k: (r[k]["q"], r[k]["z"]) for k in ("qkv", "o", "gate_up", "down")}} for r in res]
    res2, XL2 = O.quantize_transformer_stack(blocks, X0, seq, heads, 3, 0, 16, 0.01, act_dtype="f16", follow=fol,
                                             tie=1e-4)
    np.testing.assert_array_equal(XL2, XL)
    for r, r2 in zip(res, res2):
        assert r2["followed_act"] == 0
        for k in ("qkv", "o", "gate_up", "down"):
            np.testing.assert_array_equal(r2[k]["q"], r[k]["q"])
            assert r2[k]["followed"] == 0
