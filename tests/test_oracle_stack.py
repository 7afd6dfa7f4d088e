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
