"""GPU-vs-oracle parity of OBQ's greedy-order quantization
(gptq_quantize_greedy) through the C ABI.

The oracle (oracle.obq_greedy, fp64) runs on the same W and U.  Where the
GPU's fp32 arithmetic and the oracle's fp64 place a decision on different
sides of a near-tie, the oracle takes the GPU's choice: a rounding or zero
point within TIE grid steps of a boundary (as for the sweep), or a greedy pick
whose sqrt-loss is within ORDER_TIE grid steps of the oracle's own best.
After that every order entry, code and zero point must match exactly, scales
to SCALE_RTOL and each row's loss to LOSS_RTOL.  Rows are independent, so the
large cases compare a sample of rows (including the first and last row of
each pass of the resident workgroups)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from parity import SCALE_RTOL, TIE, say

pytestmark = pytest.mark.gpu

pw = pytest.importorskip("post_weight_quantization_10_amd")
DEV = "cuda:0"
ORDER_TIE = 1e-4
LOSS_RTOL = 1e-4


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def problem(m, n, wdt, seed, law="lognormal"):
    W, X = synth.small_layer(m, n, max(4 * n, 256), seed=seed, law=law, w_dtype=wdt, x_dtype="f32",
                             outlier_channels=min(2, n) if law == "lognormal" else 0)
    Hd, _ = O.damp(O.hessian([X.astype(np.float64)]), 0.01)
    U_ref, info = O.inverse_cholesky_upper(Hd)
    assert info == 0
    return W, synth.as_float64(W, wdt), Hd, U_ref.astype(np.float32)


def run_gpu(W, wdt, U32, bits, group):
    res = pw.quantize_greedy(to_dev(W, wdt), torch.from_numpy(U32).to(DEV), bits, group)
    torch.cuda.synchronize()
    n = W.shape[1]
    out = {k: v.cpu().numpy() for k, v in res.items()}
    out["q"] = O.unpack_codes(out["qcodes"].view(np.uint32), bits, n)
    return out


def greedy_check(g, Wd, U32, Hd, bits, group, rows, label):
    rows = np.asarray(rows)
    ref = O.obq_greedy(Wd[rows], U32.astype(np.float64), bits, group,
                       follow=(g["q"][rows], g["zeros"][rows], g["order"][rows].astype(np.int64)),
                       tie=TIE, order_tie=ORDER_TIE)
    say(f"  {label}: followed {ref['followed']} near-tie decisions (largest order gap {ref['order_margin']:.2e} steps)")
    bad = np.argwhere(g["order"][rows] != ref["order"])
    assert not len(bad), f"{label}: order differs at {len(bad)} steps, first row {rows[bad[0][0]]} step {bad[0][1]}"
    qbad = np.argwhere(g["q"][rows] != ref["q"])
    assert not len(qbad), f"{label}: {len(qbad)} codes differ, first row {rows[qbad[0][0]]} col {qbad[0][1]}"
    np.testing.assert_array_equal(g["zeros"][rows].astype(np.int64), ref["z"].astype(np.int64))
    srel = np.max(np.abs(g["scales"][rows] - ref["s"]) / ref["s"])
    assert srel <= SCALE_RTOL, f"{label}: scale rel {srel:.3e}"
    # Floor: the loss that fp32 rounding of each what_p alone can leave (a row
    # whose weights all sit on the grid has oracle loss 0).
    Hinv = U32.astype(np.float64).T @ U32.astype(np.float64)
    floor = Wd.shape[1] * (2.0 ** -22 * np.max(np.abs(Wd[rows]), axis=1)) ** 2 / np.min(np.diag(Hinv))
    lrel = np.max(np.maximum(np.abs(g["loss"][rows] - ref["loss"]) - floor, 0.0) / np.maximum(ref["loss"], floor))
    say(f"  {label}: loss rel {lrel:.2e} (beyond an absolute floor of up to {floor.max():.1e})")
    assert lrel <= LOSS_RTOL
    # The loss the GPU reports is the proxy loss of the codes it wrote (exact algebra).
    gi = np.zeros(Wd.shape[1], dtype=np.int64) if group <= 0 else np.arange(Wd.shape[1]) // group
    D = Wd[rows] - ref["s"][:, gi] * (g["q"][rows] - ref["z"][:, gi])
    quad = np.einsum("ij,jk,ik->i", D, Hd, D)
    assert np.all(np.abs(quad - g["loss"][rows]) <= 2e-3 * quad + floor)
    return ref


# (m, n, bits, group, dtype): rows of up to 128 keep H^-1 in LDS with four rows per CU; longer ones
# use the workspace, with deferred downdates up to 1024.
CASES = [
    (64, 96, 4, 0, "f16"), (48, 256, 4, 32, "bf16"), (32, 272, 3, 0, "f32"), (24, 273, 4, 64, "f16"),
    (16, 600, 4, 128, "f16"), (8, 1000, 2, 16, "f32"), (5, 40, 4, 128, "f16"), (3, 1, 4, 0, "f32"),
    (1, 17, 8, 0, "bf16"), (40, 130, 3, 16, "f16"), (20, 128, 4, 32, "bf16"), (20, 129, 3, 0, "f16"),
    (300, 100, 4, 0, "f32"), (3, 1100, 4, 128, "f16"), (12, 257, 3, 32, "f32"), (10, 400, 4, 64, "bf16"),
    (2, 1024, 4, 128, "bf16"),
]


@pytest.mark.parametrize("m,n,bits,group,wdt", CASES)
def test_greedy_parity(m, n, bits, group, wdt):
    say(f"[greedy] m={m} n={n} bits={bits} group={group} dtype={wdt}")
    W, Wd, Hd, U32 = problem(m, n, wdt, seed=m * 31 + n)
    g = run_gpu(W, wdt, U32, bits, group)
    for r in range(m):
        assert np.array_equal(np.sort(g["order"][r]), np.arange(n)), f"row {r}: order is not a permutation"
    greedy_check(g, Wd, U32, Hd, bits, group, np.arange(m), f"{m}x{n}")


@pytest.mark.parametrize("m,n,rows", [
    (600, 290, [0, 1, 255, 256, 511, 512, 599]),            # workspace path: 256 resident workgroups, 3 passes
    (70000, 64, [0, 1, 65534, 65535, 69999]),              # LDS path: more rows than workgroups
])
def test_greedy_resident_workgroups_take_every_row(m, n, rows):
    say(f"[greedy] m={m} n={n} sampled rows {rows}")
    W, Wd, Hd, U32 = problem(m, n, "f16", seed=m + n)
    g = run_gpu(W, "f16", U32, 4, 0)
    assert np.all(np.sort(g["order"], axis=1) == np.arange(n)), "some row was not swept"
    greedy_check(g, Wd, U32, Hd, 4, 0, rows, f"{m}x{n}")


def test_greedy_bench_layer_sampled_rows():
    """The layer `bench.py --kernel obq` times (4096 x 256 fp16, 4-bit g128,
    H from 8192 lognormal-input fp16 tokens with two outlier channels), in the
    same launch configuration, checked on sampled rows."""
    m, n = 4096, 256
    W, X = synth.small_layer(m, n, 4 * 2048, seed=41, law="lognormal", w_dtype="f16", x_dtype="f16",
                             outlier_channels=2)
    Hd, _ = O.damp(O.hessian([synth.as_float64(X, "f16")]), 0.01)
    U_ref, info = O.inverse_cholesky_upper(Hd)
    assert info == 0
    U32 = U_ref.astype(np.float32)
    g = run_gpu(W, "f16", U32, 4, 128)
    assert np.all(np.sort(g["order"], axis=1) == np.arange(n)), "some row was not swept"
    rows = [0, 1, 255, 256, 2047, 4094, 4095]
    say(f"[greedy] bench layer {m}x{n}, sampled rows {rows}")
    greedy_check(g, synth.as_float64(W, "f16"), U32, Hd, 4, 128, rows, f"{m}x{n}")


def test_greedy_equals_rtn_for_identity_hessian():
    """U = I: nothing moves, so the codes are round-to-nearest of the original
    row (exact: the same fp32 products decide both sides up to near-ties)."""
    m, n = 20, 200
    W, _ = synth.small_layer(m, n, 16, seed=3, w_dtype="f32", x_dtype="f32")
    g = run_gpu(W, "f32", np.eye(n, dtype=np.float32), 4, 64)
    ref = O.rtn(W.astype(np.float64), 4, 64)
    assert np.mean(g["q"] == ref["q"]) > 0.999


@pytest.mark.parametrize("law", ["corr", "lognormal"])
def test_greedy_against_rtn_and_fixed_order(law):
    """Same layer, same factor, same per-row grids (3-bit): the greedy order's
    proxy loss against round-to-nearest (no compensation) and the fixed-order
    sweep.  With correlated input channels the greedy order is clearly ahead
    of the fixed order (about 20 % lower here); with nearly independent
    lognormal channels H is close to diagonal, compensation does little and
    greedy lands a few percent behind the fixed order (both still below
    round-to-nearest).  [GPTQ] "Observation 1" expects the two orders to be
    close on large layers."""
    m, n = 64, 256
    W, Wd, Hd, U32 = problem(m, n, "f32", seed=77, law=law)
    g = run_gpu(W, "f32", U32, 3, 0)
    Wt = to_dev(W, "f32")
    f = pw.quantize_layer(Wt.clone(), torch.from_numpy(U32).to(DEV), 3, 0, 128, write_dequant=False)
    torch.cuda.synchronize()
    qf = O.unpack_codes(f["qcodes"].cpu().numpy().view(np.uint32), 3, n)
    sf, zf = f["scales"].cpu().numpy().astype(np.float64), f["zeros"].cpu().numpy()

    def quad(What):
        D = Wd - What
        return np.einsum("ij,jk,ik->i", D, Hd, D).sum()

    fixed = quad(sf * (qf - zf))
    rtn = quad(O.rtn(Wd, 3, 0)["What"])
    greedy = float(g["loss"].astype(np.float64).sum())
    say(f"  {law}: proxy loss greedy {greedy:.4e}, fixed order {fixed:.4e} (ratio {greedy / fixed:.3f}), "
        f"rtn {rtn:.4e}")
    assert greedy < rtn and fixed < rtn
    if law == "corr":
        assert greedy < 0.9 * fixed
    else:
        assert abs(greedy / fixed - 1.0) < 0.25
