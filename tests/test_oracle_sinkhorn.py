"""Pins of the oracle's Sinkhorn-style variance normalization.

Pages: KVarN summary (fig1.dev) "What it is" (iterative normalization over the
token and channel axes before rounding); KVarN KV Cache: Implementation and
Benchmarks (anbeeld.com) §1 (both axes rescaled; 16 Sinkhorn iterations).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from kv_cache_quantization_seal_amd import synth
from oracle import kvarn_oracle as O


def _tile(seed=0, d=128):
    return O.rotate_rows(synth.gaussian_tile(seed, 128, d).astype(np.float64))


def test_rank_one_balanced_after_one_iteration():
    rng = np.random.default_rng(1)
    a = rng.standard_normal(128) * rng.lognormal(0, 1, 128)
    b = rng.standard_normal(128) * 3
    xr = np.outer(a, b)
    for iters in (1, 16):
        y, r, c = O.sinkhorn(xr, iters)
        assert np.abs(np.abs(y) - 1.0).max() < 1e-12


def test_last_half_step_is_the_channel_step():
    # Row first, then column: after any whole number of iterations the column
    # mean squares are exactly 1 while rows are only close to 1.
    xr = _tile(2)
    for iters in (1, 2, 16):
        y, _, _ = O.sinkhorn(xr, iters)
        assert np.abs(np.mean(y * y, axis=0) - 1.0).max() < 1e-12
    y1, _, _ = O.sinkhorn(xr, 1)
    assert np.abs(np.mean(y1 * y1, axis=1) - 1.0).max() > 1e-3


def test_factors_reproduce_the_tile():
    xr = _tile(3)
    y, r, c = O.sinkhorn(xr)
    assert np.abs(xr / np.outer(r, c) - y).max() < 1e-12


def test_imbalance_monotone_and_converging():
    # max/min over all row and column mean squares never grows and tends to 1.
    xr = _tile(0)
    hist = []
    O.sinkhorn(xr, 16, history=hist)
    imb = []
    for _, rows, cols in hist:
        allms = np.concatenate([rows, cols])
        imb.append(allms.max() / allms.min())
    assert imb[0] > 10.0
    assert all(b <= a * (1 + 1e-12) for a, b in zip(imb, imb[1:]))
    assert imb[-1] < 1.001


def _two_by_two_ratio_recursion(x, iters):
    """Closed-form 2x2 Sinkhorn on squared entries via the cross-ratio.

    For B = Y*Y, a row step leaves the ratio x_t = B_t0/B_t1 of each row
    unchanged and sets the row mean to 1: row t = (2x_t/(1+x_t), 2/(1+x_t)).
    A column step multiplies column j by 2/colsum_j, so both ratios get the
    factor colsum_1/colsum_0, while the cross-ratio x_0/x_1 never changes.
    Running c_j^2 collects the inverse column factors; r_t^2 is recovered from
    the first row of the input at the end.  Exact rational arithmetic.
    """
    b = [[Fraction(v) ** 2 for v in row] for row in x]
    x0 = b[0][0] / b[0][1]
    x1 = b[1][0] / b[1][1]
    c2 = [Fraction(1), Fraction(1)]
    bfinal = None
    for _ in range(iters):
        rows = [(2 * xt / (1 + xt), 2 / (1 + xt)) for xt in (x0, x1)]
        col0 = rows[0][0] + rows[1][0]
        col1 = rows[0][1] + rows[1][1]
        c2 = [c2[0] * col0 / 2, c2[1] * col1 / 2]
        bfinal = [[rows[t][0] * 2 / col0, rows[t][1] * 2 / col1] for t in range(2)]
        x0 = x0 * col1 / col0
        x1 = x1 * col1 / col0
    return bfinal, c2


@pytest.mark.parametrize("iters", [1, 2, 7, 16])
def test_two_by_two_closed_form(iters):
    # A slowly balancing tile (cross-ratio far from 1) so the count matters.
    xr = np.array([[9.0, 0.05], [0.3, 2.0]])
    y, r, c = O.sinkhorn(xr, iters)
    bfinal, c2 = _two_by_two_ratio_recursion([[9, Fraction(1, 20)], [Fraction(3, 10), 2]], iters)
    assert np.abs(y * y - np.array([[float(v) for v in row] for row in bfinal])).max() < 1e-12
    assert np.abs(c * c / np.array([float(v) for v in c2]) - 1.0).max() < 1e-12


def test_two_by_two_iteration_count_is_visible():
    xr = np.array([[9.0, 0.05], [0.3, 2.0]])
    _, _, c15 = O.sinkhorn(xr, 15)
    _, _, c16 = O.sinkhorn(xr, 16)
    _, _, cdef = O.sinkhorn(xr)
    assert np.array_equal(c16, cdef)
    assert np.abs(c15 / c16 - 1).max() > 1e-7


def test_zero_row_and_column_keep_unit_factor():
    xr = _tile(4)
    xr[5, :] = 0.0
    xr[:, 17] = 0.0
    y, r, c = O.sinkhorn(xr)
    assert r[5] == 1.0 and c[17] == 1.0
    assert np.all(np.isfinite(y)) and np.all(y[5] == 0) and np.all(y[:, 17] == 0)


def test_token_power_of_two_scaling_is_exact():
    x = synth.gaussian_tile(7, 128, 128)
    x2 = x.copy()
    x2[9] = (x2[9].astype(np.float32) * 8).astype(np.float16)   # exact x2^3
    a = O.seal_tile(x, 2)
    b = O.seal_tile(x2, 2)
    assert np.array_equal(a["codes"], b["codes"])
    assert np.array_equal(a["c"], b["c"])
    assert b["s"][9] == 8 * a["s"][9]
    others = np.arange(128) != 9
    assert np.array_equal(a["s"][others], b["s"][others])


def test_token_permutation_equivariance():
    x = synth.gaussian_tile(8, 128, 128)
    perm = np.random.default_rng(0).permutation(128)
    a = O.seal_tile(x, 4)
    b = O.seal_tile(x[perm], 4)
    assert np.abs(b["s"] / a["s"][perm] - 1).max() < 1e-12
    assert np.abs(b["c"] / a["c"] - 1).max() < 1e-12
    assert (b["codes"] != a["codes"][perm]).mean() < 1e-4


def test_hand_derived_two_by_two_seal(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "tiny_seal_2x2.json")))
    x = np.array(g["x"], dtype=np.float16)
    out = O.seal_tile(x, g["bits"])
    assert np.abs(out["r"] / np.array(g["r"]) - 1).max() < 1e-12
    assert np.abs(out["c"] / np.array(g["c"]) - 1).max() < 1e-12
    assert np.array_equal(out["codes"], np.array(g["codes"]))
    assert np.abs(out["s"] / np.array(g["s"]) - 1).max() < 1e-12
