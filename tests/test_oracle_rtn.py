"""Pins of the oracle's round-to-nearest step (KVarN summary, fig1.dev,
"What it is": round to nearest after normalization) by brute force."""
import numpy as np
import pytest

from oracle import kvarn_oracle as O


def _brute(y, bits):
    levels = (1 << bits) - 1
    mid = levels / 2
    out = np.empty(y.shape, dtype=np.uint8)
    for t in range(y.shape[0]):
        m = np.abs(y[t]).max()
        if m == 0:
            out[t] = 1 << (bits - 1)
            continue
        delta = 2 * m / levels
        for j in range(y.shape[1]):
            u = y[t, j] / delta
            best = None
            for k in range(levels + 1):
                dist = abs(u - (k - mid))
                if best is None or dist < best[0] - 1e-15 or (abs(dist - best[0]) <= 1e-15 and k % 2 == 0):
                    best = (dist, k)
            out[t, j] = best[1]
    return out


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
def test_brute_force_tiny_tiles(bits):
    rng = np.random.default_rng(bits)
    levels = (1 << bits) - 1
    for _ in range(20):
        y = rng.standard_normal((4, 8))
        # inject exact ties: u = k - mid + 0.5 (with delta from the row max)
        m = np.abs(y[0]).max()
        delta = 2 * m / levels
        y[0, 1] = delta * (0.5 - ((levels // 2) - 0))  # a half-way point
        y[0, 2] = delta * 0.5 * (1 if bits == 2 else 3)
        codes, d, mid = O.rtn(y, bits)
        assert np.array_equal(codes, _brute(y, bits))


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
def test_error_bound_and_extremes(bits):
    rng = np.random.default_rng(10 + bits)
    y = rng.standard_normal((128, 128)) * rng.lognormal(0, 1, (128, 1))
    codes, delta, mid = O.rtn(y, bits)
    err = np.abs(y - delta[:, None] * (codes - mid))
    assert np.all(err <= delta[:, None] / 2 * (1 + 1e-12))
    levels = (1 << bits) - 1
    am = np.argmax(np.abs(y), axis=1)
    ext = codes[np.arange(128), am]
    assert np.all((ext == 0) | (ext == levels))
    assert codes.max() <= levels


def test_zero_row():
    y = np.zeros((2, 8))
    y[1, 3] = 1.0
    for bits in (2, 4):
        codes, delta, _ = O.rtn(y, bits)
        assert np.all(codes[0] == 1 << (bits - 1)) and delta[0] == 0
