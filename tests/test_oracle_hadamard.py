"""Pins of the oracle's channel rotation against closed forms and scipy.

Pages: KVarN summary (fig1.dev) "What it is"; KVarN KV Cache: Implementation
and Benchmarks (anbeeld.com) §1 -- a per-head Hadamard rotation of K and V;
the query is rotated by the same matrix, which leaves q.k unchanged.
"""
import numpy as np
import pytest
import scipy.linalg

from oracle import kvarn_oracle as O


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_sylvester_matches_scipy(d):
    # scipy.linalg.hadamard builds the Sylvester matrix in natural order.
    assert np.array_equal(O.sylvester(d), scipy.linalg.hadamard(d))


@pytest.mark.parametrize("d", [2, 8, 128, 256])
def test_hadamard_orthogonality_exact(d):
    h = O.sylvester(d)
    assert np.array_equal(h @ h.T, d * np.eye(d, dtype=np.int64))
    assert np.all(h[0] == 1) and np.all(h[:, 0] == 1)
    # every other row sums to zero: H 1 = d e0
    assert np.array_equal(h @ np.ones(d, dtype=np.int64), d * np.eye(d, dtype=np.int64)[0])


@pytest.mark.parametrize("d", [128, 256])
def test_rotation_symmetric_orthonormal(d):
    r = O.rotation(d)
    assert np.array_equal(r, r.T)
    assert np.abs(r @ r - np.eye(d)).max() < 1e-13


def test_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        O.sylvester(96)


@pytest.mark.parametrize("d", [128, 256])
def test_qk_invariance_and_norm(d):
    rng = np.random.default_rng(5)
    q = rng.standard_normal(d)
    k = rng.standard_normal((64, d)) * 7.0
    qr = O.rotate_rows(q[None])[0]
    kr = O.rotate_rows(k)
    assert np.abs(kr @ qr - k @ q).max() < 1e-10
    assert np.abs(np.linalg.norm(kr, axis=1) - np.linalg.norm(k, axis=1)).max() < 1e-10


def test_outlier_channel_is_spread():
    # One large channel becomes D entries of equal magnitude after rotation.
    d = 128
    x = np.zeros((1, d))
    x[0, 37] = 50.0
    xr = O.rotate_rows(x)
    assert np.allclose(np.abs(xr), 50.0 / np.sqrt(d), rtol=0, atol=1e-12)
