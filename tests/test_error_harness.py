"""Pins of the error-accumulation harness (tests/error_harness.py) and of the
comparison quantizers it adds to the oracle, against closed forms, the
oracle's own pinned routines and limiting cases (CPU only)."""
import numpy as np
import pytest

from kv_cache_quantization_seal_amd import synth
from oracle import kvarn_oracle as O
from tests import error_harness as H


def test_tv_distance_closed_forms():
    p = np.array([0.5, 0.25, 0.25])
    assert H.tv_distance(p, p) == 0.0
    assert H.tv_distance(np.array([1.0, 0.0]), np.array([0.0, 1.0])) == 1.0
    assert H.tv_distance(p, np.array([0.25, 0.25, 0.5])) == pytest.approx(0.25, abs=1e-15)


def test_weights_are_the_oracle_softmax():
    # attention over identity value rows returns the weights themselves
    rng = np.random.default_rng(1)
    k = rng.standard_normal((7, 16))
    q = rng.standard_normal(16)
    w = H.weights(q, k)
    assert np.allclose(w, O.attention(q, k, np.eye(7)), atol=1e-14)
    assert w.sum() == pytest.approx(1.0, abs=1e-14)


@pytest.mark.parametrize("bits", [2, 4])
def test_fake_quant_rtn_is_the_pinned_rtn(bits):
    x = synth.gaussian_tile(5, 128, 128)
    y = x.astype(np.float64)
    # per-token: the oracle's RTN codes, reconstructed with the fp16 step
    codes, delta, mid = O.rtn(y, bits)
    ref = (codes.astype(np.float64) - mid) * delta.astype(np.float16).astype(np.float64)[:, None]
    assert np.array_equal(O.fake_quant_rtn(x, bits, "token"), ref)
    # per-channel = per-token of the transpose
    codes_t, delta_t, _ = O.rtn(y.T, bits)
    ref_t = ((codes_t.astype(np.float64) - mid) * delta_t.astype(np.float16).astype(np.float64)[:, None]).T
    assert np.array_equal(O.fake_quant_rtn(x, bits, "channel"), ref_t)
    # error bound: half a step (plus the fp16 rounding of the step)
    err = np.abs(O.fake_quant_rtn(x, bits, "channel", scale16=False) - y)
    assert np.all(err <= delta_t[None, :] / 2 * (1 + 1e-12))


@pytest.mark.parametrize("bits,kind", [(2, "k"), (4, "v")])
def test_rotation_only_kvarn_is_rotated_per_token_rtn(bits, kind):
    # With 0 iterations r = c = 1, so KVarN's record is per-token RTN in the
    # Hadamard frame; the two fake-quantizers must agree.
    x = synth.gaussian_tile(6, 128, 128)
    a = O.fake_quant_kvarn(x, bits, kind, iters=0)
    b = O.fake_quant_rtn(x, bits, "token", rotate=True)
    assert np.allclose(a, b, atol=1e-12 * np.abs(b).max())


def test_no_sealed_group_means_no_error():
    # 255 tokens: sink + 127 tail tokens, nothing sealed; every method reads
    # the exact cache.
    errs = H.open_loop(0, steps=8, prompt=247)
    for m in H.METHODS:
        tv, out = errs[m]
        assert np.all(tv == 0) and np.all(out == 0), m


def test_open_loop_errors_shrink_with_width():
    e2 = H.open_loop(1, bits=(2, 2), steps=16)
    e8 = H.open_loop(1, bits=(8, 8), steps=16)
    for m in H.METHODS:
        assert e8[m][1].mean() < 0.1 * e2[m][1].mean(), m
        assert e8[m][0].mean() < 0.1 * e2[m][0].mean(), m


def test_closed_loop_feedback():
    # The exact cache reproduces its own trajectory; a quantized cache moves
    # it, more at 2 bits than at 8, and the drift persists once present.
    dec = H.ToyDecoder(3)
    h0, _ = dec.run("exact", steps=64)
    h1, _ = dec.run("exact", steps=64)
    assert np.array_equal(h0, h1)
    d2 = H.closed_loop(3, bits=(2, 2), steps=64)
    d8 = H.closed_loop(3, bits=(8, 8), steps=64)
    for m in H.METHODS:
        assert d2[m][-1] > 0 and d8[m][-1] < d2[m][-1], m
