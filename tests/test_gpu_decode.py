"""GPU decode attention vs the oracle.

Decode is checked on caches the oracle built (sink, tail and records encoded
by the oracle, so independent of the GPU seal), over ragged lengths, GQA
ratios 1/2/4, head dims 128/256 and every ordered K/V width pair (2, 3, 4,
5, 6, 8 bits).
Tolerance: 2e-3 max-abs on the fp32 output.
"""
import numpy as np
import pytest
import torch

from kv_cache_quantization_seal_amd import kvarn as K
from kv_cache_quantization_seal_amd import synth
from oracle import kvarn_oracle as O
from tests.gpu_util import ATTN_ATOL, upload_states

pytestmark = pytest.mark.gpu


def _case(d, hq, hkv, kb, vb, lens, seed):
    wl = synth.Workload("t", 90 + seed, len(lens), hq, hkv, d, max(lens), 0, kb, vb, 0)
    states, qs = [], []
    for b, n in enumerate(lens):
        row = []
        for h in range(hkv):
            k, v = synth.kv_stream(wl, b, h, max(n, 1))
            row.append(O.state_from_stream(k[:n], v[:n], kb, vb))
        states.append(row)
        qs.append(synth.queries(wl, b, 1)[0])
    return states, np.stack(qs)


def _run(d, hq, hkv, kb, vb, lens, seed=0, max_groups=None):
    states, q = _case(d, hq, hkv, kb, vb, lens, seed)
    if max_groups is None:
        max_groups = max(1, max((n - 128) // 128 for n in lens) + 1)
    cfg = K.make_config(d, hq, hkv, kb, vb)
    cache = K.KVarNCache(cfg, len(lens), max_groups)
    upload_states(cache, states)
    out = cache.decode_attn(torch.from_numpy(q).cuda())
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    err = 0.0
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(out[b] == 0)
            continue
        ref = O.decode_attention(q[b], states[b], hkv)
        err = max(err, np.abs(out[b] - ref).max())
    return err


def test_tiny_parity_workload():
    wl = synth.WORKLOADS["tiny_parity"]
    k, v = synth.kv_stream(wl, 0, 0, 512)
    q = synth.queries(wl, 0, 1)[0]
    st = O.state_from_stream(k, v, 2, 2)
    cfg = K.make_config(128, 1, 1, 2, 2)
    cache = K.KVarNCache(cfg, 1, 3)
    upload_states(cache, [[st]])
    out = cache.decode_attn(torch.from_numpy(q[None]).cuda()).cpu().numpy()[0]
    ref = O.decode_attention(q, [st], 1)
    err = np.abs(out - ref).max()
    print(f"tiny parity max abs err {err:.3e}")
    assert err <= ATTN_ATOL


@pytest.mark.parametrize("lens", [[1], [128], [129], [255], [256], [300, 77, 513], [1000, 0, 640]])
def test_ragged_lengths_gqa4(lens):
    err = _run(128, 8, 2, 2, 2, lens, seed=len(lens))
    print(f"lens={lens}: max abs err {err:.3e}")
    assert err <= ATTN_ATOL


@pytest.mark.parametrize("d,hq,hkv,kb,vb", [
    (128, 4, 4, 2, 2), (128, 4, 2, 4, 4), (128, 8, 2, 2, 4), (128, 8, 2, 4, 2),
    (256, 4, 2, 4, 2), (256, 4, 1, 2, 2), (256, 2, 2, 4, 4),
    # widths 3, 5, 6, 8 and the asymmetric presets 3-2, 5-4, 6-5
    (128, 8, 2, 3, 3), (128, 4, 2, 5, 5), (128, 4, 4, 6, 6), (128, 8, 2, 8, 8),
    (128, 8, 2, 3, 2), (128, 4, 1, 5, 4), (128, 8, 2, 6, 5),
    (256, 4, 2, 3, 3), (256, 2, 2, 5, 4), (256, 4, 1, 6, 5), (256, 4, 2, 8, 8),
])
def test_shapes_and_widths(d, hq, hkv, kb, vb):
    err = _run(d, hq, hkv, kb, vb, [700, 389], seed=d + kb * 10 + vb)
    print(f"d={d} hq={hq} hkv={hkv} k{kb} v{vb}: max abs err {err:.3e}")
    assert err <= ATTN_ATOL


WIDTHS = (2, 3, 4, 5, 6, 8)


@pytest.mark.parametrize("kb", WIDTHS)
@pytest.mark.parametrize("vb", WIDTHS)
def test_every_width_pair_d128(kb, vb):
    # every ordered (K, V) pair: 2 requests, GQA 2, three groups and a tail
    err = _run(128, 4, 2, kb, vb, [550, 301], seed=100 + 10 * kb + vb)
    print(f"d=128 k{kb} v{vb}: max abs err {err:.3e}")
    assert err <= ATTN_ATOL


@pytest.mark.parametrize("kb,vb", [(2, 8), (8, 2), (3, 6), (6, 3), (5, 2), (2, 5), (4, 6), (8, 4)])
def test_width_pairs_d256(kb, vb):
    err = _run(256, 4, 1, kb, vb, [420], seed=200 + 10 * kb + vb)
    print(f"d=256 k{kb} v{vb}: max abs err {err:.3e}")
    assert err <= ATTN_ATOL


def test_many_groups_one_request():
    err = _run(128, 4, 1, 2, 2, [128 + 128 * 40 + 17], seed=5)
    print(f"41 groups: max abs err {err:.3e}")
    assert err <= ATTN_ATOL


def test_spare_capacity_is_ignored():
    # max_groups larger than any request needs; unused record slots hold junk.
    err = _run(128, 4, 2, 2, 2, [400, 200], seed=6, max_groups=9)
    assert err <= ATTN_ATOL


def test_two_phase_equals_fused():
    d, hq, hkv, kb, vb = 128, 8, 2, 2, 2
    lens = [900, 300]
    states, q = _case(d, hq, hkv, kb, vb, lens, 11)
    cfg = K.make_config(d, hq, hkv, kb, vb)
    cache = K.KVarNCache(cfg, len(lens), 7)
    upload_states(cache, states)
    qd = torch.from_numpy(q).cuda()
    fused = cache.decode_attn(qd).clone()
    cache.decode_partial(qd)
    two = cache.decode_combine(torch.empty_like(fused))
    again = cache.decode_attn(qd)   # counters were left at zero
    torch.cuda.synchronize()
    assert torch.allclose(fused, two, atol=1e-6, rtol=1e-5)
    assert torch.equal(fused, again)


@pytest.mark.parametrize("hq,kb,vb", [(32, 2, 2), (16, 4, 4)])
def test_many_pairs(hq, kb, vb):
    # 16 requests x 8 KV heads = 128 pairs: four exact workgroups per pair
    # would hold more than half of the resident slots, so the plan takes two
    # exact splits of 128 tokens (two rounds per wave) per pair.  Lengths
    # cover an empty request, sink-only, exact tail lengths and group edges.
    lens = [0, 1, 128, 129, 200, 255, 256, 300, 383, 384, 400, 511, 512, 513, 600, 640]
    err = _run(128, hq, 8, kb, vb, lens, seed=hq + kb)
    print(f"128 pairs hq={hq} k{kb} v{vb}: max abs err {err:.3e}")
    assert err <= ATTN_ATOL


def test_grid_rounded_to_whole_cus():
    # 2 requests x 4 KV heads with capacity for 130 groups plans 33 record
    # splits per pair (264 workgroups, just above one per CU on a 256-CU
    # device), which the plan rounds down to 32: each record wave then takes
    # one or two of a request's 129 sealed groups.
    lens = [128 + 128 * 129 + 5, 128 + 128 * 100 + 77]
    err = _run(128, 16, 4, 2, 2, lens, seed=13, max_groups=130)
    print(f"rounded grid: max abs err {err:.3e}")
    assert err <= ATTN_ATOL


def test_more_splits_than_the_combine_batch():
    # One pair with 511 sealed groups plans over 80 splits (128 record + 4
    # exact), so the combine also takes its loop over the splits past its
    # first batch of loads.
    err = _run(128, 4, 1, 2, 2, [128 + 128 * 511 + 37], seed=17)
    print(f"511 groups, one pair: max abs err {err:.3e}")
    assert err <= ATTN_ATOL


def test_waves_of_three_groups():
    # 4 requests x 2 KV heads, capacity 701 groups: the plan gives each
    # record wave up to three groups (one stage refilled twice); the other
    # requests leave their waves with zero or one group.
    lens = [128 + 128 * 700 + 7, 200, 0, 129 + 128]
    err = _run(128, 8, 2, 2, 2, lens, seed=19, max_groups=701)
    print(f"waves of three groups: max abs err {err:.3e}")
    assert err <= ATTN_ATOL
