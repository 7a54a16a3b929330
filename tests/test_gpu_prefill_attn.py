"""GPU chunked-prefill attention (kvarn_prefill_attn) vs the oracle's
prefill_attention: the last `chunk` cached positions of each request attend
causally over the cache as it holds them (sink and tail exact, sealed groups
through their records).  Caches are built by the oracle and uploaded, so the
test is independent of the GPU seal.  Tolerance: 2e-3 max-abs on the fp32
output.
"""
import numpy as np
import pytest
import torch

from kv_cache_quantization_seal_amd import kvarn as K
from kv_cache_quantization_seal_amd import synth
from oracle import kvarn_oracle as O
from tests.gpu_util import ATTN_ATOL, upload_states

pytestmark = pytest.mark.gpu


def _states(d, hkv, kb, vb, lens, wid):
    wl = synth.Workload("pa", wid, len(lens), hkv, hkv, d, max(lens), 0, kb, vb, 0)
    states = []
    for b, n in enumerate(lens):
        row = []
        for h in range(hkv):
            k, v = synth.kv_stream(wl, b, h, max(n, 1))
            row.append(O.state_from_stream(k[:n], v[:n], kb, vb))
        states.append(row)
    return states


@pytest.mark.parametrize("d,hq,hkv,kb,vb,lens,chunk", [
    (128, 4, 1, 2, 2, [700], 70),          # chunk crosses from the last sealed group into the tail
    (128, 8, 2, 4, 2, [300, 513], 37),     # ragged batch, GQA 4
    (128, 2, 1, 3, 5, [260], 200),         # chunk spans sink, a sealed group and the tail; GQA 2
    (128, 4, 4, 2, 2, [129, 50], 100),     # chunk longer than request 1's cache: its first rows are unwritten
    (128, 4, 2, 2, 2, [255], 255),         # all exact (no sealed group): the whole prompt as one chunk
    (256, 2, 2, 2, 4, [600], 64),          # head dim 256, GQA 1
    (256, 4, 1, 4, 2, [640, 383], 129),    # head dim 256, GQA 4, a chunk of exactly one group + 1
    (128, 8, 2, 8, 6, [1000], 300),        # wide widths, many record tiles in the chunk
])
def test_prefill_attn_matches_oracle(d, hq, hkv, kb, vb, lens, chunk):
    states = _states(d, hkv, kb, vb, lens, 400 + d + kb + vb + chunk)
    cfg = K.make_config(d, hq, hkv, kb, vb)
    mg = max(1, max((n - 128) // 128 for n in lens) + 1)
    cache = K.KVarNCache(cfg, len(lens), mg)
    upload_states(cache, states)
    q = np.random.default_rng(chunk + d).standard_normal((len(lens), chunk, hq, d)).astype(np.float16)
    sentinel = 12345.0
    out = torch.full(q.shape, sentinel, dtype=torch.float32, device="cuda")
    cache.prefill_attn(torch.from_numpy(q).cuda(), out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    worst = 0.0
    for b, n in enumerate(lens):
        c = min(chunk, n)
        ref = O.prefill_attention(q[b, chunk - c:], states[b], hkv)
        worst = max(worst, float(np.abs(got[b, chunk - c:] - ref).max()))
        # rows whose position would be negative are not written
        assert np.all(got[b, :chunk - c] == sentinel)
    print(f"d={d} hq={hq} hkv={hkv} k{kb} v{vb} lens={lens} chunk={chunk}: max abs err {worst:.3e}")
    assert worst <= ATTN_ATOL


def test_prefill_attn_last_row_equals_decode():
    # The chunk's last query sees the whole cache, as a decode query does.
    d, hq, hkv = 128, 8, 2
    lens = [900, 451]
    states = _states(d, hkv, 2, 2, lens, 480)
    cfg = K.make_config(d, hq, hkv, 2, 2)
    cache = K.KVarNCache(cfg, len(lens), 7)
    upload_states(cache, states)
    q = torch.from_numpy(np.random.default_rng(3).standard_normal((2, 16, hq, d)).astype(np.float16)).cuda()
    pa = cache.prefill_attn(q)
    dec = cache.decode_attn(q[:, -1].contiguous())
    torch.cuda.synchronize()
    assert float((pa[:, -1] - dec).abs().max()) <= 1e-4


def test_prefill_attn_full_size_sampled():
    """Llama-3.1-8B shape (32 q / 8 KV heads, D 128, 2-bit): the benchmark's
    2,048-token chunk at the end of a 32k context (eight-wave workgroups),
    built on the GPU by the bulk seal; sampled rows of two KV heads checked
    against the oracle (its own seal of the sampled heads' streams)."""
    wl = synth.WORKLOADS["llama31_8b_32k"]
    dev = torch.device("cuda:0")
    n, chunk = wl.context, 2048
    pairs = [(0, 0), (0, 5)]
    Kd, Vd = synth.kv_streams_device(wl, n, dev, pairs_from_host=pairs)
    cfg = K.make_config(wl.head_dim, wl.num_q_heads, wl.num_kv_heads, wl.k_bits, wl.v_bits)
    cache = K.KVarNCache(cfg, 1, wl.max_groups(), device=dev)
    cache.prefill(Kd, Vd, [n])
    q = np.random.default_rng(11).standard_normal((1, chunk, wl.num_q_heads, wl.head_dim)).astype(np.float16)
    out = cache.prefill_attn(torch.from_numpy(q).to(dev)).cpu().numpy()
    gq = wl.num_q_heads // wl.num_kv_heads
    worst = 0.0
    for b, h in pairs:
        k, v = synth.kv_stream(wl, b, h, n)
        st = O.state_from_stream(k, v, wl.k_bits, wl.v_bits)
        kall, vall = st.materialize()
        for i in (0, 1, 255, 256, 1023, 1024, 2046, 2047):
            p = n - chunk + i
            for hh in range(gq):
                ref = O.attention(q[0, i, h * gq + hh], kall[:p + 1], vall[:p + 1])
                worst = max(worst, float(np.abs(out[0, i, h * gq + hh] - ref).max()))
    print(f"llama 32k chunk 2048: sampled max abs err {worst:.3e}")
    assert worst <= ATTN_ATOL


def test_prefill_attn_paged_with_absent_group():
    """Block-table cache (shuffled blocks of a shared pool) with one table
    entry outside the pool: that group has no storage and every query skips
    its 128 positions; the other positions keep their places (the reference
    attends over the oracle's full materialization minus that group)."""
    d, hq, hkv, kb, vb = 128, 8, 2, 2, 4
    lens, chunk, mg = [700, 460], 300, 5
    B = len(lens)
    states = _states(d, hkv, kb, vb, lens, 470)
    cfg = K.make_config(d, hq, hkv, kb, vb)
    nblk = B * mg + 3
    cache = K.KVarNCache(cfg, B, mg, num_blocks=nblk)
    table = np.random.default_rng(5).permutation(nblk)[:B * mg].astype(np.int32).reshape(B, mg)
    absent = (0, 2)   # request 0, group 2: positions 384 .. 511
    table[absent] = -1
    cache.block_table.copy_(torch.from_numpy(table))
    dev = cache.sink_k.device
    for b, row in enumerate(states):
        for h, st in enumerate(row):
            cache.sink_k[b, h, :len(st.sink_k)] = torch.from_numpy(np.stack(st.sink_k)).to(dev)
            cache.sink_v[b, h, :len(st.sink_v)] = torch.from_numpy(np.stack(st.sink_v)).to(dev)
            if st.tail_k:
                cache.tail_k[b, h, :st.tail_len] = torch.from_numpy(np.stack(st.tail_k)).to(dev)
                cache.tail_v[b, h, :st.tail_len] = torch.from_numpy(np.stack(st.tail_v)).to(dev)
            for g, (rk, rv) in enumerate(zip(st.rec_k, st.rec_v)):
                if (b, g) != absent:
                    cache.record(b, h, g, "k").copy_(torch.frombuffer(bytearray(rk), dtype=torch.uint8).to(dev))
                    cache.record(b, h, g, "v").copy_(torch.frombuffer(bytearray(rv), dtype=torch.uint8).to(dev))
    cache.seq_len.copy_(torch.tensor(lens, dtype=torch.int32, device=dev))
    q = np.random.default_rng(8).standard_normal((B, chunk, hq, d)).astype(np.float16)
    out = cache.prefill_attn(torch.from_numpy(q).to(dev)).cpu().numpy()
    gq = hq // hkv
    worst = 0.0
    for b, n in enumerate(lens):
        mats = [st.materialize() for st in states[b]]
        keep = np.ones(n, dtype=bool)
        if b == absent[0]:
            keep[128 + 128 * absent[1]:256 + 128 * absent[1]] = False
        for i in range(0, chunk, 7):
            p = n - chunk + i
            sel = np.flatnonzero(keep[:p + 1])
            for h in range(hq):
                kall, vall = mats[h // gq]
                ref = O.attention(q[b, i, h], kall[sel], vall[sel])
                worst = max(worst, float(np.abs(out[b, i, h] - ref).max()))
    print(f"paged, absent group: max abs err {worst:.3e}")
    assert worst <= ATTN_ATOL


@pytest.mark.parametrize("kb,vb,lens", [
    (2, 4, [2100, 1900]),   # two requests, tails of 52 and 108 tokens
    (6, 5, [2200, 700]),    # wide codes; the second request's chunk starts before its cache
])
def test_prefill_attn_eight_wave_grid(kb, vb, lens):
    """A grid large enough for eight-wave workgroups (at least one per CU):
    8 KV heads x GQ 4, a 2,048-token chunk; every 41st row of every head
    against the oracle, and rows before a request's first position left
    untouched."""
    d, hq, hkv, chunk = 128, 32, 8, 2048
    states = _states(d, hkv, kb, vb, lens, 900 + kb + vb)
    cfg = K.make_config(d, hq, hkv, kb, vb)
    mg = max((n - 128) // 128 for n in lens) + 1
    cache = K.KVarNCache(cfg, len(lens), mg)
    upload_states(cache, states)
    q = np.random.default_rng(kb * 10 + vb).standard_normal((len(lens), chunk, hq, d)).astype(np.float16)
    sentinel = 12345.0
    out = torch.full(q.shape, sentinel, dtype=torch.float32, device="cuda")
    cache.prefill_attn(torch.from_numpy(q).cuda(), out=out)
    got = out.cpu().numpy()
    gq = hq // hkv
    worst = 0.0
    for b, n in enumerate(lens):
        c = min(chunk, n)
        assert np.all(got[b, :chunk - c] == sentinel)
        mats = [st.materialize() for st in states[b]]
        for i in range(chunk - c, chunk, 41):
            p = n - chunk + i
            for h in range(hq):
                kall, vall = mats[h // gq]
                ref = O.attention(q[b, i, h], kall[:p + 1], vall[:p + 1])
                worst = max(worst, float(np.abs(got[b, i, h] - ref).max()))
    print(f"eight-wave grid k{kb} v{vb} lens={lens}: sampled max abs err {worst:.3e}")
    assert worst <= ATTN_ATOL


def test_prefill_attn_eight_wave_paged_absent_groups():
    """Eight-wave workgroups over a block-table cache with two entries outside
    the pool: request 0's first sealed group (so the first record tile has no
    storage and its c^K buffer is never staged) and a middle group of request
    1.  Every query skips those 128 positions; every 41st row of every head
    against the oracle's materialization without them."""
    d, hq, hkv, kb, vb, chunk = 128, 32, 8, 2, 2, 2048
    lens = [2100, 2080]   # both longer than the chunk: every row has a position
    B = len(lens)
    mg = max((n - 128) // 128 for n in lens) + 1
    states = _states(d, hkv, kb, vb, lens, 930)
    cfg = K.make_config(d, hq, hkv, kb, vb)
    nblk = B * mg + 2
    cache = K.KVarNCache(cfg, B, mg, num_blocks=nblk)
    table = np.random.default_rng(17).permutation(nblk)[:B * mg].astype(np.int32).reshape(B, mg)
    absent = [(0, 0), (1, 6)]
    for r, g in absent:
        table[r, g] = nblk + 5   # past the pool: no storage
    cache.block_table.copy_(torch.from_numpy(table))
    dev = cache.sink_k.device
    for b, row in enumerate(states):
        for h, st in enumerate(row):
            cache.sink_k[b, h, :len(st.sink_k)] = torch.from_numpy(np.stack(st.sink_k)).to(dev)
            cache.sink_v[b, h, :len(st.sink_v)] = torch.from_numpy(np.stack(st.sink_v)).to(dev)
            if st.tail_k:
                cache.tail_k[b, h, :st.tail_len] = torch.from_numpy(np.stack(st.tail_k)).to(dev)
                cache.tail_v[b, h, :st.tail_len] = torch.from_numpy(np.stack(st.tail_v)).to(dev)
            for g, (rk, rv) in enumerate(zip(st.rec_k, st.rec_v)):
                if (b, g) not in absent:
                    cache.record(b, h, g, "k").copy_(torch.frombuffer(bytearray(rk), dtype=torch.uint8).to(dev))
                    cache.record(b, h, g, "v").copy_(torch.frombuffer(bytearray(rv), dtype=torch.uint8).to(dev))
    cache.seq_len.copy_(torch.tensor(lens, dtype=torch.int32, device=dev))
    q = np.random.default_rng(19).standard_normal((B, chunk, hq, d)).astype(np.float16)
    out = cache.prefill_attn(torch.from_numpy(q).to(dev)).cpu().numpy()
    assert np.isfinite(out).all()
    gq = hq // hkv
    worst = 0.0
    for b, n in enumerate(lens):
        mats = [st.materialize() for st in states[b]]
        keep = np.ones(n, dtype=bool)
        for r, g in absent:
            if r == b:
                keep[128 + 128 * g:256 + 128 * g] = False
        for i in range(0, chunk, 41):
            p = n - chunk + i
            sel = np.flatnonzero(keep[:p + 1])
            for h in range(hq):
                kall, vall = mats[h // gq]
                ref = O.attention(q[b, i, h], kall[sel], vall[sel])
                worst = max(worst, float(np.abs(out[b, i, h] - ref).max()))
    print(f"eight-wave grid, paged with absent groups: sampled max abs err {worst:.3e}")
    assert worst <= ATTN_ATOL
