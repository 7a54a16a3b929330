"""GPU decode step (kvarn_decode_step) against its definition: the same step
as kvarn_append_seal followed by kvarn_decode_attn.  Two caches built from
the same prompts take the same tokens and queries, one through
decode_step with host lengths (the append folded into the decode launches on
every step where no request completes a group), the other through the two
calls; every step's output and, at the end, every cache buffer must be
bit-identical.  Lengths cross the sink/tail border, complete groups (those
steps fall back to three launches) and reach capacity.  The two-call path
itself is held to the oracle by the decode and cache tests.
"""
import numpy as np
import pytest
import torch

from kv_cache_quantization_seal_amd import kvarn as K

pytestmark = pytest.mark.gpu


def _pair(cfg, batch, max_groups, lens, seed, num_blocks=None):
    g = torch.Generator(device="cuda").manual_seed(seed)
    n = max(max(lens), 1)
    shape = (batch, cfg.num_kv_heads, n, cfg.head_dim)
    k = torch.randn(shape, generator=g, device="cuda").half()
    v = torch.randn(shape, generator=g, device="cuda").half()
    caches = []
    for _ in range(2):
        c = K.KVarNCache(cfg, batch, max_groups, num_blocks=num_blocks)
        if num_blocks is not None:
            perm = torch.randperm(num_blocks, generator=torch.Generator().manual_seed(seed))[:batch * max_groups]
            c.block_table.copy_(perm.to(torch.int32).reshape(batch, max_groups))
        c.prefill(k, v, lens)
        caches.append(c)
    return caches


def _state(c):
    return [c.sink_k, c.sink_v, c.tail_k, c.tail_v, c.records, c.seq_len]


@pytest.mark.parametrize("d,hq,hkv,kb,vb,lens,mg,steps,paged", [
    (128, 8, 2, 2, 2, [0, 120, 250, 383, 1000], 8, 140, False),  # sink -> tail, seals, ragged
    (128, 4, 4, 3, 5, [127, 400], 2, 160, False),                  # reaches capacity (mg 2: 511 tokens)
    (256, 8, 4, 4, 2, [500, 130], 4, 100, False),                  # head dim 256
    (128, 8, 2, 4, 4, [300, 900, 20], 8, 130, True),               # paged records
    (256, 4, 4, 8, 8, [330, 140], 4, 60, False),                   # head dim 256, GQ 1, 8-bit codes
    (128, 16, 4, 6, 5, [129, 1500], 12, 80, False),                # wide codes, a long request
    (256, 8, 2, 2, 2, [0, 700], 6, 70, True),                      # paged, head dim 256, an empty request
])
def test_decode_step_equals_append_then_decode(d, hq, hkv, kb, vb, lens, mg, steps, paged):
    cfg = K.make_config(d, hq, hkv, kb, vb)
    B = len(lens)
    nblk = B * mg + 5 if paged else None
    fused, ref = _pair(cfg, B, mg, lens, 100 + d + steps, nblk)
    cap = fused.capacity
    g = torch.Generator(device="cuda").manual_seed(7)
    cur = list(lens)
    n_fold = 0
    for s in range(steps):
        kn = torch.randn((B, hkv, d), generator=g, device="cuda").half()
        vn = torch.randn((B, hkv, d), generator=g, device="cuda").half()
        q = torch.randn((B, hq, d), generator=g, device="cuda").half()
        out_f = fused.decode_step(kn, vn, q, lengths=cur)
        ref.append_seal(kn, vn)
        out_r = ref.decode_attn(q)
        torch.cuda.synchronize()
        assert torch.equal(out_f, out_r), f"step {s}: lengths {cur}"
        if all(n < cap and not (n + 1 >= 256 and (n + 1 - 128) % 128 == 0) for n in cur):
            n_fold += 1
        cur = [n + 1 if n < cap else n for n in cur]
    for a, b in zip(_state(fused), _state(ref)):
        assert torch.equal(a, b)
    assert fused.seq_len.cpu().tolist() == cur
    assert 0 < n_fold < steps
    print(f"d={d} lens={lens} mg={mg} paged={paged}: {steps} steps, {n_fold} with the append folded in")


def test_decode_step_without_lengths_is_the_two_calls():
    cfg = K.make_config(128, 4, 2, 2, 2)
    fused, ref = _pair(cfg, 2, 4, [200, 40], 5)
    g = torch.Generator(device="cuda").manual_seed(9)
    for _ in range(5):
        kn = torch.randn((2, 2, 128), generator=g, device="cuda").half()
        vn = torch.randn((2, 2, 128), generator=g, device="cuda").half()
        q = torch.randn((2, 4, 128), generator=g, device="cuda").half()
        out_f = fused.decode_step(kn, vn, q)
        ref.append_seal(kn, vn)
        assert torch.equal(out_f, ref.decode_attn(q))
    for a, b in zip(_state(fused), _state(ref)):
        assert torch.equal(a, b)


def test_decode_step_rejects_negative_length():
    cfg = K.make_config(128, 4, 2, 2, 2)
    c = K.KVarNCache(cfg, 2, 2)
    z = torch.zeros((2, 2, 128), dtype=torch.float16, device="cuda")
    q = torch.zeros((2, 4, 128), dtype=torch.float16, device="cuda")
    with pytest.raises(K.KvarnError):
        c.decode_step(z, z, q, lengths=[0, -1])
    torch.cuda.synchronize()
    assert c.seq_len.cpu().tolist() == [0, 0]


def test_decode_step_graph_replays():
    """Steps captured in a HIP graph (as the benchmark runs them), replayed
    three times with the lengths reset and eager work in between: every
    replay gives the eager steps' outputs and cache bit for bit (the folded
    append writes the cache from inside the split kernel; nothing in the
    step is a memset node)."""
    cfg = K.make_config(128, 8, 2, 2, 2)
    lens = [250, 383]   # the sixth step completes a group of request 0 (three launches)
    eager, graphed = _pair(cfg, 2, 4, lens, 21)
    g = torch.Generator(device="cuda").manual_seed(4)
    steps = 6
    kn = torch.randn((steps, 2, 2, 128), generator=g, device="cuda").half()
    vn = torch.randn((steps, 2, 2, 128), generator=g, device="cuda").half()
    q = torch.randn((steps, 2, 8, 128), generator=g, device="cuda").half()
    ref = [eager.decode_step(kn[s], vn[s], q[s], lengths=[n + s for n in lens]) for s in range(steps)]
    torch.cuda.synchronize()
    seq0 = graphed.seq_len.clone()
    tail0 = (graphed.tail_k.clone(), graphed.tail_v.clone(), graphed.records.clone())
    outs = [torch.empty((2, 8, 128), dtype=torch.float32, device="cuda") for _ in range(steps)]
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=st):
            for s in range(steps):
                graphed.decode_step(kn[s], vn[s], q[s], lengths=[n + s for n in lens], out=outs[s], stream=st)
    for rep in range(3):
        graphed.seq_len.copy_(seq0)
        graphed.tail_k.copy_(tail0[0])
        graphed.tail_v.copy_(tail0[1])
        graphed.records.copy_(tail0[2])
        for o in outs:
            o.fill_(float("nan"))
        _ = (torch.randn(1024, 1024, device="cuda") @ torch.randn(1024, 1024, device="cuda")).sum().item()
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            gr.replay()
        torch.cuda.synchronize()
        for s in range(steps):
            assert torch.equal(outs[s], ref[s]), f"replay {rep}, step {s}"
        for a, b in zip(_state(graphed), _state(eager)):
            assert torch.equal(a, b), f"replay {rep}: cache state"


def test_decode_step_wrong_host_length_leaves_request_unchanged():
    """Host lengths that claim no group completes when, by the cache's own
    length, request 0's token does: request 0 is left as it was (no token
    written, length unchanged) instead of having the token written into a
    sink row; request 1 appends as usual."""
    cfg = K.make_config(128, 4, 2, 2, 2)
    c, _ = _pair(cfg, 2, 2, [255, 100], 31)
    before = [t.clone() for t in _state(c)]
    g = torch.Generator(device="cuda").manual_seed(2)
    kn = torch.randn((2, 2, 128), generator=g, device="cuda").half()
    vn = torch.randn((2, 2, 128), generator=g, device="cuda").half()
    q = torch.randn((2, 4, 128), generator=g, device="cuda").half()
    c.decode_step(kn, vn, q, lengths=[254, 100])   # wrong for request 0 (its cache holds 255)
    torch.cuda.synchronize()
    assert c.seq_len.cpu().tolist() == [255, 101]
    for name, t0 in zip(("sink_k", "sink_v", "tail_k", "tail_v"), before[:4]):
        t = getattr(c, name)
        assert torch.equal(t[0], t0[0]), name
    assert torch.equal(c.sink_k[1, :, 100], kn[1]) and torch.equal(c.sink_v[1, :, 100], vn[1])
    assert torch.equal(c.records, before[4])
