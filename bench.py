#!/usr/bin/env python3
"""Benchmark of the KVarN hot path on one MI355X.

Workload (default): the Llama-3.1-8B attention shape -- 32 query / 8 KV
heads, head dim 128, batch 1, 32768 cached tokens (128-token fp16 sink + 255
sealed 2-bit groups), 2-bit K and V.  One *step* is one pass of the whole hot
path over one layer's cache: append the new token's K/V, seal the group if its
128th token just arrived, then decode attention for the 32 query heads.

Caches of `--copies` layers (distinct memory, 20 MB each) are visited in
turn, as a model's layers would be, so every step reads its records from HBM
rather than from the 256 MB Infinity Cache.  Layer caches advance in
lockstep: step s appends token s // copies to layer s % copies, so each layer
sees 256 appended tokens (two seals) in the default run.

The timed region is a HIP graph of exactly K steps replayed on one stream,
bracketed by a device synchronization and HIP events.  Everything the steps
read is resident in HBM before the timer starts.

Printed (one JSON line): decode tokens/s per layer (value), the roofline of
the dominant kernel (the split-K decode kernel, timed live with HIP events
around a graph of back-to-back launches), bulk-seal groups/s, and the CPU
oracle timed on this host on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
VALU_FP32_PEAK = 157.3e12  # flop/s, fp32 vector (packed) MI355X


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=8192)
    ap.add_argument("--warmup", type=int, default=256)
    ap.add_argument("--copies", type=int, default=32)
    ap.add_argument("--workload", default="llama31_8b_32k")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seal-groups", type=int, default=48)
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="if > 0: run this many eager steps only (for rocprofv3) and exit")
    return ap.parse_args()


def algorithmic_decode_bytes(wl, lens, k_rec, v_rec):
    """Bytes one decode launch must move: records + exact fp16 rows + q + out."""
    total = 0
    for n in lens:
        g = max(0, (n - 128) // 128)
        exact = min(n, 128) + (n - 128 - 128 * g if n > 128 else 0)
        total += wl.num_kv_heads * (g * (k_rec + v_rec) + exact * wl.head_dim * 2 * 2)
    total += wl.batch * wl.num_q_heads * wl.head_dim * (2 + 4)
    return total


def cpu_baseline(wl, k_stream0, v_stream0, q0, n_seal_groups):
    """The oracle, as it stands, on a bounded sample of the same workload.

    Seal: ``n_seal_groups`` groups (K and V tiles) of KV head 0.  Decode: one
    step (all query heads of KV head 0 over its 32k cache, the oracle state
    built beforehand), scaled to the full step by the number of KV heads.
    """
    from oracle import kvarn_oracle as O
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([d.get("num_threads", 1) for d in info] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    n0 = wl.start_len(0)
    t0 = time.perf_counter()
    for g in range(n_seal_groups):
        lo = 128 + 128 * g
        O.encode_record(**_enc(O.seal_tile(k_stream0[lo:lo + 128], wl.k_bits), wl.k_bits, "k"))
        O.encode_record(**_enc(O.seal_tile(v_stream0[lo:lo + 128], wl.v_bits), wl.v_bits, "v"))
    t_seal = time.perf_counter() - t0
    st = O.state_from_stream(k_stream0[:n0], v_stream0[:n0], wl.k_bits, wl.v_bits)
    g = wl.num_q_heads // wl.num_kv_heads
    t1 = time.perf_counter()
    for h in range(g):
        st.attend(q0[h])
    t_dec = time.perf_counter() - t1
    step_s = t_dec * wl.num_kv_heads
    return {
        "value": wl.batch / step_s, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
        "seal_groups_per_s": n_seal_groups / t_seal,
        "sample": (f"decode: query heads 0..{g - 1} (KV head 0) over {n0} tokens, one step, x{wl.num_kv_heads} "
                   f"KV heads; seal: {n_seal_groups} groups (K+V tiles) of KV head 0; float64 NumPy"),
        "seconds": round(t_seal + t_dec, 2),
    }


def _enc(out, bits, kind):
    return dict(codes=out["codes"], s16=out["s16"], c16=out["c16"], bits=bits, kind=kind)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the KVarN hot path here is built and measured on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    import torch
    from kv_cache_quantization_seal_amd import kvarn as K
    from kv_cache_quantization_seal_amd import synth

    wl = synth.WORKLOADS[args.workload]
    B, hq, hkv, d = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    ncopy = args.copies
    tokens = -(-max(args.steps, args.warmup) // ncopy)  # tokens appended per layer cache
    tokens = max(tokens, 1)
    lens0 = [wl.start_len(b) for b in range(B)]
    lmax = max(lens0) + tokens
    max_groups = (lmax - 128) // 128 + 1
    torch.cuda.init()
    dev = torch.device("cuda:0")
    print(f"[bench] workload {wl.name}: B={B} Hq={hq} Hkv={hkv} D={d} ctx={lens0[0]} "
          f"k{wl.k_bits}/v{wl.v_bits}, copies={ncopy}, steps={args.steps}", file=sys.stderr, flush=True)

    # ---- inputs (seeded, synthetic), generated on the host then uploaded ----
    t0 = time.time()
    kh = np.empty((B, hkv, lmax, d), np.float16)
    vh = np.empty((B, hkv, lmax, d), np.float16)
    for b in range(B):
        for h in range(hkv):
            kk, vv = synth.kv_stream(wl, b, h, lmax)
            kh[b, h], vh[b, h] = kk, vv
    qh = np.stack([synth.queries(wl, b, tokens) for b in range(B)], axis=1)  # [T][B][Hq][D]
    print(f"[bench] inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    k_all = torch.from_numpy(kh).to(dev)
    v_all = torch.from_numpy(vh).to(dev)
    new_k = torch.stack([k_all[b, :, lens0[b]:lens0[b] + tokens] for b in range(B)])  # [B][Hkv][T][D]
    new_v = torch.stack([v_all[b, :, lens0[b]:lens0[b] + tokens] for b in range(B)])
    new_k = new_k.permute(2, 0, 1, 3).contiguous()  # [T][B][Hkv][D]
    new_v = new_v.permute(2, 0, 1, 3).contiguous()
    q_all = torch.from_numpy(qh).to(dev).contiguous()
    cfg = K.make_config(d, hq, hkv, wl.k_bits, wl.v_bits)

    # ---- bulk seal (prefill) of layer 0, timed -----------------------------
    cache0 = K.KVarNCache(cfg, B, max_groups, device=dev)
    cache0.prefill(k_all, v_all, lens0)
    torch.cuda.synchronize()
    n_groups_seal = sum(hkv * ((n - 128) // 128) for n in lens0 if n > 128)
    seal_reps = 5
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(seal_reps):
        cache0.prefill(k_all, v_all, lens0)
    e1.record()
    torch.cuda.synchronize()
    t_prefill = e0.elapsed_time(e1) / 1e3 / seal_reps
    k_rec, v_rec = K.record_bytes(d, wl.k_bits), K.record_bytes(d, wl.v_bits)
    seal_bytes_per_group = 2 * 128 * d * 2 + k_rec + v_rec   # fp16 K+V tiles in, two records out
    sinkhorn_flops_per_group = 2 * 16 * 2 * 128 * d * 2        # 2 tiles x 16 iters x 2 mat-vecs x T*D FMAs
    seal = {
        "groups_per_s": n_groups_seal / t_prefill,
        "groups_per_call": n_groups_seal,
        "ms_per_call": t_prefill * 1e3,
        "hbm_GBps": n_groups_seal * seal_bytes_per_group / t_prefill / 1e9,
        "hbm_frac": n_groups_seal * seal_bytes_per_group / t_prefill / HBM_PEAK,
        "sinkhorn_valu_frac": n_groups_seal * sinkhorn_flops_per_group / t_prefill / VALU_FP32_PEAK,
        "note": "bulk ingest via kvarn_prefill (sink/tail copy + seal kernel), K and V tiles",
    }
    print(f"[bench] seal: {seal['groups_per_s'] / 1e6:.2f} M groups/s ({seal['hbm_frac'] * 100:.1f}% of HBM)",
          file=sys.stderr, flush=True)

    # ---- layer caches ----------------------------------------------------
    caches = [cache0]
    for c in range(1, ncopy):
        cc = K.KVarNCache(cfg, B, max_groups, device=dev)
        for name in ("sink_k", "sink_v", "tail_k", "tail_v", "records", "seq_len"):
            getattr(cc, name).copy_(getattr(cache0, name))
        caches.append(cc)
    seq0 = cache0.seq_len.clone()
    outs = [torch.empty(B, hq, d, dtype=torch.float32, device=dev) for _ in range(ncopy)]
    torch.cuda.synchronize()

    def reset():
        for c in caches:
            c.seq_len.copy_(seq0)

    def step(s):
        c = caches[s % ncopy]
        tok = s // ncopy
        c.append(new_k[tok], new_v[tok])
        c.seal_group()
        c.decode_attn(q_all[tok], out=outs[s % ncopy])

    if args.profile_steps > 0:
        for s in range(args.profile_steps):
            step(s)
        torch.cuda.synchronize()
        print(f"[bench] profile run: {args.profile_steps} eager steps done", file=sys.stderr, flush=True)
        return

    # ---- graphs ------------------------------------------------------------
    stream = torch.cuda.Stream()
    def capture(nsteps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for s in range(nsteps):
                step(s)
        return g

    reset()
    torch.cuda.synchronize()
    g_warm = capture(args.warmup) if args.warmup > 0 else None
    g_main = capture(args.steps)
    torch.cuda.synchronize()
    if g_warm is not None:
        reset()
        torch.cuda.synchronize()
        g_warm.replay()
        torch.cuda.synchronize()
    reset()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        g_main.replay()
        ev1.record(stream)
    torch.cuda.synchronize()
    t_total = ev0.elapsed_time(ev1) / 1e3
    steps_per_s = args.steps / t_total
    value = B * steps_per_s

    # ---- live timing of the dominant kernel (the fused decode kernel) -----
    reset()
    torch.cuda.synchronize()
    reps = 8 * ncopy
    gk = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gk, stream=stream):
        for r in range(reps):
            caches[r % ncopy].decode_attn(q_all[0], out=outs[r % ncopy])
    torch.cuda.synchronize()
    gk.replay()  # warm
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        ev0.record(stream)
        gk.replay()
        ev1.record(stream)
    torch.cuda.synchronize()
    t_kernel = ev0.elapsed_time(ev1) / 1e3 / reps
    bytes_launch = algorithmic_decode_bytes(wl, lens0, k_rec, v_rec)
    achieved = bytes_launch / t_kernel
    print(f"[bench] decode kernel: {t_kernel * 1e6:.2f} us/launch, {achieved / 1e12:.2f} TB/s "
          f"({achieved / HBM_PEAK * 100:.1f}% of HBM); step {t_total / args.steps * 1e6:.2f} us",
          file=sys.stderr, flush=True)

    line = {
        "metric": "quantized decode-attn tokens/s + % HBM peak; seal_group groups/s (1 MI355X)",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_total / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8-mfma+f32",
        "data": "synthetic (seeded K/V/q with outlier channels and lognormal token norms)",
        "config": {"workload": wl.name, "batch": B, "q_heads": hq, "kv_heads": hkv, "head_dim": d,
                   "context": lens0[0], "k_bits": wl.k_bits, "v_bits": wl.v_bits, "layer_caches": ncopy,
                   "step": "append + seal-if-due + decode attention (one layer)"},
        "roofline": {"bound": "hbm", "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK, "traffic": None,
                     "kernel": "decode_split_kernel", "bytes_per_launch": bytes_launch,
                     "us_per_launch": t_kernel * 1e6},
        "seal": seal,
    }
    if not args.no_cpu:
        print("[bench] timing the CPU oracle on a bounded sample...", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl, kh[0, 0], vh[0, 0], qh[0, 0], args.cpu_seal_groups)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line))


if __name__ == "__main__":
    main()
