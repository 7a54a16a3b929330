#!/usr/bin/env python3
"""Benchmark of the KVarN hot path on one MI355X.

Workload (default): the Llama-3.1-8B attention shape -- 32 query / 8 KV
heads, head dim 128, batch 1, 32768 cached tokens (128-token fp16 sink + 255
sealed 2-bit groups), 2-bit K and V.  One *step* is one pass of the whole hot
path over one layer's cache: append the new token's K/V and seal the group if
its 128th token just arrived (one launch, kvarn_append_seal), then decode
attention for the 32 query heads (split kernel + combine kernel).

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
MFMA_F16_PEAK = 2.5e15     # flop/s, dense fp16 MFMA, MI355X
# fp32 vector peak without packed instructions (the library is compiled with them off):
# 256 CUs x 4 SIMDs x 16 lanes x 2 flop per FMA x 2.4 GHz.  The 157.3 TFLOP/s
# vendor figure counts packed FMAs, which no kernel here issues.
VALU_FP32_PEAK = 78.6e12


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=8192,
                    help="decode steps timed (at most copies x 256 fit the workload's capacity)")
    ap.add_argument("--warmup", type=int, default=256)
    ap.add_argument("--copies", type=int, default=32)
    ap.add_argument("--workload", default="llama31_8b_32k")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seal-groups", type=int, default=48)
    ap.add_argument("--prefill-chunk", type=int, default=2048,
                    help="query tokens of the chunked-prefill attention measurement (the last chunk of the prompt)")
    ap.add_argument("--other-workloads", default="qwen3_4b_16k_b16,qwen3_4b_16k_b16_aligned,phi4_14b_32k_b8,longctx_d256_64k_b4,"
                    "llama31_8b_32k_k3v2,llama31_8b_32k_k6v5",
                    help="comma-separated workloads measured after the headline one and reported under "
                         "'workloads' (empty: none)")
    ap.add_argument("--other-steps", type=int, default=256, help="decode steps timed per other workload")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="if > 0: run this many eager steps only (for rocprofv3) and exit")
    ap.add_argument("--profile-seal", type=int, default=0, metavar="N",
                    help="if > 0: run N bulk seals (kvarn_prefill of the workload's prompt, K and V) only "
                         "(for rocprofv3) and exit")
    ap.add_argument("--profile-prefill", type=int, default=0, metavar="N",
                    help="if > 0: build the workload's cache, then run N chunked-prefill attention calls "
                         "(--prefill-chunk query tokens) only (for rocprofv3) and exit")
    ap.add_argument("--counter-summary", nargs="+", metavar="DIR",
                    help="print, per kernel whose name contains --kernel, the median over dispatches of every "
                         "counter found in the rocprofv3 --pmc output directories DIR..., and exit")
    ap.add_argument("--kernel", default="seal_prefill_kernel", help="kernel name filter for --counter-summary")
    ap.add_argument("--trace-max-groups", type=int, default=0,
                    help="with --trace: cache capacity in groups (default: the workload's own)")
    ap.add_argument("--trace", choices=["decode", "seal", "prefill"],
                    help="load the trace build (libkvarn_trace.so), run the decode split kernel, the bulk seal or "
                         "the chunked-prefill attention of the workload cold a few times, print per-wave phase "
                         "timestamps (prefill: cycles per phase summed over the tiles) as JSON, and exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 8 device-to-device copies of MIB MiB (a plain copy kernel of known "
                         "size, the reference for the HBM counters) and exit")
    ap.add_argument("--traffic-summary", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_DIRS"),
                    help="summarize rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of --profile-steps and of "
                         "--copy-calibration (COPY_DIRS = 'fetch_dir,write_dir') into profiles/ and exit")
    return ap.parse_args()


def algorithmic_decode_bytes(wl, lens, k_rec, v_rec):
    """Bytes the split kernel must move per launch: every sealed record once,
    the exact fp16 sink and tail rows (K and V), and the query."""
    total = 0
    for n in lens:
        g = max(0, (n - 128) // 128)
        exact = min(n, 128) + (n - 128 - 128 * g if n > 128 else 0)
        total += wl.num_kv_heads * (g * (k_rec + v_rec) + exact * wl.head_dim * 2 * 2)
    total += wl.batch * wl.num_q_heads * wl.head_dim * 2
    return total


def decode_source_sha():
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for f in ("decode.hip", "decode_impl.hpp", "decode_k2.hip", "decode_k3.hip", "decode_k4.hip", "decode_k5.hip",
              "decode_k6.hip", "decode_k8.hip", "common.hpp", "kernels.hpp"):
        with open(os.path.join(here, "kv_cache_quantization_seal_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_file(workload):
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        f"decode_split_kernel_{workload}_hbm_traffic.txt")


def read_traffic(workload):
    """Measured HBM bytes per split-kernel launch, if the counters were taken
    on the current kernel source; else None."""
    try:
        kv = {}
        with open(traffic_file(workload)) as fh:
            for line in fh:
                if "=" in line and not line.startswith("#"):
                    k, v = line.split("=", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("decode_source_sha") != decode_source_sha():
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def _pmc_rows(d, counter, kernel_substr):
    import csv
    import glob
    vals = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") == counter and kernel_substr in r.get("Kernel_Name", ""):
                    vals.append(float(r["Counter_Value"]))
    return vals


def traffic_summary(args):
    """Scale the decode kernel's FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by
    what the same counters read for a plain copy of known size."""
    fetch_dir, write_dir, copy_dirs = args.traffic_summary
    cfetch_dir, cwrite_dir = copy_dirs.split(",")
    from kv_cache_quantization_seal_amd import synth, kvarn as K
    wl = synth.WORKLOADS[args.workload]
    copy_bytes = args.copy_calibration * 2**20
    if copy_bytes <= 0:
        sys.exit("--traffic-summary needs --copy-calibration MIB (the size the copy runs used)")
    cf = _pmc_rows(cfetch_dir, "FETCH_SIZE", "copy")
    cw = _pmc_rows(cwrite_dir, "WRITE_SIZE", "copy")
    df = _pmc_rows(fetch_dir, "FETCH_SIZE", "decode_split_kernel")
    dw = _pmc_rows(write_dir, "WRITE_SIZE", "decode_split_kernel")
    if not (cf and cw and df and dw):
        sys.exit("missing counter rows (copy fetch/write, decode fetch/write): "
                 f"{len(cf)} {len(cw)} {len(df)} {len(dw)}")
    # Per copy dispatch the kernel reads and writes copy_bytes.
    f_scale = copy_bytes / (np.median(cf) * 1024)
    w_scale = copy_bytes / (np.median(cw) * 1024)
    fetch = np.median(df) * 1024 * f_scale
    write = np.median(dw) * 1024 * w_scale
    lens = [wl.start_len(b) for b in range(wl.batch)]
    alg = algorithmic_decode_bytes(wl, lens, K.record_bytes(wl.head_dim, wl.k_bits),
                                   K.record_bytes(wl.head_dim, wl.v_bits))
    with open(traffic_file(wl.name), "w") as fh:
        fh.write(f"# HBM traffic of decode_split_kernel, workload {wl.name}, from rocprofv3 --pmc\n")
        fh.write("# FETCH_SIZE and WRITE_SIZE (KiB per dispatch, median over dispatches), each scaled by\n")
        fh.write(f"# bytes / counter of a plain {args.copy_calibration} MiB device copy run the same way.\n")
        fh.write(f"decode_source_sha = {decode_source_sha()}\n")
        fh.write(f"copy_bytes = {copy_bytes}\n")
        fh.write(f"copy_fetch_kib = {np.median(cf):.1f}\ncopy_write_kib = {np.median(cw):.1f}\n")
        fh.write(f"fetch_scale = {f_scale:.4f}\nwrite_scale = {w_scale:.4f}\n")
        fh.write(f"decode_fetch_kib = {np.median(df):.1f}  (dispatches {len(df)})\n")
        fh.write(f"decode_write_kib = {np.median(dw):.1f}  (dispatches {len(dw)})\n")
        fh.write(f"fetch_bytes_per_launch = {fetch:.0f}\nwrite_bytes_per_launch = {write:.0f}\n")
        fh.write(f"traffic_bytes_per_launch = {fetch + write:.0f}\n")
        fh.write(f"algorithmic_bytes_per_launch = {alg}\n")
        fh.write(f"traffic_over_algorithmic = {(fetch + write) / alg:.3f}\n")
    print(open(traffic_file(wl.name)).read())


def counter_summary(args):
    """Median per dispatch of every PMC counter in the given rocprofv3 output
    directories, for the dispatches of kernels matching --kernel; prints
    'counter = value' lines (the figures the profile summaries quote)."""
    import csv
    import glob
    vals = {}
    names = set()
    for d in args.counter_summary:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if args.kernel in r.get("Kernel_Name", ""):
                        names.add(r["Kernel_Name"].split("(")[0])
                        vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not vals:
        sys.exit(f"no counter rows for kernels matching {args.kernel!r} in {args.counter_summary}")
    print(f"# kernels: {', '.join(sorted(names))}")
    for k in sorted(vals):
        v = np.asarray(vals[k])
        print(f"{k} = {np.median(v):.6g}  (dispatches {v.size}, min {v.min():.6g}, max {v.max():.6g})")


def trace_run(args, reps=8):
    """Per-wave phase timestamps from the trace build: each repetition
    flushes the Infinity Cache, clears the trace buffer, launches the kernel
    once on a layer cache not used before and reads the marks back."""
    import torch
    from kv_cache_quantization_seal_amd import kvarn as K
    from kv_cache_quantization_seal_amd import probe, synth, wavetrace
    wl = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    B, hq, hkv, d = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    lens = [wl.start_len(b) for b in range(B)]
    kd, vd = synth.kv_streams_device(wl, max(lens), dev)
    cfg = K.make_config(d, hq, hkv, wl.k_bits, wl.v_bits)
    mg = args.trace_max_groups or wl.max_groups()
    flush_buf = torch.zeros(2**30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    caches = [K.KVarNCache(cfg, B, mg, device=dev) for _ in range(reps)]
    for c in caches:
        c.prefill(kd, vd, lens)
    q = torch.from_numpy(np.stack([synth.queries(wl, b, 1)[0] for b in range(B)])).to(dev)
    plan = K.decode_plan(cfg, B, mg)
    torch.cuda.synchronize()
    summaries = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if args.trace == "prefill":
        print(json.dumps(prefill_trace(args, wl, caches, e0, e1, flush_buf, sink)))
        return
    for r in range(reps):
        probe.read(flush_buf, sink)
        torch.cuda.synchronize()
        which = wavetrace.decode(wl.k_bits) if args.trace == "decode" else wavetrace.SEAL
        wavetrace.clear(which)
        e0.record()
        if args.trace == "decode":
            caches[r].decode_partial(q)
        else:
            caches[r].prefill(kd, vd, lens)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3
        if args.trace == "decode":
            n_ex, n_rec = plan["exact_workgroups"], plan["record_workgroups"]
            rec = wavetrace.read(which, 4 * (n_ex + n_rec))
            names = {0: "start", 1: "query", 2: "first_ck", 3: "first_qk", 4: "first_pv", 5: "groups_done",
                     6: "partial_written"}
            # the split kernel's grid order, as the plan chooses it: record
            # workgroups first when each pair has four exact splits (few
            # pairs) and the record workgroups are one per CU at most
            cus = torch.cuda.get_device_properties(0).multi_processor_count
            if plan["exact_splits"] == 4 and n_rec <= cus:
                groups = {"record": range(0, 4 * n_rec), "exact": range(4 * n_rec, 4 * (n_ex + n_rec))}
            else:
                groups = {"exact": range(0, 4 * n_ex), "record": range(4 * n_ex, 4 * (n_ex + n_rec))}
        else:
            n_tiles = 2 * B * hkv * max(0, (max(lens) - 128) // 128)
            rec = wavetrace.read(which, n_tiles * d // 16)
            names = {0: "start", 1: "rotated", 2: "iterated", 3: "stored"}
            groups = None
        summ = wavetrace.summarize(rec, names, groups)
        summ["event_us"] = us
        summaries.append(summ)
    print(json.dumps({"workload": wl.name, "trace": args.trace, "plan": plan, "reps": summaries}))


# Phases of the chunked-prefill trace build (per tile).  In eight-wave
# workgroups waves 0-3 stage only K halves and waves 4-7 only V halves, so
# the two kinds are summarized apart.
PREFILL_PHASES = ["issue_next_record", "query_operand", "qk_mfma", "softmax_and_pv_operands", "barrier_a",
                  "stage_k", "pv_mfma", "barrier_b", "stage_v"]


def prefill_trace(args, wl, caches, e0, e1, flush_buf, sink):
    """Trace build, chunked-prefill attention: core-clock cycles per phase of
    every wave, summed over its tiles; median over waves, per tile."""
    import torch
    from kv_cache_quantization_seal_amd import probe, wavetrace
    dev = caches[0].sink_k.device
    chunk = args.prefill_chunk
    q = torch.from_numpy(np.random.default_rng(7).standard_normal(
        (wl.batch, chunk, wl.num_q_heads, wl.head_dim)).astype(np.float16)).to(dev)
    gq = wl.num_q_heads // wl.num_kv_heads
    # Workgroups of 8 waves (128 query rows) at D 128 when that grid has one
    # per CU, else of 4 waves (64 rows): the launch's own rule.
    wgs8 = -(-chunk * gq // 128) * wl.num_kv_heads * wl.batch
    eight = wl.head_dim == 128 and wgs8 >= torch.cuda.get_device_properties(0).multi_processor_count
    n_waves = wgs8 * 8 if eight else -(-chunk * gq // 64) * wl.num_kv_heads * wl.batch * 4
    reps = []
    for c in caches[:3]:
        probe.read(flush_buf, sink)
        torch.cuda.synchronize()
        wavetrace.clear(wavetrace.PREFILL_ATTN)
        e0.record()
        c.prefill_attn(q)
        e1.record()
        torch.cuda.synchronize()
        rec = wavetrace.read(wavetrace.PREFILL_ATTN, n_waves).astype(np.int64)
        ran = rec[:, 15] > rec[:, 1]
        tiles = 1 + (wl.context - 128) // 128 + 1
        life = (rec[ran][:, 15] - rec[ran][:, 1]).astype(np.float64)
        # the slot of a wave is its workgroup's index times the waves per workgroup plus the wave
        wave = np.arange(n_waves) % (8 if eight else 4)
        kinds = ({"k_staging_waves": wave < 4, "v_staging_waves": wave >= 4} if eight else {"all_waves": wave >= 0})
        phases = {}
        for kind, sel in kinds.items():
            cyc = rec[ran & sel][:, 2:2 + len(PREFILL_PHASES)].astype(np.float64)
            phases[kind] = {n: float(np.median(cyc[:, i]) / tiles) for i, n in enumerate(PREFILL_PHASES)}
        reps.append({"event_us": e0.elapsed_time(e1) * 1e3, "waves": int(ran.sum()), "tiles_per_wave": tiles,
                     "waves_per_workgroup": 8 if eight else 4,
                     "wave_cycles_per_tile": float(np.median(life) / tiles),
                     "phase_cycles_per_tile": phases})
    return {"workload": wl.name, "trace": "prefill", "chunk": chunk, "reps": reps}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_threads():
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        return max([d.get("num_threads", 1) for d in info] or [1])
    except Exception:  # pragma: no cover
        return 1


def _oracle_unit(task):
    """One independent unit of the oracle: part `part` of `parts` of a
    (request, KV head): seal groups [g0, g0 + n_seal) of its stream, then
    (state built untimed) one decode step of its share of the query heads.
    Returns (seal seconds, decode seconds)."""
    name, b, h, n_seal, part, parts = task
    from kv_cache_quantization_seal_amd import synth
    from oracle import kvarn_oracle as O
    wl = synth.WORKLOADS[name]
    n0 = wl.start_len(b)
    k, v = synth.kv_stream(wl, b, h, n0)
    q = synth.queries(wl, b, 1)[0]
    t0 = time.perf_counter()
    for g in range(part * n_seal, (part + 1) * n_seal):
        lo = 128 + 128 * g
        O.encode_record(**_enc(O.seal_tile(k[lo:lo + 128], wl.k_bits), wl.k_bits, "k"))
        O.encode_record(**_enc(O.seal_tile(v[lo:lo + 128], wl.v_bits), wl.v_bits, "v"))
    t_seal = time.perf_counter() - t0
    st = O.state_from_stream(k, v, wl.k_bits, wl.v_bits)
    gq = wl.num_q_heads // wl.num_kv_heads
    t1 = time.perf_counter()
    for hh in range(gq * part // parts, gq * (part + 1) // parts):
        st.attend(q[h * gq + hh])
    return t_seal, time.perf_counter() - t1


def cpu_baseline(wl, n_seal_groups):
    """The oracle, as it stands, on a bounded sample of the same workload, in
    two modes.  Units are the KV heads of request 0 (independent: each seals
    its own groups and attends its own query heads).

    * One process (NumPy with its BLAS threads): unit 0 alone, its decode step
      scaled by the number of KV heads, ``n_seal_groups`` seal groups.
    * A pool of P worker processes with one BLAS thread each, P = the CPU
      affinity (at most 16, the host share of one GPU): each KV head is split
      into S = P // KV heads parts (at most its query heads), a part sealing
      its share of the groups and attending its share of the query heads;
      every unit at once.  The decode step takes the slowest unit's time;
      seal throughput is all units' groups over the slowest unit's seal time.

    Runs before the GPU is initialized (the pool's workers are spawned).
    """
    import multiprocessing as mp
    t_start = time.perf_counter()
    blas = _blas_threads()
    t_seal1, t_dec1 = _oracle_unit((wl.name, 0, 0, n_seal_groups, 0, 1))
    single = {"value": wl.batch / (t_dec1 * wl.num_kv_heads), "seal_groups_per_s": n_seal_groups / t_seal1,
              "threads": int(blas)}
    gq = wl.num_q_heads // wl.num_kv_heads
    aff = max(1, min(16, len(os.sched_getaffinity(0))))
    parts = max(1, min(gq, aff // wl.num_kv_heads))
    units = wl.num_kv_heads * parts
    P = max(1, min(aff, units))
    per_unit = max(1, n_seal_groups // units)
    env = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in env:
        os.environ[k] = "1"
    try:
        with mp.get_context("spawn").Pool(P) as pool:
            res = pool.map(_oracle_unit, [(wl.name, 0, h, per_unit, p, parts)
                                          for h in range(wl.num_kv_heads) for p in range(parts)])
    finally:
        for k, val in env.items():
            if val is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = val
    t_seal_p = max(r[0] for r in res)
    t_dec_p = max(r[1] for r in res)
    n0 = wl.start_len(0)
    return {
        "value": wl.batch / t_dec_p, "unit": "tokens/s", "cores": int(P), "kind": "oracle",
        "seal_groups_per_s": units * per_unit / t_seal_p,
        "sample": (f"one decode step of request 0 over {n0} tokens ({wl.num_kv_heads} KV heads x {gq} query "
                   f"heads) and {units * per_unit} seal groups (K+V tiles), as {units} units ({parts} per KV "
                   f"head) on {P} worker processes with one BLAS thread each; float64 NumPy oracle"),
        "single_process": dict(single, sample=(f"KV head 0 only ({gq} query heads, step scaled x{units}), "
                                               f"{n_seal_groups} seal groups")),
        "cpu_model": _cpu_model(),
        "seconds": round(time.perf_counter() - t_start, 2),
    }


def _enc(out, bits, kind):
    return dict(codes=out["codes"], s16=out["s16"], c16=out["c16"], bits=bits, kind=kind)


def measure_workload(torch, K, probe, synth, dev, name, steps, hbm_target_bytes=768 * 2**20):
    """Decode step and bulk seal of one more workload, measured like the
    headline one: K/V drawn on the device with the synthetic recipe, enough
    layer caches (at least 2) to exceed `hbm_target_bytes` so steps read HBM
    rather than the Infinity Cache, a HIP graph of `steps` steps rotating over
    them, then HIP-event timing of the split kernel alone (median of 50
    replays).  A step is append + seal-if-due + decode attention for workloads
    that decode (at most their own number of steps per cache, so the cache
    capacity is the workload's own and the decode plan is the one the
    full-size parity test checks), and decode attention alone for the
    steady-state workload."""
    wl = synth.WORKLOADS[name]
    B, hq, hkv, d = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    lens0 = [wl.start_len(b) for b in range(B)]
    k_rec, v_rec = K.record_bytes(d, wl.k_bits), K.record_bytes(d, wl.v_bits)
    bytes_launch = algorithmic_decode_bytes(wl, lens0, k_rec, v_rec)
    ncopy = max(2, -(-hbm_target_bytes // bytes_launch))
    decoding = wl.steps > 0
    tokens = min(wl.steps, max(1, -(-steps // ncopy))) if decoding else 1
    max_groups = wl.max_groups()
    lmax = max(lens0) + tokens
    kd, vd = synth.kv_streams_device(wl, lmax, dev)
    idx = torch.tensor([[n + t for n in lens0] for t in range(tokens)], device=dev)   # [T][B]
    ar = torch.arange(B, device=dev)
    new_k = torch.stack([kd[ar, :, idx[t]] for t in range(tokens)]).contiguous()      # [T][B][Hkv][D]
    new_v = torch.stack([vd[ar, :, idx[t]] for t in range(tokens)]).contiguous()
    q_all = torch.from_numpy(np.stack([synth.queries(wl, b, tokens) for b in range(B)], axis=1)).to(dev)
    cfg = K.make_config(d, hq, hkv, wl.k_bits, wl.v_bits)
    plan = K.decode_plan(cfg, B, max_groups)
    caches = [K.KVarNCache(cfg, B, max_groups, device=dev) for _ in range(ncopy)]
    for c in caches:
        c.prefill(kd, vd, lens0)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    # bulk seal, timed on cache 0 (median of 50 graph replays)
    n_groups_seal = sum(hkv * ((n - 128) // 128) for n in lens0 if n > 128)
    g_seal = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_seal, stream=stream):
        caches[0].prefill(kd, vd, lens0, stream=stream)
    t_prefill = float(np.median(_timed_replays(torch, stream, g_seal, 50)))
    del g_seal, kd, vd
    seq0 = caches[0].seq_len.clone()
    outs = [torch.empty(B, hq, d, dtype=torch.float32, device=dev) for _ in range(ncopy)]
    flush_buf = torch.zeros(2**30, dtype=torch.uint8, device=dev)
    flush_sink = torch.zeros(4, dtype=torch.int32, device=dev)

    def reset():
        for c in caches:
            c.seq_len.copy_(seq0)

    def timed_graph(fn, n, reps):
        reset()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for r in range(n):
                fn(r)
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ts = _timed_replays(torch, stream, g, reps, before=lambda: (reset(), probe.read(flush_buf, flush_sink)),
                            per=n)
        del g
        return _stats(ts)

    def step(s):
        c = caches[s % ncopy]
        t = s // ncopy
        if decoding:
            c.decode_step(new_k[t], new_v[t], q_all[t], lengths=[n + t for n in lens0], out=outs[s % ncopy])
        else:
            c.decode_attn(q_all[t], out=outs[s % ncopy])

    st_step = timed_graph(step, tokens * ncopy, 20)
    st_split = timed_graph(lambda r: caches[r % ncopy].decode_partial(q_all[0]), 8 * ncopy, 50)
    t_step, t_split = st_step["median"], st_split["median"]
    achieved = bytes_launch / t_split
    seal_bytes_per_group = 2 * 128 * d * 2 + k_rec + v_rec
    us = lambda st: {k: (v * 1e6 if k != "reps" else v) for k, v in st.items()}
    out = {
        "tokens_per_s": B / t_step, "ms_per_step": t_step * 1e3, "step_us_stats": us(st_step),
        "config": {"batch": B, "q_heads": hq, "kv_heads": hkv, "head_dim": d, "context": lens0[0],
                   "context_stagger": wl.stagger, "k_bits": wl.k_bits, "v_bits": wl.v_bits,
                   "layer_caches": ncopy, "steps": tokens * ncopy, "max_groups": max_groups,
                   "step": ("append + seal-if-due + decode attention" if decoding else "decode attention")},
        "decode_plan": plan,
        "roofline": {"bound": "hbm", "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK, "kernel": "decode_split_kernel",
                     "bytes_per_launch": bytes_launch, "us_per_launch": t_split * 1e6, "us_stats": us(st_split)},
        "seal": {"groups_per_s": n_groups_seal / t_prefill,
                 "hbm_frac": n_groups_seal * seal_bytes_per_group / t_prefill / HBM_PEAK},
    }
    del caches, outs, new_k, new_v, q_all, flush_buf
    torch.cuda.empty_cache()
    return out


def _stats(xs):
    xs = np.asarray(xs, dtype=np.float64)
    return {"median": float(np.median(xs)), "p10": float(np.percentile(xs, 10)),
            "p90": float(np.percentile(xs, 90)), "reps": int(xs.size)}


def _timed_replays(torch, stream, g, reps, before=None, per=1):
    """Replay graph g `reps` times on `stream`, each bracketed by its own HIP
    events (recorded on that stream); `before` runs untimed before every
    replay.  Returns the per-replay times in seconds divided by `per`."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for e0, e1 in evs:
            if before is not None:
                before()   # queued on `stream`, ahead of the replay
            e0.record(stream)
            g.replay()
            e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) / 1e3 / per for e0, e1 in evs]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the KVarN hot path here is built and measured on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    if args.traffic_summary:
        traffic_summary(args)
        return
    if args.counter_summary:
        counter_summary(args)
        return
    if args.trace:
        os.environ["KVARN_LIBRARY"] = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                   "kv_cache_quantization_seal_amd", "libkvarn_trace.so")
        trace_run(args)
        return
    import torch
    from kv_cache_quantization_seal_amd import kvarn as K
    from kv_cache_quantization_seal_amd import probe
    from kv_cache_quantization_seal_amd import synth

    if args.profile_seal > 0:
        # Bulk seal of the workload's prompt only: the seal kernel's
        # dispatches for a profiler, nothing else of note on the GPU.
        wl = synth.WORKLOADS[args.workload]
        lens = [wl.start_len(b) for b in range(wl.batch)]
        kd, vd = synth.kv_streams_device(wl, max(lens), torch.device("cuda:0"))
        cfg = K.make_config(wl.head_dim, wl.num_q_heads, wl.num_kv_heads, wl.k_bits, wl.v_bits)
        cache = K.KVarNCache(cfg, wl.batch, wl.max_groups(), device="cuda:0")
        for _ in range(args.profile_seal):
            cache.prefill(kd, vd, lens)
        torch.cuda.synchronize()
        print(f"[bench] seal profile run: {args.profile_seal} bulk seals of {wl.name}", file=sys.stderr, flush=True)
        return

    if args.profile_prefill > 0:
        # Chunked-prefill attention only (after one bulk seal that builds the
        # cache): its dispatches for a profiler.
        wl = synth.WORKLOADS[args.workload]
        lens = [wl.start_len(b) for b in range(wl.batch)]
        dev = torch.device("cuda:0")
        kd, vd = synth.kv_streams_device(wl, max(lens), dev)
        cfg = K.make_config(wl.head_dim, wl.num_q_heads, wl.num_kv_heads, wl.k_bits, wl.v_bits)
        cache = K.KVarNCache(cfg, wl.batch, wl.max_groups(), device=dev)
        cache.prefill(kd, vd, lens)
        q = torch.from_numpy(np.random.default_rng(7).standard_normal(
            (wl.batch, args.prefill_chunk, wl.num_q_heads, wl.head_dim)).astype(np.float16)).to(dev)
        out = torch.empty(q.shape, dtype=torch.float32, device=dev)
        for _ in range(args.profile_prefill):
            cache.prefill_attn(q, out=out)
        torch.cuda.synchronize()
        print(f"[bench] prefill attention profile run: {args.profile_prefill} calls, {args.prefill_chunk}-token "
              f"chunk of {wl.name}", file=sys.stderr, flush=True)
        return

    if args.copy_calibration > 0:
        n = args.copy_calibration * 2**20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: 8 copies of {n} bytes", file=sys.stderr, flush=True)
        return

    wl = synth.WORKLOADS[args.workload]
    B, hq, hkv, d = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    ncopy = args.copies
    # The cache capacity is the workload's own (every group its decode steps
    # seal), independent of --steps, so every run launches the decode plan
    # that the full-size parity test checks and the profile measures.
    max_groups = wl.max_groups()
    cap = 128 + 128 * max_groups + 127
    lens0 = [wl.start_len(b) for b in range(B)]
    # Layer caches start at spread phases of the group cycle: layer c holds
    # 127 - floor(128 c / copies) more tail tokens than the context, so layer 0
    # seals on its first step.  Layers advance in lockstep (step s appends to
    # layer s % copies), so any window of steps sees the seal cadence of a
    # steady decode (one seal per 128 tokens per layer), and at least one.
    phases = [127 - (128 * c) // ncopy for c in range(ncopy)]
    tokens = max(1, -(-max(args.steps, args.warmup) // ncopy))  # tokens appended per layer cache
    if max(lens0) + max(phases) + tokens > cap:
        sys.exit(f"--steps {args.steps} appends {tokens} tokens per layer cache, more than the "
                 f"{wl.name} capacity ({cap} tokens) leaves room for; use at most "
                 f"{(cap - max(lens0) - max(phases)) * ncopy} steps")
    lmax = max(lens0) + max(phases) + tokens
    # The CPU oracle baseline runs first, before the GPU is initialized (its
    # worker pool is spawned).
    cpu_line = None
    if not args.no_cpu:
        print("[bench] timing the CPU oracle on a bounded sample...", file=sys.stderr, flush=True)
        cpu_line = cpu_baseline(wl, args.cpu_seal_groups)
        print(f"[bench] cpu oracle: {cpu_line['value']:.4f} tokens/s on {cpu_line['cores']} processes, "
              f"{cpu_line['seconds']} s", file=sys.stderr, flush=True)
    torch.cuda.init()
    dev = torch.device("cuda:0")
    print(f"[bench] workload {wl.name}: B={B} Hq={hq} Hkv={hkv} D={d} ctx={lens0[0]} "
          f"k{wl.k_bits}/v{wl.v_bits}, copies={ncopy}, steps={args.steps}, max_groups={max_groups}",
          file=sys.stderr, flush=True)

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
    del kh, vh
    lens_c = [[n + ph for n in lens0] for ph in phases]
    ar = torch.arange(B, device=dev)
    # new_k[c][t]: the token layer c appends at its t-th step, [B][Hkv][D].
    new_k = torch.empty((ncopy, tokens, B, hkv, d), dtype=torch.float16, device=dev)
    new_v = torch.empty_like(new_k)
    for c in range(ncopy):
        for t in range(tokens):
            pos = torch.tensor([n + t for n in lens_c[c]], device=dev)
            new_k[c, t] = k_all[ar, :, pos]
            new_v[c, t] = v_all[ar, :, pos]
    q_all = torch.from_numpy(qh).to(dev).contiguous()
    cfg = K.make_config(d, hq, hkv, wl.k_bits, wl.v_bits)
    plan = K.decode_plan(cfg, B, max_groups)
    flush_buf = torch.zeros(2**30, dtype=torch.uint8, device=dev)
    flush_sink = torch.zeros(4, dtype=torch.int32, device=dev)

    def flush():
        """Stream 1 GiB so that nothing a timed region reads is left in the
        256 MB Infinity Cache by the work before it."""
        probe.read(flush_buf, flush_sink)

    # ---- bulk seal (prefill of the 32k prompt), timed -----------------------
    cache0 = K.KVarNCache(cfg, B, max_groups, device=dev)
    cache0.prefill(k_all, v_all, lens0)
    torch.cuda.synchronize()
    n_groups_seal = sum(hkv * ((n - 128) // 128) for n in lens0 if n > 128)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        g_seal = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_seal, stream=stream):
            cache0.prefill(k_all, v_all, lens0, stream=stream)
    t_seals = _timed_replays(torch, stream, g_seal, 50)
    del g_seal
    t_prefill = float(np.median(t_seals))
    k_rec, v_rec = K.record_bytes(d, wl.k_bits), K.record_bytes(d, wl.v_bits)
    seal_bytes_per_group = 2 * 128 * d * 2 + k_rec + v_rec   # fp16 K+V tiles in, two records out
    sinkhorn_flops_per_group = 2 * 16 * 2 * 128 * d * 2        # 2 tiles x 16 iters x 2 mat-vecs x T*D FMAs
    seal = {
        "groups_per_s": n_groups_seal / t_prefill,
        "groups_per_call": n_groups_seal,
        "ms_per_call": t_prefill * 1e3,
        "us_per_call_stats": {k: (v * 1e6 if k != "reps" else v) for k, v in _stats(t_seals).items()},
        "hbm_GBps": n_groups_seal * seal_bytes_per_group / t_prefill / 1e9,
        "hbm_frac": n_groups_seal * seal_bytes_per_group / t_prefill / HBM_PEAK,
        "sinkhorn_valu_frac": n_groups_seal * sinkhorn_flops_per_group / t_prefill / VALU_FP32_PEAK,
        "valu_peak_TFLOPs": VALU_FP32_PEAK / 1e12,
        "valu_ceiling_groups_per_s": VALU_FP32_PEAK / sinkhorn_flops_per_group,
        "note": "bulk ingest via kvarn_prefill (sink/tail copy + seal kernel), K and V tiles; median of 50 "
                "graph replays; VALU fraction of the Sinkhorn FMAs against the non-packed fp32 peak",
    }
    print(f"[bench] seal: {seal['groups_per_s'] / 1e6:.2f} M groups/s ({seal['hbm_frac'] * 100:.1f}% of HBM, "
          f"{seal['sinkhorn_valu_frac'] * 100:.1f}% of the VALU peak)", file=sys.stderr, flush=True)

    # ---- record -> fp16 conversion of every record slot of layer 0, timed ----
    gb = k_rec + v_rec
    slots = cache0.records.view(torch.uint8).reshape(-1, gb)
    dq_out = torch.empty(slots.shape[0], 128, d, dtype=torch.float16, device=dev)
    for kind, lo, bits in (("k", 0, wl.k_bits), ("v", k_rec, wl.v_bits)):
        K.dequant_records(slots[:, lo:], d, bits, kind, out=dq_out)
    torch.cuda.synchronize()
    dq_reps = 5
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(dq_reps):
        for kind, lo, bits in (("k", 0, wl.k_bits), ("v", k_rec, wl.v_bits)):
            K.dequant_records(slots[:, lo:], d, bits, kind, out=dq_out)
    e1.record()
    torch.cuda.synchronize()
    t_dq = e0.elapsed_time(e1) / 1e3 / dq_reps
    dq_bytes = slots.shape[0] * (k_rec + v_rec + 2 * 128 * d * 2)   # records in, fp16 tiles out
    dequant = {"records_per_s": 2 * slots.shape[0] / t_dq, "us_per_call": t_dq * 1e6 / 2,
               "hbm_GBps": dq_bytes / t_dq / 1e9, "hbm_frac": dq_bytes / t_dq / HBM_PEAK,
               "note": f"kvarn_dequant_records over all {slots.shape[0]} record slots, K then V"}
    del dq_out
    print(f"[bench] record -> fp16: {dequant['hbm_GBps']:.0f} GB/s ({dequant['hbm_frac'] * 100:.1f}% of HBM)",
          file=sys.stderr, flush=True)

    # ---- chunked-prefill attention over records: the last `chunk` positions
    # of the prompt attend causally over the cache (cache0 holds the prompt)
    chunk = min(args.prefill_chunk, min(lens0))
    qp = torch.from_numpy(np.random.default_rng(5).standard_normal((B, chunk, hq, d)).astype(np.float16)).to(dev)
    outp = torch.empty(B, chunk, hq, d, dtype=torch.float32, device=dev)
    gp = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gp, stream=stream):
        cache0.prefill_attn(qp, out=outp, stream=stream)
    t_pa = _timed_replays(torch, stream, gp, 20)
    del gp
    st_pa = _stats(t_pa)
    # useful flops: QK and PV over positions 0..p for every query row
    pa_flops = sum(hq * 4 * d * sum(n - chunk + i + 1 for i in range(chunk)) for n in lens0)
    prefill_attn = {
        "chunk": chunk, "us_per_call": st_pa["median"] * 1e6,
        "us_stats": {k: (v * 1e6 if k != "reps" else v) for k, v in st_pa.items()},
        "tflops": pa_flops / st_pa["median"] / 1e12,
        "roofline": {"bound": "mfma", "achieved": pa_flops / st_pa["median"] / 1e12,
                     "peak": MFMA_F16_PEAK / 1e12, "unit": "TFLOP/s",
                     "frac": pa_flops / st_pa["median"] / MFMA_F16_PEAK},
        "query_tokens_per_s": B * chunk / st_pa["median"],
        "note": (f"kvarn_prefill_attn: the last {chunk} prompt positions attend causally over the {lens0[0]}-token "
                 "cache (records read directly); flops = 4 D (p+1) per query row and head (QK and PV), against "
                 "the dense fp16 MFMA peak; median of 20 graph replays"),
    }
    del qp, outp
    print(f"[bench] prefill attention, {chunk}-token chunk over {lens0[0]}: {st_pa['median'] * 1e6:.1f} us, "
          f"{prefill_attn['tflops']:.1f} TFLOP/s ({prefill_attn['roofline']['frac'] * 100:.1f}% of fp16 MFMA peak)",
          file=sys.stderr, flush=True)

    # ---- layer caches at their phases -------------------------------------
    caches = [cache0]
    for c in range(1, ncopy):
        caches.append(K.KVarNCache(cfg, B, max_groups, device=dev))
    # ---- multi-layer bulk seal: one prompt into every layer cache, one
    # kvarn_prefill_layers call (one seal launch per 16 layers) against a
    # loop of per-layer kvarn_prefill calls, for a short and the full prompt.
    seal_layers = {}
    for label, plen in (("prompt_2k", [min(2048, n) for n in lens0]), ("prompt_full", lens0)):
        g_layers = sum(hkv * ((n - 128) // 128) for n in plen if n > 128) * ncopy
        graphs = {}
        for mode in ("per_layer", "one_call"):
            gg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gg, stream=stream):
                if mode == "per_layer":
                    for c in caches:
                        c.prefill(k_all, v_all, plen, stream=stream)
                else:
                    K.prefill_layers(caches, [k_all] * ncopy, [v_all] * ncopy, plen, stream=stream)
            graphs[mode] = gg
        res = {"groups_per_call": g_layers, "layers": ncopy, "prompt_tokens": plen[0]}
        for mode, gg in graphs.items():
            t = float(np.median(_timed_replays(torch, stream, gg, 20)))
            res[mode] = {"us_per_call": t * 1e6, "groups_per_s": g_layers / t,
                         "hbm_frac": g_layers * seal_bytes_per_group / t / HBM_PEAK}
        del graphs
        seal_layers[label] = res
        print(f"[bench] multi-layer seal, {plen[0]}-token prompt x {ncopy} layers: one call "
              f"{res['one_call']['groups_per_s'] / 1e6:.2f} M groups/s vs per-layer "
              f"{res['per_layer']['groups_per_s'] / 1e6:.2f} M groups/s", file=sys.stderr, flush=True)
    seal_layers["note"] = ("kvarn_prefill_layers over all layer caches (one seal launch per 16 layers) vs one "
                           "kvarn_prefill per layer, both captured in a HIP graph; median of 20 replays")

    for c in range(ncopy):
        caches[c].prefill(k_all, v_all, lens_c[c])
    seq0 = [c.seq_len.clone() for c in caches]
    outs = [torch.empty(B, hq, d, dtype=torch.float32, device=dev) for _ in range(ncopy)]
    torch.cuda.synchronize()

    def reset():
        for c, s0 in zip(caches, seq0):
            c.seq_len.copy_(s0)

    def step(s):
        # kvarn_decode_step with the lengths the host keeps: the append rides
        # in the decode launches unless the token completes a group.
        c = s % ncopy
        tok = s // ncopy
        caches[c].decode_step(new_k[c, tok], new_v[c, tok], q_all[tok], lengths=[n + tok for n in lens_c[c]],
                              out=outs[c])

    if args.profile_steps > 0:
        for s in range(args.profile_steps):
            step(s)
        torch.cuda.synchronize()
        print(f"[bench] profile run: {args.profile_steps} eager steps done", file=sys.stderr, flush=True)
        return

    # ---- graphs ------------------------------------------------------------
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
    flush()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        g_main.replay()
        ev1.record(stream)
    torch.cuda.synchronize()
    t_total = ev0.elapsed_time(ev1) / 1e3
    seals_timed = sum(1 for s in range(args.steps)
                      if (lens_c[s % ncopy][0] + s // ncopy + 1 - 128) % 128 == 0)
    steps_per_s = args.steps / t_total
    value = B * steps_per_s
    # The same K steps again, 50 times (lengths reset, Infinity Cache flushed
    # before each): distribution of the per-step time.
    t_step_reps = _timed_replays(torch, stream, g_main, 50, before=lambda: (reset(), flush()), per=args.steps)
    del g_main, g_warm

    # ---- live timing of the dominant kernel (the split kernel) and the combine
    def time_graph(fn, reps_graph=50):
        reset()
        torch.cuda.synchronize()
        n = 8 * ncopy
        gk = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gk, stream=stream):
            for r in range(n):
                fn(r)
        torch.cuda.synchronize()
        gk.replay()  # warm
        torch.cuda.synchronize()
        ts = _timed_replays(torch, stream, gk, reps_graph, per=n)
        del gk
        return _stats(ts)

    # A/B for folding the append (and seal-if-due) into the decode launches:
    # the same steps without the append launch bound what a fused step saves.
    st_noappend = time_graph(lambda r: caches[r % ncopy].decode_attn(q_all[0], out=outs[r % ncopy]))
    st_kernel = time_graph(lambda r: caches[r % ncopy].decode_partial(q_all[0]))
    st_combine = time_graph(lambda r: caches[r % ncopy].decode_combine(outs[r % ncopy]))
    t_kernel, t_combine = st_kernel["median"], st_combine["median"]

    # ---- one streaming seal event (the append that completes a group, K and
    # V of every KV head sealed in the same launch) against an append that
    # seals nothing: every layer cache is put 127 tokens into its tail (the
    # tail rows are real tokens of the stream), then one graph of append+seal
    # launches over the layer caches is timed, each launch sealing a group.
    n_due = lens0[0] + 127
    def set_len(n):
        for c in caches:
            c.seq_len.fill_(n)
    saved_tails = [(c.tail_k.clone(), c.tail_v.clone()) for c in caches]
    for c in caches:   # the prompt's last 127 tokens stand in for the tail
        c.tail_k[:, :, :127].copy_(k_all[:, :, lens0[0] - 127:lens0[0]])
        c.tail_v[:, :, :127].copy_(v_all[:, :, lens0[0] - 127:lens0[0]])
    ev_times = {}
    for label, n in (("seal_event", n_due), ("append_only", lens0[0])):
        set_len(n)
        torch.cuda.synchronize()
        gs = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gs, stream=stream):
            for r in range(ncopy):
                caches[r].append_seal(new_k[0, 0], new_v[0, 0])
        ts = _timed_replays(torch, stream, gs, 50, before=lambda: set_len(n), per=ncopy)
        ev_times[label] = _stats([t * 1e6 for t in ts])
        del gs
        n_after = int(caches[-1].seq_len[0].item())
        if n_after != n + 1:
            raise RuntimeError(f"{label}: length {n_after} after the append, expected {n + 1}")
    for c, (tk, tv) in zip(caches, saved_tails):
        c.tail_k.copy_(tk)
        c.tail_v.copy_(tv)
    del saved_tails
    reset()
    seal_event = {"us_seal_event": ev_times["seal_event"]["median"],
                  "us_append_only": ev_times["append_only"]["median"],
                  "seal_event_stats_us": ev_times["seal_event"], "append_only_stats_us": ev_times["append_only"],
                  "tiles": 2 * B * hkv,
                  "note": "kvarn_append_seal launches back to back in a graph over the layer caches: each "
                          "completes a group (K and V of every KV head sealed) vs each only appends; "
                          "median of 50 replays"}
    print(f"[bench] seal event: {seal_event['us_seal_event']:.2f} us per append+seal launch that seals "
          f"{2 * B * hkv} tiles; {seal_event['us_append_only']:.2f} us when nothing is due",
          file=sys.stderr, flush=True)

    # ---- streaming-read ceiling: the plain read probe over 4 GiB
    # (reported beside the 8 TB/s peak; not the target)
    del flush_buf
    rd = torch.zeros(2**32, dtype=torch.uint8, device=dev)
    probe.read(rd, flush_sink)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        probe.read(rd, flush_sink)
    e1.record()
    torch.cuda.synchronize()
    read_ceiling = rd.numel() * 5 / (e0.elapsed_time(e1) / 1e3)
    del rd
    print(f"[bench] streaming-read ceiling (read probe over 4 GiB): {read_ceiling / 1e12:.2f} TB/s",
          file=sys.stderr, flush=True)
    # Algorithmic bytes of one split-kernel launch, averaged over the layer
    # caches the timing graph rotates over (their phases differ in tail length).
    bytes_launch = float(np.mean([algorithmic_decode_bytes(wl, lens_c[c], k_rec, v_rec) for c in range(ncopy)]))
    achieved = bytes_launch / t_kernel
    traffic = read_traffic(wl.name)
    print(f"[bench] decode split kernel: {t_kernel * 1e6:.2f} us/launch, {achieved / 1e12:.2f} TB/s "
          f"({achieved / HBM_PEAK * 100:.1f}% of HBM); combine {t_combine * 1e6:.2f} us; "
          f"step {t_total / args.steps * 1e6:.2f} us; plan {plan}", file=sys.stderr, flush=True)

    # ---- the same split kernel over paged records: every layer cache's
    # records moved to a shuffled block table over a pool with spare blocks.
    nblk = B * max_groups + 64
    perm = torch.from_numpy(np.random.default_rng(11).permutation(nblk)[:B * max_groups].astype(np.int32)).to(dev)
    reset()
    paged = []
    for c in caches:
        pc = K.KVarNCache(cfg, B, max_groups, device=dev, num_blocks=nblk)
        pc.block_table.copy_(perm.view(B, max_groups))
        src = c.records.view(B, hkv, max_groups, gb).permute(0, 2, 1, 3).reshape(B * max_groups, hkv, gb)
        pc.records.view(nblk, hkv, gb)[perm.long()] = src
        for name in ("sink_k", "sink_v", "tail_k", "tail_v", "seq_len"):
            getattr(pc, name).copy_(getattr(c, name))
        paged.append(pc)
    torch.cuda.synchronize()
    pdiff = (paged[0].decode_attn(q_all[0]) - caches[0].decode_attn(q_all[0])).abs().max().item()
    if not pdiff <= 1e-5:
        raise RuntimeError(f"paged decode differs from the contiguous one by {pdiff}")
    st_paged = time_graph(lambda r: paged[r % ncopy].decode_partial(q_all[0]))
    t_paged = st_paged["median"]
    paged_line = {"us_per_launch": t_paged * 1e6, "GBps": bytes_launch / t_paged / 1e9,
                  "frac": bytes_launch / t_paged / HBM_PEAK,
                  "us_stats": {k: (v * 1e6 if k != "reps" else v) for k, v in st_paged.items()},
                  "note": f"decode split kernel, records behind a shuffled block table over {nblk} blocks"}
    del paged
    print(f"[bench] paged records: split kernel {t_paged * 1e6:.2f} us/launch "
          f"({paged_line['frac'] * 100:.1f}% of HBM)", file=sys.stderr, flush=True)

    others = {}
    for name in [x for x in args.other_workloads.split(",") if x and x != wl.name]:
        others[name] = measure_workload(torch, K, probe, synth, dev, name, args.other_steps)
        o = others[name]
        print(f"[bench] {name}: {o['tokens_per_s']:.0f} tokens/s, step {o['ms_per_step'] * 1e3:.1f} us, split "
              f"{o['roofline']['us_per_launch']:.1f} us = {o['roofline']['achieved']:.0f} GB/s "
              f"({o['roofline']['frac'] * 100:.1f}% of HBM); seal {o['seal']['groups_per_s'] / 1e6:.2f} M groups/s",
              file=sys.stderr, flush=True)

    us = lambda st: {k: (v * 1e6 if k != "reps" else v) for k, v in st.items()}
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
                   "tail_phase": f"layer c starts 127 - floor(128 c / {ncopy}) tokens into its tail",
                   "max_groups": max_groups, "seals_in_timed_steps": seals_timed,
                   "step": "kvarn_decode_step: append + seal-if-due + decode attention (one layer); the "
                           "append rides in the decode launches unless the token completes a group"},
        "step_us_stats": us(_stats(t_step_reps)),
        "step_without_append_us_stats": us(st_noappend),
        "seal_cadence": {
            "us_step_no_seal": float(np.median(t_step_reps)) * 1e6,
            "us_step_with_seal": seal_event["us_seal_event"] + us(st_noappend)["median"],
            "us_per_step_one_seal_per_128": (127 * float(np.median(t_step_reps)) * 1e6
                                             + seal_event["us_seal_event"] + us(st_noappend)["median"]) / 128,
            "note": "a step that completes a group is the append+seal launch (seal_event) followed by the decode "
                    "launches (step_without_append); every request seals once per 128 steps",
        },
        "decode_plan": plan,
        "roofline": {"bound": "hbm", "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK, "traffic": traffic,
                     "kernel": "decode_split_kernel", "bytes_per_launch": bytes_launch,
                     "us_per_launch": t_kernel * 1e6, "us_stats": us(st_kernel),
                     "combine_us_per_launch": t_combine * 1e6, "combine_us_stats": us(st_combine),
                     "read_ceiling_GBps": read_ceiling / 1e9, "frac_of_read_ceiling": achieved / read_ceiling},
        "seal_event": seal_event,
        "seal": seal,
        "seal_layers": seal_layers,
        "prefill_attn": prefill_attn,
        "dequant": dequant,
        "paged": paged_line,
        "workloads": others,
    }
    line["cpu_baseline"] = cpu_line
    print(json.dumps(line))


if __name__ == "__main__":
    main()
