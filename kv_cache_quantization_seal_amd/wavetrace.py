"""Reader of the trace build's per-wave phase timestamps (libkvarn_trace.so,
built with ``python -m kv_cache_quantization_seal_amd.build --trace`` and
selected with KVARN_LIBRARY).  Diagnostic only: the product library has no
trace code.

Each wave slot holds (see csrc/trace.hpp): hardware ids, the core-clock
counter at its start and at its last mark, and the 100 MHz real-time counter
at phase marks 0..11 (0 = start; 0 where a wave did not reach a mark); for
the chunked-prefill attention kernel (a loop over tiles) the slots hold
instead the core-clock cycles of each phase summed over the wave's tiles."""
from __future__ import annotations

import ctypes

import numpy as np

WORDS = 16
SLOTS = 32768
REALTIME_HZ = 100e6
SEAL = 1
PREFILL_ATTN = 2   # loop kernel: record [2 + p] = core-clock cycles of phase p, summed over its tiles


def decode(k_bits: int) -> int:
    """Trace buffer of the decode split kernel for K records of k_bits."""
    return 100 + k_bits


def _lib():
    from kv_cache_quantization_seal_amd import kvarn as K
    L = K.lib()
    if not hasattr(L, "kvarn_trace_io"):
        raise RuntimeError("the loaded library is not the trace build: set KVARN_LIBRARY to libkvarn_trace.so")
    L.kvarn_trace_io.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t]
    L.kvarn_trace_io.restype = ctypes.c_int
    return L


def clear(which: int) -> None:
    if _lib().kvarn_trace_io(which, None, 0) != 0:
        raise RuntimeError("kvarn_trace_io clear failed")


def read(which: int, n_slots: int) -> np.ndarray:
    """uint64 [n_slots][16] records of the first n_slots wave slots."""
    n_slots = min(n_slots, SLOTS)
    buf = np.zeros((n_slots, WORDS), dtype=np.uint64)
    if _lib().kvarn_trace_io(which, buf.ctypes.data, buf.nbytes) != 0:
        raise RuntimeError("kvarn_trace_io read failed")
    return buf


def summarize(rec: np.ndarray, names: dict, groups: dict | None = None) -> dict:
    """Per-phase statistics (us, relative to the earliest wave start) over the
    waves that reached each mark, per named group of slots (default: all
    waves that started), and the core clock from the counters of each wave."""
    started = rec[:, 2] > 0
    if not started.any():
        return {}
    t0 = rec[started, 2].min()
    out = {}
    groups = groups or {"all": np.arange(len(rec))}
    for gname, idx in groups.items():
        idx = np.asarray([i for i in idx if i < len(rec) and started[i]], dtype=np.int64)
        if idx.size == 0:
            continue
        g = {"waves": int(idx.size)}
        for ph, pname in names.items():
            col = rec[idx, 2 + ph]
            ok = col > 0
            if not ok.any():
                continue
            t = (col[ok].astype(np.float64) - float(t0)) / REALTIME_HZ * 1e6
            g[pname] = {"p10": float(np.percentile(t, 10)), "median": float(np.median(t)),
                        "p90": float(np.percentile(t, 90)), "max": float(t.max()), "waves": int(ok.sum())}
        # core clock: core-clock ticks over real time between start and last mark
        last = rec[idx, 2:2 + 12].max(axis=1).astype(np.float64)
        dt = (last - rec[idx, 2].astype(np.float64)) / REALTIME_HZ
        dc = rec[idx, WORDS - 1].astype(np.float64) - rec[idx, 1].astype(np.float64)
        ok = (dt > 2e-6) & (rec[idx, WORDS - 1] > 0)
        if ok.any():
            g["core_clock_GHz"] = float(np.median(dc[ok] / dt[ok]) / 1e9)
        out[gname] = g
    return out
