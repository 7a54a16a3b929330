"""Helpers shared by the GPU parity tests (comparison rules and cache upload).

Comparison rules for a sealed tile, GPU vs oracle:
  * packing and indexing: the GPU record must equal, byte for byte, the
    oracle's own packing of the oracle's codes and fp16 scales, where only the
    entries accepted below as legitimate rounding ties take the GPU's value;
  * pre-rounding scales s_t, c_j (GPU debug output, fp32) within 1e-5 relative
    of the float64 oracle;
  * codes: at least 99.99% identical, never more than one level apart, and a
    differing code is only accepted where the oracle's pre-rounding value
    u = Y/delta + mid lies within CODE_TIE_TOL of a rounding boundary
    (u - floor(u) = 1/2): there the fp32 kernel and the float64 oracle may
    legitimately round to different neighbours;
  * stored fp16 scales: identical, except one ulp apart where the float64
    value lies within 1e-5 relative of the midpoint between two fp16 values.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import kvarn_oracle as O

SCALE_RTOL = 1e-5
CODE_MATCH_MIN = 0.9999
CODE_TIE_TOL = 2e-4
ATTN_ATOL = 2e-3


def fp16_tie_ok(x64: np.ndarray, a16: np.ndarray, b16: np.ndarray) -> np.ndarray:
    """True where a16 == b16, or both are neighbours of x64 near a midpoint."""
    same = a16.view(np.uint16) == b16.view(np.uint16)
    x = np.asarray(x64, dtype=np.float64)
    lo = x.astype(np.float16)
    lo = np.where(lo.astype(np.float64) > x, np.nextafter(lo, np.float16(-np.inf)), lo)
    hi = np.nextafter(lo, np.float16(np.inf))
    mid = (lo.astype(np.float64) + hi.astype(np.float64)) / 2
    near = np.abs(x - mid) <= SCALE_RTOL * np.abs(x)
    pair = ((a16 == lo) | (a16 == hi)) & ((b16 == lo) | (b16 == hi))
    return same | (near & pair)


def check_sealed_tile(rec: bytes, dbg: np.ndarray | None, ref: dict, d: int, bits: int, kind: str,
                      stats: dict | None = None) -> None:
    codes, s16, c16 = O.decode_record(rec, d, bits, kind)
    if dbg is not None:
        s_g, c_g = dbg[:O.GROUP].astype(np.float64), dbg[O.GROUP:].astype(np.float64)
        zero = ref["s"] == 0
        assert np.all(s_g[zero] == 0)
        rs = np.abs(s_g[~zero] / ref["s"][~zero] - 1)
        rc = np.abs(c_g / ref["c"] - 1)
        assert rs.max(initial=0) <= SCALE_RTOL, f"token scale rel err {rs.max()}"
        assert rc.max(initial=0) <= SCALE_RTOL, f"channel scale rel err {rc.max()}"
    diff = codes.astype(np.int32) - ref["codes"].astype(np.int32)
    assert np.abs(diff).max(initial=0) <= 1
    bad = diff != 0
    if bad.any():
        delta = ref["delta"]
        u = ref["y"] / np.where(delta == 0, 1, delta)[:, None] + ref["mid"]
        frac = u - np.floor(u)
        assert np.all(np.abs(frac[bad] - 0.5) <= CODE_TIE_TOL), "a code differs away from a rounding tie"
    assert 1 - bad.mean() >= CODE_MATCH_MIN
    assert np.all(fp16_tie_ok(ref["s"], s16, ref["s16"])), "stored token scales differ"
    assert np.all(fp16_tie_ok(ref["c"], c16, ref["c16"])), "stored channel scales differ"
    # Packing and indexing, bit-exact: the oracle packs its own codes and
    # scales, with the GPU's value only where a tie was accepted above.
    exp_codes = np.where(bad, codes, ref["codes"])
    exp_s16 = np.where(s16.view(np.uint16) == ref["s16"].view(np.uint16), ref["s16"], s16)
    exp_c16 = np.where(c16.view(np.uint16) == ref["c16"].view(np.uint16), ref["c16"], c16)
    assert O.encode_record(exp_codes, exp_s16, exp_c16, bits, kind) == rec, "packing is not bit-exact"
    if stats is not None:
        stats["codes"] = stats.get("codes", 0) + codes.size
        stats["code_mismatch"] = stats.get("code_mismatch", 0) + int(bad.sum())


def upload_states(cache, states) -> None:
    """Copy oracle states [b][h] (KVarNState) into a device KVarNCache."""
    dev = cache.sink_k.device
    seq = []
    for b, row in enumerate(states):
        n = row[0].n
        seq.append(n)
        for h, st in enumerate(row):
            assert st.n == n
            if st.sink_k:
                cache.sink_k[b, h, :len(st.sink_k)] = torch.from_numpy(np.stack(st.sink_k)).to(dev)
                cache.sink_v[b, h, :len(st.sink_v)] = torch.from_numpy(np.stack(st.sink_v)).to(dev)
            if st.tail_k:
                cache.tail_k[b, h, :st.tail_len] = torch.from_numpy(np.stack(st.tail_k)).to(dev)
                cache.tail_v[b, h, :st.tail_len] = torch.from_numpy(np.stack(st.tail_v)).to(dev)
            for g, (rk, rv) in enumerate(zip(st.rec_k, st.rec_v)):
                cache.record(b, h, g, "k").copy_(torch.frombuffer(bytearray(rk), dtype=torch.uint8).to(dev))
                cache.record(b, h, g, "v").copy_(torch.frombuffer(bytearray(rv), dtype=torch.uint8).to(dev))
    cache.seq_len.copy_(torch.tensor(seq, dtype=torch.int32, device=dev))
