"""KVarN CPU oracle: plain, slow, float64 NumPy definition of the hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library and imports nothing from it.

Sources ("the pages"):

* P1 = "KVarN: Variance-Normalized KV-Cache Quantization Mitigates Error
  Accumulation in Reasoning Tasks", fig1.dev summary of arXiv 2606.03458,
  sections "What it is", "Why it matters", "Practical takeaway", "Key result".
* P2 = "KVarN KV Cache: Implementation and Benchmarks" (anbeeld.com),
  §1 "Where KVarN Comes From", §2.1 "Sink, Body, And Tail",
  §2.2 "What This Implementation Changes".

What the pages fix, and how each step below follows them:

* A Hadamard rotation along the channel axis, per head, applied to post-RoPE
  K and V; the query is rotated by the same matrix so q.k is unchanged and the
  attention output is rotated back once per token (P1 "What it is"; P2 §1).
* A Sinkhorn-style variance normalization over the token and the channel axis,
  run as 16 iterations, rescaling both axes of each matrix (P1 "What it is";
  P2 §1).
* Round-to-nearest quantization afterwards (P1 "What it is"), at about 2.3 bits
  per element for the 2-bit cache (P1 "Why it matters", "Key result").
* The first 128 tokens stay exact forever (the sink); later tokens are sealed
  in groups of 128 the moment a group's last token arrives; the partial group
  (the tail) stays exact until it seals; the record keeps the quantized payload
  with its scale metadata (P2 §2.1).

Where the pages leave a step open, the readings taken are (each also listed in
the design notes of the repository):

R1  Hadamard = Sylvester construction in natural order, scaled by 1/sqrt(D),
    no random signs (the plainest deterministic reading of "a Hadamard
    rotation"; it is symmetric and orthonormal).
R2  Sink and tail are stored exactly as appended (original frame, fp16 bits);
    only sealed groups are rotated.
R3  "Variance" = mean square about zero; each Sinkhorn step divides a row
    (column) by its root mean square so its mean square becomes 1.
R4  One iteration = token (row) step, then channel (column) step; exactly 16
    iterations; factors start at 1; no damping or early exit.
R5  A row or column whose mean square is 0 keeps factor 1.
R6  RTN grid: symmetric mid-rise uniform grid per token, levels (k - mid)*delta,
    k = 0..2^b-1, mid = (2^b-1)/2, delta_t = 2*max_j|Y_tj|/(2^b-1) taken from
    the normalized tile, so nothing clips.  The token step folds into the
    stored per-token scale s_t = r_t*delta_t; c_j is the per-channel scale.
R7  Ties round half to even; an all-zero token row gets code 2^(b-1), s_t = 0.
R8  s and c are stored as fp16 (round to nearest even); codes come from the
    unrounded float64 values; dequantization uses the stored fp16 scales.
R9  Record = [codes][s: 128 x fp16][c: D x fp16].  K codes token-major (row t
    holds token t's D codes), V codes channel-major (row j holds channel j's
    128 codes).  A row is a little-endian bit stream: code i occupies bits
    [b*i, b*i + b) (bit k of the row is bit k mod 8 of byte k div 8).  For
    b = 2, 4, 8 this is code i at bit b*(i mod 32/b) of the 32-bit
    little-endian word floor(i*b/32).
R15 Widths: b in {2, 3, 4, 5, 6, 8} for K and V independently.  The pages
    name whole widths from two to eight bits and K/V pairs built from them
    (P2 §5 "Changing Only The Format", §6 "Splitting K And V"); seven bits is
    named by none of them and is left out.
R10 Sink = positions [0, 128); group g = positions [128+128g, 256+128g), sealed
    when position 255+128g is appended.  A decode step is append -> seal if
    due -> attend.
R12 Attention: scale 1/sqrt(D), the query attends to every cached position
    (its own included), no mask; query head h reads KV head floor(h*Hkv/Hq).
R13 K and V go through the identical procedure, each with its own bit width.

Parity status: the Hadamard, rotation invariance, Sinkhorn behaviour, RTN,
packing, sink/tail state machine and decode are pinned by the tests in
``tests/test_oracle_*.py`` against closed forms, library routines, brute force
and the page constants in ``tests/golden/``.  The quantizer choices R3, R6, R7,
R8 and R9 are readings of silent pages: no page prints a tile, a scale or a
code, so those choices are parity unpinned beyond this frozen specification.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np

GROUP = 128          # tokens per sealed group (P2 §2.1)
SINK = 128           # permanently exact leading tokens (P2 §2.1)
TAIL_CAP = 128       # region R: the exact in-progress group (P2 §2.1)
SINKHORN_ITERS = 16  # P2 §1
WIDTHS = (2, 3, 4, 5, 6, 8)  # code widths in bits (reading R15)


# --------------------------------------------------------------------------
# Hadamard rotation (P1 "What it is"; P2 §1; reading R1)
# --------------------------------------------------------------------------
def sylvester(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix H_d with entries +-1 (int64), natural order.

    H_1 = [1]; H_2n = [[H_n, H_n], [H_n, -H_n]].
    """
    if d < 1 or d & (d - 1):
        raise ValueError("Hadamard size must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation(d: int) -> np.ndarray:
    """Orthonormal channel rotation H_d / sqrt(d) (float64, symmetric)."""
    return sylvester(d).astype(np.float64) / np.sqrt(d)


def rotate_rows(x: np.ndarray) -> np.ndarray:
    """x [..., D] -> x @ (H_D / sqrt(D)) in float64 (rows are tokens)."""
    x = np.asarray(x, dtype=np.float64)
    return x @ rotation(x.shape[-1])


# --------------------------------------------------------------------------
# Sinkhorn-style variance normalization (P1 "What it is"; P2 §1; R3-R5)
# --------------------------------------------------------------------------
def sinkhorn(xr: np.ndarray, iters: int = SINKHORN_ITERS, history: Optional[list] = None):
    """Literal alternating rescaling of a rotated tile xr [T][D] (float64).

    Each iteration divides every token row by its root mean square, then every
    channel column by its root mean square, and multiplies the running factors
    r (per token) and c (per channel) by the divisors.  Returns (Y, r, c) with
    Y = xr / (r c^T).

    If ``history`` is a list, the row and column mean squares of Y before each
    half-step are appended to it (used by the convergence tests).
    """
    y = np.array(xr, dtype=np.float64, copy=True)
    t, d = y.shape
    r = np.ones(t)
    c = np.ones(d)
    for _ in range(iters):
        rho = np.sqrt(np.mean(y * y, axis=1))
        if history is not None:
            history.append(("row", rho ** 2, np.mean(y * y, axis=0)))
        rho = np.where(rho == 0.0, 1.0, rho)
        y = y / rho[:, None]
        r = r * rho
        gam = np.sqrt(np.mean(y * y, axis=0))
        if history is not None:
            history.append(("col", np.mean(y * y, axis=1), gam ** 2))
        gam = np.where(gam == 0.0, 1.0, gam)
        y = y / gam[None, :]
        c = c * gam
    return y, r, c


# --------------------------------------------------------------------------
# Round to nearest (P1 "What it is"; readings R6-R8)
# --------------------------------------------------------------------------
def rtn(y: np.ndarray, bits: int):
    """Per-token symmetric mid-rise RTN of a normalized tile y [T][D].

    Returns (codes uint8 [T][D], delta [T], mid).  code = clip(rint(y/delta +
    mid), 0, 2^b-1) with rint = round half to even; a zero row gets 2^(b-1).
    """
    if bits not in WIDTHS:
        raise ValueError(f"bits must be one of {WIDTHS}")
    levels = (1 << bits) - 1
    mid = levels / 2.0
    m = np.max(np.abs(y), axis=1)
    delta = 2.0 * m / levels
    codes = np.empty(y.shape, dtype=np.uint8)
    for t in range(y.shape[0]):
        if delta[t] == 0.0:
            codes[t, :] = 1 << (bits - 1)
        else:
            codes[t, :] = np.clip(np.rint(y[t] / delta[t] + mid), 0, levels).astype(np.uint8)
    return codes, delta, mid


def seal_tile(x: np.ndarray, bits: int, iters: int = SINKHORN_ITERS) -> dict:
    """Seal one [T][D] fp16 tile (T = 128 for a real group).

    Steps: rotate (float64) -> ``iters`` Sinkhorn iterations -> RTN.  Returns
    a dict with codes, float64 s and c, their fp16 versions, the normalized
    tile Y, the factors r and the per-token step delta.
    """
    x = np.asarray(x)
    if x.dtype != np.float16:
        raise TypeError("tiles are fp16")
    xr = rotate_rows(x.astype(np.float64))
    y, r, c = sinkhorn(xr, iters)
    codes, delta, mid = rtn(y, bits)
    s = r * delta
    return dict(codes=codes, s=s, c=c, s16=s.astype(np.float16), c16=c.astype(np.float16),
                y=y, r=r, delta=delta, mid=mid, xr=xr)


# --------------------------------------------------------------------------
# Comparison quantizers for the error-accumulation harness (not KVarN): the
# baselines the pages set KVarN against -- RTN without the variance
# normalization, with per-channel or per-token steps (P1 "What it is": KIVI-
# style per-channel keys; P2 §1: per-token scales and their error).  Each
# returns the fake-quantized tile (dequantized, float64, original frame).
# --------------------------------------------------------------------------
def fake_quant_rtn(x: np.ndarray, bits: int, axis: str, rotate: bool = False,
                   scale16: bool = True) -> np.ndarray:
    """Symmetric mid-rise RTN of a tile x [T][D] with one step per token row
    (axis 'token') or per channel column (axis 'channel'), optionally in the
    Hadamard frame (rotate=True: quantize x H/sqrt(D), rotate back).  The step
    of a row/column is 2 max|.|/(2^b - 1) (no clipping), rounded to fp16 when
    scale16, as the record stores its scales; ties round half to even."""
    if axis not in ("token", "channel"):
        raise ValueError("axis must be 'token' or 'channel'")
    y = np.asarray(x, dtype=np.float64)
    if rotate:
        y = rotate_rows(y)
    if axis == "channel":
        y = y.T
    levels = (1 << bits) - 1
    mid = levels / 2.0
    delta = 2.0 * np.max(np.abs(y), axis=1) / levels
    # Codes from the unrounded step, reconstruction from the stored one
    # (as for KVarN's records, reading R8).
    stored = delta.astype(np.float16).astype(np.float64) if scale16 else delta
    out = np.zeros_like(y)
    for i in range(y.shape[0]):
        if delta[i] > 0:
            q = np.clip(np.rint(y[i] / delta[i] + mid), 0, levels)
            out[i] = (q - mid) * stored[i]
    if axis == "channel":
        out = out.T
    if rotate:
        out = out @ rotation(out.shape[1]).T
    return out


def fake_quant_kvarn(x: np.ndarray, bits: int, kind: str, iters: int = SINKHORN_ITERS) -> np.ndarray:
    """KVarN's record of a tile, decoded back (original frame, float64):
    seal_tile with ``iters`` iterations (0 = rotation-only: per-token RTN in
    the Hadamard frame), encoded and dequantized from the stored scales."""
    out = seal_tile(np.asarray(x, dtype=np.float16), bits, iters)
    rec = encode_record(out["codes"], out["s16"], out["c16"], bits, kind)
    return dequant_record(rec, x.shape[1], bits, kind)


# --------------------------------------------------------------------------
# Packing and the record layout (P2 §2.1 "payload with its scale metadata"; R9)
# --------------------------------------------------------------------------
def pack_row(codes: np.ndarray, bits: int) -> bytes:
    """Pack one row of codes as a little-endian bit stream: code i occupies
    bits [b*i, b*i + b) (reading R9)."""
    n = len(codes)
    if (n * bits) % 8:
        raise ValueError("row length times bits must fill whole bytes")
    v = 0
    for i in range(n):
        code = int(codes[i])
        if code < 0 or code >> bits:
            raise ValueError("code out of range")
        v |= code << (bits * i)
    return v.to_bytes(n * bits // 8, "little")


def unpack_row(buf: bytes, n: int, bits: int) -> np.ndarray:
    v = int.from_bytes(bytes(buf), "little")
    out = np.empty(n, dtype=np.uint8)
    for i in range(n):
        out[i] = (v >> (bits * i)) & ((1 << bits) - 1)
    return out


def record_bytes(d: int, bits: int, tokens: int = GROUP) -> int:
    """Bytes of one record: codes + tokens fp16 s + d fp16 c."""
    return tokens * d * bits // 8 + 2 * tokens + 2 * d


def encode_record(codes: np.ndarray, s16: np.ndarray, c16: np.ndarray, bits: int, kind: str) -> bytes:
    """Serialize a sealed tile. kind 'k' = token-major codes, 'v' = channel-major."""
    t, d = codes.shape
    rows = codes if kind == "k" else codes.T
    if kind not in ("k", "v"):
        raise ValueError("kind must be 'k' or 'v'")
    payload = b"".join(pack_row(row, bits) for row in rows)
    return payload + np.asarray(s16, dtype="<f2").tobytes() + np.asarray(c16, dtype="<f2").tobytes()


def decode_record(buf: bytes, d: int, bits: int, kind: str, tokens: int = GROUP):
    """Inverse of encode_record: (codes [T][D], s16 [T], c16 [D])."""
    nbytes = record_bytes(d, bits, tokens)
    if len(buf) != nbytes:
        raise ValueError(f"record is {len(buf)} bytes, expected {nbytes}")
    code_bytes = tokens * d * bits // 8
    if kind == "k":
        row_len, nrows = d, tokens
    else:
        row_len, nrows = tokens, d
    rb = row_len * bits // 8
    rows = [unpack_row(buf[i * rb:(i + 1) * rb], row_len, bits) for i in range(nrows)]
    codes = np.stack(rows)
    if kind == "v":
        codes = codes.T
    s16 = np.frombuffer(buf[code_bytes:code_bytes + 2 * tokens], dtype="<f2").copy()
    c16 = np.frombuffer(buf[code_bytes + 2 * tokens:], dtype="<f2").copy()
    return np.ascontiguousarray(codes), s16, c16


def dequant(codes: np.ndarray, s16: np.ndarray, c16: np.ndarray, bits: int) -> np.ndarray:
    """Original-frame float64 reconstruction from stored fp16 scales.

    X_hat = (s_t * (q_tj - mid) * c_j) @ (H_D / sqrt(D))^T.
    """
    mid = ((1 << bits) - 1) / 2.0
    yr = s16.astype(np.float64)[:, None] * (codes.astype(np.float64) - mid) * c16.astype(np.float64)[None, :]
    return yr @ rotation(codes.shape[1]).T


def dequant_record(buf: bytes, d: int, bits: int, kind: str) -> np.ndarray:
    codes, s16, c16 = decode_record(buf, d, bits, kind)
    return dequant(codes, s16, c16, bits)


# --------------------------------------------------------------------------
# Attention over the cache (P2 §1 rotated frame; P2 §2.1 records; R12)
# --------------------------------------------------------------------------
def attention(q: np.ndarray, k_all: np.ndarray, v_all: np.ndarray, scale: Optional[float] = None) -> np.ndarray:
    """softmax(k_all q * scale) @ v_all for one query row, float64."""
    q = np.asarray(q, dtype=np.float64)
    k_all = np.asarray(k_all, dtype=np.float64)
    v_all = np.asarray(v_all, dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    logits = k_all @ q * scale
    p = np.exp(logits - logits.max())
    return (p @ v_all) / p.sum()


class KVarNState:
    """Cache of one (request, KV head): sink, sealed records and tail.

    ``append`` stores a token at position n (sink if n < 128, else the tail),
    increments n, and seals the tail into a record when it has just filled
    (reading R10).  Records are kept as bytes in the layout of reading R9.
    """

    def __init__(self, head_dim: int, k_bits: int, v_bits: int):
        self.d = head_dim
        self.k_bits = k_bits
        self.v_bits = v_bits
        self.n = 0
        self.sink_k: List[np.ndarray] = []
        self.sink_v: List[np.ndarray] = []
        self.tail_k: List[np.ndarray] = []
        self.tail_v: List[np.ndarray] = []
        self.rec_k: List[bytes] = []
        self.rec_v: List[bytes] = []
        self.seal_positions: List[int] = []

    @property
    def tail_len(self) -> int:
        return len(self.tail_k)

    def append(self, k: np.ndarray, v: np.ndarray) -> bool:
        """Append one fp16 token; returns True if this token sealed a group."""
        k = np.asarray(k, dtype=np.float16).copy()
        v = np.asarray(v, dtype=np.float16).copy()
        pos = self.n
        if pos < SINK:
            self.sink_k.append(k)
            self.sink_v.append(v)
        else:
            self.tail_k.append(k)
            self.tail_v.append(v)
        self.n += 1
        if self.n >= SINK + GROUP and (self.n - SINK) % GROUP == 0:
            tk = np.stack(self.tail_k)
            tv = np.stack(self.tail_v)
            sk = seal_tile(tk, self.k_bits)
            sv = seal_tile(tv, self.v_bits)
            self.rec_k.append(encode_record(sk["codes"], sk["s16"], sk["c16"], self.k_bits, "k"))
            self.rec_v.append(encode_record(sv["codes"], sv["s16"], sv["c16"], self.v_bits, "v"))
            self.tail_k.clear()
            self.tail_v.clear()
            self.seal_positions.append(pos)
            return True
        return False

    def extend(self, k: np.ndarray, v: np.ndarray) -> None:
        for i in range(len(k)):
            self.append(k[i], v[i])

    def materialize(self):
        """Float64 original-frame K and V of every cached position, in order."""
        d = self.d
        ks = [np.stack(self.sink_k).astype(np.float64)] if self.sink_k else []
        vs = [np.stack(self.sink_v).astype(np.float64)] if self.sink_v else []
        for rk, rv in zip(self.rec_k, self.rec_v):
            ks.append(dequant_record(rk, d, self.k_bits, "k"))
            vs.append(dequant_record(rv, d, self.v_bits, "v"))
        if self.tail_k:
            ks.append(np.stack(self.tail_k).astype(np.float64))
            vs.append(np.stack(self.tail_v).astype(np.float64))
        return np.concatenate(ks), np.concatenate(vs)

    def attend(self, q: np.ndarray, scale: Optional[float] = None) -> np.ndarray:
        k_all, v_all = self.materialize()
        return attention(q, k_all, v_all, scale)


def decode_attention(q: np.ndarray, states: List[KVarNState], num_kv_heads: int,
                     scale: Optional[float] = None) -> np.ndarray:
    """One request's decode: q [Hq][D] over per-KV-head states -> [Hq][D]."""
    hq = q.shape[0]
    out = np.empty(q.shape, dtype=np.float64)
    mats = [st.materialize() for st in states]
    for h in range(hq):
        kvh = (h * num_kv_heads) // hq
        out[h] = attention(q[h], mats[kvh][0], mats[kvh][1], scale)
    return out


def prefill_attention(q: np.ndarray, states: List[KVarNState], num_kv_heads: int, scale: Optional[float] = None) -> np.ndarray:
    """Chunked-prefill attention of one request over its cache (reading N1).

    q [C][Hq][D]: the queries of the chunk, i.e. of the last C cached
    positions n-C .. n-1, taken after the chunk has been appended and every
    group it completed sealed.  The query at position p attends causally over
    positions 0..p as the cache holds them: the sink and the tail exact, the
    sealed groups through their records (P2 §2.1: attention paths read the
    records; the chunk is appended before its attention, as a decode step
    appends before it attends).  One plain attention per query position and
    head; returns [C][Hq][D] float64.
    """
    c, hq = q.shape[0], q.shape[1]
    n = states[0].n
    if c > n:
        raise ValueError("the chunk is longer than the cache")
    mats = [st.materialize() for st in states]
    out = np.empty(q.shape, dtype=np.float64)
    for i in range(c):
        p = n - c + i
        for h in range(hq):
            kvh = (h * num_kv_heads) // hq
            out[i, h] = attention(q[i, h], mats[kvh][0][:p + 1], mats[kvh][1][:p + 1], scale)
    return out


def seal_stream(k: np.ndarray, v: np.ndarray, k_bits: int, v_bits: int):
    """Records of every complete group of a prefilled fp16 stream [L][D].

    Group g covers positions [128 + 128 g, 256 + 128 g).  Returns two lists of
    record bytes (K and V).
    """
    n_groups = max(0, (len(k) - SINK) // GROUP)
    rk, rv = [], []
    for g in range(n_groups):
        lo = SINK + GROUP * g
        sk = seal_tile(k[lo:lo + GROUP], k_bits)
        sv = seal_tile(v[lo:lo + GROUP], v_bits)
        rk.append(encode_record(sk["codes"], sk["s16"], sk["c16"], k_bits, "k"))
        rv.append(encode_record(sv["codes"], sv["s16"], sv["c16"], v_bits, "v"))
    return rk, rv


def state_from_stream(k: np.ndarray, v: np.ndarray, k_bits: int, v_bits: int) -> KVarNState:
    """A KVarNState holding the first len(k) tokens of a stream (bulk form).

    Equivalent to appending every token one at a time, without the per-token
    Python overhead.
    """
    st = KVarNState(k.shape[1], k_bits, v_bits)
    n = len(k)
    ns = min(n, SINK)
    st.sink_k = [row for row in k[:ns]]
    st.sink_v = [row for row in v[:ns]]
    st.rec_k, st.rec_v = seal_stream(k[:n], v[:n], k_bits, v_bits)
    n_groups = len(st.rec_k)
    st.seal_positions = [SINK + GROUP * g + GROUP - 1 for g in range(n_groups)]
    lo = SINK + GROUP * n_groups
    st.tail_k = [row for row in k[lo:n]] if n > SINK else []
    st.tail_v = [row for row in v[lo:n]] if n > SINK else []
    st.n = n
    return st
