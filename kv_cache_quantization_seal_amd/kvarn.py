"""ctypes binding of libkvarn.so (the C ABI declared in include/kvarn.h).

Argument marshalling only: every step of the hot path runs in the HIP
kernels.  PyTorch provides device memory and the current HIP stream.  If the
native library is missing, every call raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

# KVARN_LIBRARY may name another build of the same ABI (the trace build,
# libkvarn_trace.so, for per-wave timestamps); the default is libkvarn.so.
_LIB_PATH = os.environ.get("KVARN_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                            "libkvarn.so")
_lib = None

OK, EINVAL, EUNSUPPORTED, ERANGE, EWORKSPACE, EHIP = 0, -1, -2, -3, -4, -5
GROUP = 128
SINK = 128
SINKHORN_ITERS = 16
EXPORTS = (
    "kvarn_check_config", "kvarn_record_bytes", "kvarn_group_bytes", "kvarn_decode_workspace_bytes",
    "kvarn_decode_plan",
    "kvarn_last_error", "kvarn_status_string", "kvarn_append", "kvarn_append_seal", "kvarn_seal_group",
    "kvarn_prefill", "kvarn_prefill_layers",
    "kvarn_decode_attn", "kvarn_decode_attn_noalloc", "kvarn_decode_step", "kvarn_decode_attn_partial",
    "kvarn_decode_attn_combine", "kvarn_seal_tiles",
    "kvarn_dequant_records", "kvarn_prefill_attn",
)


class KvarnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_name(status)}: {message}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32), ("group", ctypes.c_int32),
                ("sink", ctypes.c_int32), ("sinkhorn_iters", ctypes.c_int32)]


class CacheView(ctypes.Structure):
    _fields_ = [("sink_k", ctypes.c_void_p), ("sink_v", ctypes.c_void_p), ("tail_k", ctypes.c_void_p),
                ("tail_v", ctypes.c_void_p), ("records", ctypes.c_void_p),
                ("seq_len", ctypes.c_void_p), ("batch", ctypes.c_int32), ("max_groups", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("num_blocks", ctypes.c_int32)]


def lib():
    """Load libkvarn.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m kv_cache_quantization_seal_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        cp, vp, i32, i64, f32 = ctypes.POINTER, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        sz = ctypes.c_size_t
        L.kvarn_check_config.argtypes = [cp(Config)]
        L.kvarn_record_bytes.argtypes = [i32, i32]
        L.kvarn_record_bytes.restype = sz
        L.kvarn_group_bytes.argtypes = [cp(Config)]
        L.kvarn_group_bytes.restype = sz
        L.kvarn_decode_workspace_bytes.argtypes = [cp(Config), i32, i32]
        L.kvarn_decode_workspace_bytes.restype = sz
        L.kvarn_decode_plan.argtypes = [cp(Config), i32, i32, cp(i32)]
        L.kvarn_last_error.restype = ctypes.c_char_p
        L.kvarn_status_string.argtypes = [ctypes.c_int]
        L.kvarn_status_string.restype = ctypes.c_char_p
        L.kvarn_append.argtypes = [cp(Config), cp(CacheView), vp, vp, vp]
        L.kvarn_append_seal.argtypes = [cp(Config), cp(CacheView), vp, vp, vp]
        L.kvarn_seal_group.argtypes = [cp(Config), cp(CacheView), vp, vp, i32, vp]
        L.kvarn_prefill.argtypes = [cp(Config), cp(CacheView), vp, vp, i64, cp(i32), vp]
        L.kvarn_prefill_layers.argtypes = [cp(Config), cp(CacheView), i32, cp(vp), cp(vp), i64, cp(i32), vp]
        L.kvarn_decode_attn.argtypes = [cp(Config), cp(CacheView), vp, vp, f32, vp, sz, vp]
        L.kvarn_decode_attn_noalloc.argtypes = [cp(Config), cp(CacheView), vp, vp, f32, vp]
        L.kvarn_decode_step.argtypes = [cp(Config), cp(CacheView), vp, vp, vp, vp, f32, cp(i32), vp, sz, vp]
        L.kvarn_decode_attn_partial.argtypes = [cp(Config), cp(CacheView), vp, f32, vp, sz, vp]
        L.kvarn_decode_attn_combine.argtypes = [cp(Config), cp(CacheView), vp, vp, sz, vp]
        L.kvarn_seal_tiles.argtypes = [i32, i32, i32, i32, vp, vp, i64, vp, i32, vp]
        L.kvarn_dequant_records.argtypes = [i32, i32, i32, vp, i64, vp, i32, vp]
        L.kvarn_prefill_attn.argtypes = [cp(Config), cp(CacheView), vp, i32, vp, f32, vp]
        for name in EXPORTS:
            if name not in ("kvarn_record_bytes", "kvarn_group_bytes", "kvarn_decode_workspace_bytes",
                            "kvarn_last_error", "kvarn_status_string"):
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_name(s: int) -> str:
    return {0: "KVARN_OK", -1: "KVARN_EINVAL", -2: "KVARN_EUNSUPPORTED", -3: "KVARN_ERANGE",
            -4: "KVARN_EWORKSPACE", -5: "KVARN_EHIP"}.get(s, f"status {s}")


def _check(status: int) -> None:
    if status != OK:
        raise KvarnError(status, lib().kvarn_last_error().decode())


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the KVarN library must be contiguous")
    return t.data_ptr()


def make_config(head_dim: int, num_q_heads: int, num_kv_heads: int, k_bits: int, v_bits: int,
                sinkhorn_iters: int = SINKHORN_ITERS) -> Config:
    return Config(head_dim, num_q_heads, num_kv_heads, k_bits, v_bits, GROUP, SINK, sinkhorn_iters)


def record_bytes(head_dim: int, bits: int) -> int:
    return int(lib().kvarn_record_bytes(head_dim, bits))


def group_bytes(cfg: Config) -> int:
    return int(lib().kvarn_group_bytes(ctypes.byref(cfg)))


def check_config(cfg: Config) -> int:
    return int(lib().kvarn_check_config(ctypes.byref(cfg)))


def decode_workspace_bytes(cfg: Config, batch: int, max_groups: int) -> int:
    return int(lib().kvarn_decode_workspace_bytes(ctypes.byref(cfg), batch, max_groups))


def decode_plan(cfg: Config, batch: int, max_groups: int) -> dict:
    """The decode launch plan on the current device (see kvarn_decode_plan)."""
    out = (ctypes.c_int32 * 5)()
    _check(lib().kvarn_decode_plan(ctypes.byref(cfg), batch, max_groups, out))
    return {"record_splits": out[0], "exact_splits": out[1], "groups_per_wave": out[2],
            "record_workgroups": out[3], "exact_workgroups": out[4], "max_groups": max_groups}


class KVarNCache:
    """Device-resident KVarN cache of one attention layer (torch-allocated).

    With ``num_blocks`` the records live in a pool of that many blocks (one
    block = the Hkv record pairs of one 128-token group) addressed through
    ``block_table`` (int32 [batch][max_groups], initially block
    ``b * max_groups + g`` for group g of request b; the caller may rewrite
    it).  Without it the records are one contiguous [B][Hkv][max_groups]
    array."""

    def __init__(self, cfg: Config, batch: int, max_groups: int, device="cuda", num_blocks: Optional[int] = None):
        self.cfg = cfg
        self.batch = batch
        self.max_groups = max_groups
        d, hkv = cfg.head_dim, cfg.num_kv_heads
        f16 = dict(dtype=torch.float16, device=device)
        self.sink_k = torch.zeros(batch, hkv, SINK, d, **f16)
        self.sink_v = torch.zeros(batch, hkv, SINK, d, **f16)
        self.tail_k = torch.zeros(batch, hkv, GROUP, d, **f16)
        self.tail_v = torch.zeros(batch, hkv, GROUP, d, **f16)
        self.rec_k_bytes = record_bytes(d, cfg.k_bits)
        self.group_bytes = group_bytes(cfg)
        self.num_blocks = num_blocks
        pairs = batch * hkv * max_groups if num_blocks is None else num_blocks * hkv
        self.records = torch.zeros(max(1, pairs * self.group_bytes), dtype=torch.uint8, device=device)
        self.block_table = None
        if num_blocks is not None:
            self.block_table = torch.arange(batch * max_groups, dtype=torch.int32, device=device).reshape(
                batch, max_groups)
        self.seq_len = torch.zeros(batch, dtype=torch.int32, device=device)
        ws = decode_workspace_bytes(cfg, batch, max_groups)
        self.workspace = torch.zeros(max(256, ws), dtype=torch.uint8, device=device)  # counters start at 0
        self.view = CacheView(_ptr(self.sink_k), _ptr(self.sink_v), _ptr(self.tail_k), _ptr(self.tail_v),
                              _ptr(self.records), _ptr(self.seq_len), batch, max_groups,
                              None if self.block_table is None else _ptr(self.block_table),
                              0 if num_blocks is None else int(num_blocks))

    @property
    def capacity(self) -> int:
        return SINK + GROUP * self.max_groups + GROUP - 1

    def record(self, b: int, h: int, g: int, kind: str) -> torch.Tensor:
        """Bytes of one stored record (a view)."""
        if self.block_table is None:
            pair = (b * self.cfg.num_kv_heads + h) * self.max_groups + g
        else:
            pair = int(self.block_table[b, g]) * self.cfg.num_kv_heads + h
        base = pair * self.group_bytes
        if kind == "k":
            return self.records[base:base + self.rec_k_bytes]
        return self.records[base + self.rec_k_bytes:base + self.group_bytes]

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor, stream=None) -> None:
        _check(lib().kvarn_append(ctypes.byref(self.cfg), ctypes.byref(self.view), _ptr(k_new), _ptr(v_new),
                                  _stream(stream)))

    def append_seal(self, k_new: torch.Tensor, v_new: torch.Tensor, stream=None) -> None:
        """append() then seal_group(), in one launch."""
        _check(lib().kvarn_append_seal(ctypes.byref(self.cfg), ctypes.byref(self.view), _ptr(k_new), _ptr(v_new),
                                       _stream(stream)))

    def seal_group(self, req: Optional[torch.Tensor] = None, group: Optional[torch.Tensor] = None,
                   stream=None) -> None:
        """Seal every request whose tail just filled (no lists), or the listed
        (request, group) entries (device int32 tensors of equal length)."""
        if (req is None) != (group is None):
            raise ValueError("req and group must be given together")
        n = self.batch if req is None else int(req.numel())
        if req is not None and (req.dtype != torch.int32 or group.dtype != torch.int32 or group.numel() != n):
            raise ValueError("req and group must be int32 tensors of equal length")
        _check(lib().kvarn_seal_group(ctypes.byref(self.cfg), ctypes.byref(self.view), _ptr(req), _ptr(group), n,
                                      _stream(stream)))

    def prefill(self, k: torch.Tensor, v: torch.Tensor, lengths: Sequence[int], stream=None) -> None:
        arr = (ctypes.c_int32 * self.batch)(*[int(x) for x in lengths])
        _check(lib().kvarn_prefill(ctypes.byref(self.cfg), ctypes.byref(self.view), _ptr(k), _ptr(v),
                                   int(k.shape[2]), arr, _stream(stream)))

    def decode_attn(self, q: torch.Tensor, out: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                    stream=None) -> torch.Tensor:
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        if scale is None:
            scale = self.cfg.head_dim ** -0.5
        _check(lib().kvarn_decode_attn(ctypes.byref(self.cfg), ctypes.byref(self.view), _ptr(q), _ptr(out),
                                       float(scale), _ptr(self.workspace), self.workspace.numel(),
                                       _stream(stream)))
        return out

    def decode_step(self, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                    lengths: Optional[Sequence[int]] = None, out: Optional[torch.Tensor] = None,
                    scale: Optional[float] = None, stream=None) -> torch.Tensor:
        """append_seal(k_new, v_new) then decode_attn(q) through
        kvarn_decode_step; ``lengths`` (each request's length before the
        step, as the caller counts it) lets the library fold the append into
        the decode launches when no group completes."""
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        if scale is None:
            scale = self.cfg.head_dim ** -0.5
        if lengths is not None and len(lengths) != self.batch:
            raise ValueError(f"lengths has {len(lengths)} entries for a batch of {self.batch}")
        lens = None if lengths is None else (ctypes.c_int32 * self.batch)(*[int(x) for x in lengths])
        _check(lib().kvarn_decode_step(ctypes.byref(self.cfg), ctypes.byref(self.view), _ptr(k_new), _ptr(v_new),
                                       _ptr(q), _ptr(out), float(scale), lens, _ptr(self.workspace),
                                       self.workspace.numel(), _stream(stream)))
        return out

    def decode_attn_noalloc(self, q: torch.Tensor, out: torch.Tensor, scale: Optional[float] = None,
                            stream=None) -> torch.Tensor:
        """decode_attn through kvarn_decode_attn_noalloc (the library's fixed
        scratch instead of this cache's workspace; allocates nothing)."""
        if scale is None:
            scale = self.cfg.head_dim ** -0.5
        _check(lib().kvarn_decode_attn_noalloc(ctypes.byref(self.cfg), ctypes.byref(self.view), _ptr(q), _ptr(out),
                                               float(scale), _stream(stream)))
        return out

    def prefill_attn(self, q: torch.Tensor, out: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                     stream=None) -> torch.Tensor:
        """Chunked-prefill attention of the last q.shape[1] cached positions
        (q fp16 [B][chunk][Hq][D]); returns fp32 [B][chunk][Hq][D]."""
        if out is None:
            out = torch.zeros(q.shape, dtype=torch.float32, device=q.device)
        if scale is None:
            scale = self.cfg.head_dim ** -0.5
        _check(lib().kvarn_prefill_attn(ctypes.byref(self.cfg), ctypes.byref(self.view), _ptr(q), int(q.shape[1]),
                                        _ptr(out), float(scale), _stream(stream)))
        return out

    def decode_partial(self, q: torch.Tensor, scale: Optional[float] = None, stream=None) -> None:
        if scale is None:
            scale = self.cfg.head_dim ** -0.5
        _check(lib().kvarn_decode_attn_partial(ctypes.byref(self.cfg), ctypes.byref(self.view), _ptr(q),
                                               float(scale), _ptr(self.workspace), self.workspace.numel(),
                                               _stream(stream)))

    def decode_combine(self, out: torch.Tensor, stream=None) -> torch.Tensor:
        _check(lib().kvarn_decode_attn_combine(ctypes.byref(self.cfg), ctypes.byref(self.view), _ptr(out),
                                               _ptr(self.workspace), self.workspace.numel(), _stream(stream)))
        return out


def prefill_layers(caches: Sequence["KVarNCache"], ks: Sequence[torch.Tensor], vs: Sequence[torch.Tensor],
                   lengths: Sequence[int], stream=None) -> None:
    """KVarNCache.prefill for every layer cache at once (kvarn_prefill_layers):
    caches share config, batch and max_groups; ks[i], vs[i] are layer i's
    prompt K/V [B][Hkv][src_tokens][D]."""
    n = len(caches)
    if not (len(ks) == len(vs) == n) or n == 0:
        raise ValueError("one K and one V tensor per layer cache")
    src_tokens = int(ks[0].shape[2])
    if any(int(t.shape[2]) != src_tokens for t in list(ks) + list(vs)):
        raise ValueError("every layer's K and V need the same number of tokens")
    views = (CacheView * n)(*[c.view for c in caches])
    kp = (ctypes.c_void_p * n)(*[_ptr(t) for t in ks])
    vp_ = (ctypes.c_void_p * n)(*[_ptr(t) for t in vs])
    arr = (ctypes.c_int32 * caches[0].batch)(*[int(x) for x in lengths])
    _check(lib().kvarn_prefill_layers(ctypes.byref(caches[0].cfg), views, n, kp, vp_, src_tokens, arr,
                                      _stream(stream)))


def seal_tiles(src: torch.Tensor, bits: int, kind: str, out: Optional[torch.Tensor] = None,
               dbg: Optional[torch.Tensor] = None, iters: int = SINKHORN_ITERS, stream=None) -> torch.Tensor:
    """Seal fp16 tiles [n][128][D]; returns records as uint8 [n][record_bytes]."""
    n, t, d = src.shape
    rb = record_bytes(d, bits)
    if out is None:
        out = torch.empty(n, rb, dtype=torch.uint8, device=src.device)
    _check(lib().kvarn_seal_tiles(d, bits, 0 if kind == "k" else 1, iters, _ptr(src), _ptr(out),
                                  out.stride(0), _ptr(dbg), n, _stream(stream)))
    return out


def dequant_records(recs: torch.Tensor, head_dim: int, bits: int, kind: str, out: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """Records uint8 [n][>= record_bytes] -> fp16 [n][128][D], original frame.

    Rows may be strided (a view into a cache's record slots): each row must be
    contiguous and the row stride a multiple of 16 bytes."""
    n = recs.shape[0]
    if out is None:
        out = torch.empty(n, GROUP, head_dim, dtype=torch.float16, device=recs.device)
    if recs.dim() != 2 or recs.dtype != torch.uint8 or recs.stride(1) != 1:
        raise ValueError("recs must be a uint8 [n][bytes] tensor with contiguous rows")
    _check(lib().kvarn_dequant_records(head_dim, bits, 0 if kind == "k" else 1, ctypes.c_void_p(recs.data_ptr()),
                                       recs.stride(0), _ptr(out), n, _stream(stream)))
    return out
