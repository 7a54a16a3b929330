"""Seeded synthetic K/V/q generators for the KVarN hot path.

This module holds input generation only (random draws and the model-side RoPE
that produces post-RoPE keys); none of KVarN's own arithmetic lives here.  Both
the CPU oracle tests and the GPU benchmarks draw their inputs from it.

The value structure follows what the pages blame for quantization error:

* outlier channels in K that a channel rotation spreads
  (KVarN KV Cache: Implementation and Benchmarks, §1 "Where KVarN Comes From");
* per-token norm disparity that corrupts per-token scales (same section), drawn
  here as a lognormal per-token multiplier on K and V.

Recipe for one (request b, KV head h) stream of L tokens, drawn in this order
from ``default_rng(SeedSequence(seed, spawn_key=(workload_id, 0, b, h)))``:

1. K_pre ~ N(0, 1), shape [L][D];
2. ``n_out`` outlier channels chosen without replacement, multiplied by ``m_out``;
3. a per-token multiplier ~ lognormal(0, 0.5) applied to K;
4. NeoX rotate-half RoPE with theta = 1e6 at positions 0..L-1, then fp16 (RNE);
5. V ~ N(0, 1) times its own lognormal(0, 0.5) per-token multiplier, fp16.

Queries of request b come from their own stream
``SeedSequence(seed, spawn_key=(workload_id, 1, b))``: for each decode step,
N(0, 1) per query head, RoPE at the position of the newest token, fp16.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Tuple

import numpy as np

ROPE_THETA = 1.0e6
TOKEN_SIGMA = 0.5


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one synthetic KVarN workload."""
    name: str
    wid: int             # stream id used in the seed spawn keys
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    context: int         # tokens in the cache of request 0 before decoding
    stagger: int         # request b starts with context + stagger * b tokens
    k_bits: int
    v_bits: int
    steps: int           # decode steps (append -> seal if due -> attend)
    n_out: int = 4       # outlier channels in K
    m_out: float = 10.0  # outlier multiplier
    seed: int = 0

    def start_len(self, b: int) -> int:
        return self.context + self.stagger * b

    def max_len(self) -> int:
        return self.start_len(self.batch - 1) + self.steps

    def max_groups(self) -> int:
        """Record slots per request that hold every group the workload seals:
        capacity 128 + 128 max_groups + 127 >= max_len()."""
        return max(1, (self.max_len() - 128) // 128 + 1)


# Shapes follow the model families the pages evaluate on
# (KVarN summary page, "Key result": Qwen3-4B, Llama-3.1-8B, Phi-4-14B).
WORKLOADS: Dict[str, Workload] = {
    # One KV head, 512 tokens = 128-token sink + 3 sealed groups, one query.
    "tiny_parity": Workload("tiny_parity", 0, 1, 1, 1, 128, 512, 0, 2, 2, 0),
    # Llama-3.1-8B attention shape: 32 q / 8 kv heads, 32k context, 256 steps.
    "llama31_8b_32k": Workload("llama31_8b_32k", 1, 1, 32, 8, 128, 32768, 0, 2, 2, 256),
    # The same shape at two of the K/V width presets (3-2 and 6-5 bits).
    "llama31_8b_32k_k3v2": Workload("llama31_8b_32k_k3v2", 6, 1, 32, 8, 128, 32768, 0, 3, 2, 256),
    "llama31_8b_32k_k6v5": Workload("llama31_8b_32k_k6v5", 7, 1, 32, 8, 128, 32768, 0, 6, 5, 256),
    # Qwen3-4B attention shape, batch 16 at 16k, staggered so seals interleave.
    "qwen3_4b_16k_b16": Workload("qwen3_4b_16k_b16", 2, 16, 32, 8, 128, 16384, 8, 2, 2, 256),
    # The same with every request at 16k: all 16 requests seal on the same step.
    "qwen3_4b_16k_b16_aligned": Workload("qwen3_4b_16k_b16_aligned", 5, 16, 32, 8, 128, 16384, 0, 2, 2, 256),
    # Phi-4-14B attention shape, 4-bit K and V, batch 8 at 32k, tails 0..112.
    "phi4_14b_32k_b8": Workload("phi4_14b_32k_b8", 3, 8, 40, 10, 128, 32768, 16, 4, 4, 0),
    # Head dim 256, 64k context, K 4-bit / V 2-bit, 2% outlier channels x20.
    "longctx_d256_64k_b4": Workload("longctx_d256_64k_b4", 4, 4, 32, 16, 256, 65536, 32, 4, 2, 128,
                                    n_out=5, m_out=20.0),
}


def rope_neox(x: np.ndarray, positions: np.ndarray, theta: float = ROPE_THETA) -> np.ndarray:
    """Rotate-half RoPE in float64: x [..., L, D] with positions [L]."""
    d = x.shape[-1]
    half = d // 2
    inv_freq = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = positions.astype(np.float64)[:, None] * inv_freq[None, :]
    cos, sin = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def _kv_rng(wl: Workload, b: int, h: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(wl.seed, spawn_key=(wl.wid, 0, b, h)))


def _q_rng(wl: Workload, b: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(wl.seed, spawn_key=(wl.wid, 1, b)))


def kv_stream(wl: Workload, b: int, h: int, length: int | None = None) -> Tuple[np.ndarray, np.ndarray]:
    """Post-RoPE fp16 K and V of request b, KV head h: each [length][D].

    ``length`` defaults to the longest the workload ever reaches for request b
    (its start length plus every decode step), so the tokens a decode step
    appends are the continuation of the prefilled ones.
    """
    if length is None:
        length = wl.start_len(b) + wl.steps
    rng = _kv_rng(wl, b, h)
    d = wl.head_dim
    k = rng.standard_normal((length, d))
    out = rng.choice(d, wl.n_out, replace=False)
    k[:, out] *= wl.m_out
    k *= rng.lognormal(0.0, TOKEN_SIGMA, size=(length, 1))
    k = rope_neox(k, np.arange(length))
    v = rng.standard_normal((length, d))
    v *= rng.lognormal(0.0, TOKEN_SIGMA, size=(length, 1))
    return k.astype(np.float16), v.astype(np.float16)


def queries(wl: Workload, b: int, n_queries: int | None = None) -> np.ndarray:
    """fp16 decode queries of request b: [n_queries][Hq][D].

    Query i is the one issued after the cache of request b holds
    ``start_len(b) + i + 1`` tokens when the workload decodes (or
    ``start_len(b)`` tokens, i = 0, for attend-only workloads), so it carries
    RoPE at the newest token's position.
    """
    if n_queries is None:
        n_queries = max(1, wl.steps)
    rng = _q_rng(wl, b)
    q = rng.standard_normal((n_queries, wl.num_q_heads, wl.head_dim))
    newest = wl.start_len(b) - 1 + (np.arange(n_queries) + (1 if wl.steps else 0))
    out = np.empty_like(q)
    for i in range(n_queries):
        out[i] = rope_neox(q[i], np.full(wl.num_q_heads, newest[i]))
    return out.astype(np.float16)


def gaussian_tile(seed: int, tokens: int, dim: int, n_out: int = 4, m_out: float = 10.0) -> np.ndarray:
    """One fp16 [tokens][dim] tile with the same value recipe (no RoPE)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((tokens, dim))
    if n_out:
        x[:, rng.choice(dim, n_out, replace=False)] *= m_out
    x *= rng.lognormal(0.0, TOKEN_SIGMA, size=(tokens, 1))
    return x.astype(np.float16)


def kv_streams_device(wl: Workload, length: int, device, pairs_from_host=()):
    """fp16 K and V of every (request, KV head) at once: [B][Hkv][length][D].

    Same recipe as ``kv_stream`` (outlier channels, lognormal token norms,
    NeoX RoPE with theta 1e6), drawn on the device from a torch generator
    seeded per (workload, request, head), so a full-size cache is built in
    seconds.  These values are not the host stream's; the pairs listed in
    ``pairs_from_host`` are filled from ``kv_stream`` instead, so the oracle
    can be run on exactly those.
    """
    import torch
    B, H, d = wl.batch, wl.num_kv_heads, wl.head_dim
    K = torch.empty((B, H, length, d), dtype=torch.float16, device=device)
    V = torch.empty_like(K)
    half = d // 2
    inv_freq = ROPE_THETA ** (-torch.arange(half, dtype=torch.float64, device=device) * 2.0 / d)
    ang = torch.arange(length, dtype=torch.float64, device=device)[:, None] * inv_freq[None, :]
    cos, sin = torch.cos(ang).float(), torch.sin(ang).float()
    gen = torch.Generator(device=device)
    for b in range(B):
        for h in range(H):
            gen.manual_seed(((wl.seed * 1000003 + wl.wid) * 1000003 + b) * 1000003 + h)
            k = torch.randn((length, d), generator=gen, device=device)
            out = torch.randperm(d, generator=gen, device=device)[:wl.n_out]
            k[:, out] *= wl.m_out
            k *= torch.exp(TOKEN_SIGMA * torch.randn((length, 1), generator=gen, device=device))
            k1, k2 = k[:, :half], k[:, half:]
            K[b, h] = torch.cat([k1 * cos - k2 * sin, k2 * cos + k1 * sin], dim=-1).half()
            v = torch.randn((length, d), generator=gen, device=device)
            v *= torch.exp(TOKEN_SIGMA * torch.randn((length, 1), generator=gen, device=device))
            V[b, h] = v.half()
    for b, h in pairs_from_host:
        k, v = kv_stream(wl, b, h, length)
        K[b, h] = torch.from_numpy(k).to(device)
        V[b, h] = torch.from_numpy(v).to(device)
    return K, V
