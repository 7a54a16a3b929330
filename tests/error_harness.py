"""Pseudo-decode error-accumulation harness (test infrastructure: runs the CPU
oracle; nothing in the product path imports it).

The pages' claim is about mechanism: quantization error of a KV cache
compounds over long decoding, and per-token scales are what make it grow,
which KVarN's variance normalization counters (KVarN summary page, "What it
is", "Practical takeaway": evaluate by pseudo-decoding, re-quantizing every
block and forcing later tokens to read it; "KVarN KV Cache: Implementation
and Benchmarks", §1 "Where KVarN Comes From").  Without trained weights or
datasets this harness measures it on synthetic caches, two ways:

* Open loop.  A synthetic post-RoPE stream (the inputs' recipe: outlier
  channels in K, lognormal token norms) is decoded step by step.  At step p
  the query attends over positions [0, p]: the 128-token sink and the tail
  exact, every complete 128-token group read back through the method under
  test, as the cache would hold it.  Metrics, per step and query head: the
  total variation distance between the attention weights over the cached
  positions and the exact cache's (only the keys matter), and the L2 error
  of the attention output against the exact cache's, in units of the RMS
  norm of the cached value rows (an attention output over random values is
  an average that is much shorter than a value row, so an error relative to
  the output itself says little).
* Closed loop.  A toy recurrent decoder with fixed random projections feeds
  each step's attention output back into the next token's hidden state, from
  which that token's q, k and v are made (K with the recipe's outlier
  channels and lognormal token norms, then RoPE).  The error of step t thus
  perturbs every later token, which is the accumulation the pages describe.
  Metric: relative L2 distance of the hidden state from the exact-cache
  trajectory, per step.

Methods (each a fake-quantizer of a complete group, K and V with their own
kind): 'kvarn' (rotation + 16 Sinkhorn iterations + RTN, the record decoded
back), 'rotation_only' (the same with 0 iterations), 'rtn_channel'
(per-channel RTN, no rotation), 'rtn_token' (per-token RTN, no rotation).

Run ``python -m tests.error_harness`` for the table quoted in the design
notes (a few minutes on one core).
"""
from __future__ import annotations

import sys

import numpy as np

from kv_cache_quantization_seal_amd import synth
from oracle import kvarn_oracle as O

METHODS = ("kvarn", "rotation_only", "rtn_channel", "rtn_token")
SINK = 128
GROUP = 128


def fake_quant(x: np.ndarray, bits: int, kind: str, method: str) -> np.ndarray:
    """Complete group x (fp16 [128][D]) as `method` stores and reads it back."""
    if method == "kvarn":
        return O.fake_quant_kvarn(x, bits, kind, 16)
    if method == "rotation_only":
        return O.fake_quant_kvarn(x, bits, kind, 0)
    if method == "rtn_channel":
        return O.fake_quant_rtn(x, bits, "channel")
    if method == "rtn_token":
        return O.fake_quant_rtn(x, bits, "token")
    if method == "exact":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(method)


def tv_distance(p: np.ndarray, ref: np.ndarray) -> float:
    """Total variation distance 1/2 sum |p - ref| of two distributions."""
    return 0.5 * float(np.abs(np.asarray(p, np.float64) - np.asarray(ref, np.float64)).sum())


def weights(q: np.ndarray, k_all: np.ndarray) -> np.ndarray:
    """Softmax attention weights of one query over the rows of k_all (scale
    1/sqrt(D)), float64."""
    logits = np.asarray(k_all, np.float64) @ np.asarray(q, np.float64) / np.sqrt(k_all.shape[1])
    e = np.exp(logits - logits.max())
    return e / e.sum()


def rel_err(a: np.ndarray, ref: np.ndarray) -> float:
    """||a - ref||_2 / ||ref||_2 over the last axis (0 when both are 0)."""
    num = float(np.linalg.norm(np.asarray(a, np.float64) - np.asarray(ref, np.float64)))
    den = float(np.linalg.norm(np.asarray(ref, np.float64)))
    return 0.0 if num == 0.0 else num / den


class ReadCache:
    """What attention reads for one (request, KV head): float64 K and V of
    every cached position, complete groups replaced by their fake-quantized
    version when they seal (append -> seal if due -> attend)."""

    def __init__(self, d: int, cap: int, kb: int, vb: int, method: str):
        self.k = np.zeros((cap, d))
        self.v = np.zeros((cap, d))
        self.k16 = np.zeros((cap, d), np.float16)
        self.v16 = np.zeros((cap, d), np.float16)
        self.n = 0
        self.kb, self.vb, self.method = kb, vb, method

    def append(self, k16: np.ndarray, v16: np.ndarray) -> None:
        p = self.n
        self.k16[p], self.v16[p] = k16, v16
        self.k[p], self.v[p] = k16.astype(np.float64), v16.astype(np.float64)
        self.n += 1
        if self.n >= SINK + GROUP and (self.n - SINK) % GROUP == 0:
            lo = self.n - GROUP
            self.k[lo:self.n] = fake_quant(self.k16[lo:self.n], self.kb, "k", self.method)
            self.v[lo:self.n] = fake_quant(self.v16[lo:self.n], self.vb, "v", self.method)

    def attend(self, q: np.ndarray) -> np.ndarray:
        return O.attention(q, self.k[:self.n], self.v[:self.n])

    def weights(self, q: np.ndarray) -> np.ndarray:
        return weights(q, self.k[:self.n])

    def value_rms(self) -> float:
        """RMS L2 norm of the exact (fp16) value rows cached so far."""
        v = self.v16[:self.n].astype(np.float64)
        return float(np.sqrt(np.mean(np.sum(v * v, axis=1))))


def open_loop(seed: int, bits=(2, 2), d: int = 128, gq: int = 4, prompt: int = 384, steps: int = 1024,
              methods=METHODS):
    """Per-step errors {method: (tv [steps][gq], out [steps][gq])}: attention
    weight total variation and output error in value-RMS units."""
    wl = synth.Workload("harness_open", 200 + seed, 1, gq, 1, d, prompt, 0, bits[0], bits[1], steps)
    k, v = synth.kv_stream(wl, 0, 0, prompt + steps)
    qs = synth.queries(wl, 0, steps)
    caches = {m: ReadCache(d, prompt + steps, bits[0], bits[1], m) for m in ("exact",) + tuple(methods)}
    for c in caches.values():
        for p in range(prompt):
            c.append(k[p], v[p])
    tv = {m: np.zeros((steps, gq)) for m in methods}
    out = {m: np.zeros((steps, gq)) for m in methods}
    for s in range(steps):
        p = prompt + s
        for c in caches.values():
            c.append(k[p], v[p])
        vrms = caches["exact"].value_rms()
        for h in range(gq):
            w_ref = caches["exact"].weights(qs[s, h])
            o_ref = w_ref @ caches["exact"].v[:p + 1]
            for m in methods:
                w = caches[m].weights(qs[s, h])
                tv[m][s, h] = tv_distance(w, w_ref)
                out[m][s, h] = float(np.linalg.norm(w @ caches[m].v[:p + 1] - o_ref)) / vrms
    return {m: (tv[m], out[m]) for m in methods}


class ToyDecoder:
    """Fixed random projections of a one-KV-head attention layer with its
    output fed back: h_{t+1} = unit-RMS(alpha W_o o_t + beta xi_t), where xi_t
    is a fresh N(0, 1) input (the same for every method).  Token t's key is
    RoPE((W_k h_t) with n_out outlier channels x m_out, times a lognormal(0,
    0.5) token norm), its value W_v h_t times its own lognormal norm, its
    queries RoPE(W_q h_t) per query head."""

    def __init__(self, seed: int, d: int = 128, gq: int = 4, alpha: float = 0.25, beta: float = 1.0,
                 n_out: int = 4, m_out: float = 10.0):
        rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(300,)))
        self.d, self.gq, self.alpha, self.beta = d, gq, alpha, beta
        self.wq = rng.standard_normal((gq, d, d)) / np.sqrt(d)
        self.wk = rng.standard_normal((d, d)) / np.sqrt(d)
        self.wv = rng.standard_normal((d, d)) / np.sqrt(d)
        self.wo = rng.standard_normal((d, gq * d)) / np.sqrt(gq * d)
        self.kscale = np.ones(d)
        self.kscale[rng.choice(d, n_out, replace=False)] = m_out
        self.rng_seed = seed

    @staticmethod
    def unit_rms(x: np.ndarray) -> np.ndarray:
        return x / np.sqrt(np.mean(x * x))

    def token(self, h: np.ndarray, pos: int, knorm: float, vnorm: float):
        k = synth.rope_neox((self.wk @ h * self.kscale * knorm)[None], np.array([pos]))[0]
        v = self.wv @ h * vnorm
        q = synth.rope_neox(np.einsum("gij,j->gi", self.wq, h), np.full(self.gq, pos))
        return k.astype(np.float16), v.astype(np.float16), q.astype(np.float16)

    def run(self, method: str, bits=(2, 2), prompt: int = 384, steps: int = 1024):
        """Hidden states [steps][d] and attention outputs [steps][gq][d]."""
        d, gq = self.d, self.gq
        rng = np.random.default_rng(np.random.SeedSequence(self.rng_seed, spawn_key=(301,)))
        n = prompt + steps
        xi = rng.standard_normal((n + 1, d))
        knorm = rng.lognormal(0.0, synth.TOKEN_SIGMA, n + 1)
        vnorm = rng.lognormal(0.0, synth.TOKEN_SIGMA, n + 1)
        cache = ReadCache(d, n + 1, bits[0], bits[1], method)
        h = self.unit_rms(xi[0])
        hs, outs = np.zeros((steps, d)), np.zeros((steps, gq, d))
        for t in range(n):
            k, v, q = self.token(h, t, knorm[t], vnorm[t])
            cache.append(k, v)
            if t < prompt:   # the prompt: hidden states from the inputs alone
                h = self.unit_rms(xi[t + 1])
                continue
            o = np.stack([cache.attend(q[g]) for g in range(gq)])
            s = t - prompt
            hs[s], outs[s] = h, o
            h = self.unit_rms(self.alpha * (self.wo @ o.reshape(-1)) + self.beta * xi[t + 1])
        return hs, outs


def closed_loop(seed: int, bits=(2, 2), prompt: int = 384, steps: int = 1024, methods=METHODS):
    """Per-step relative hidden-state distance from the exact trajectory."""
    dec = ToyDecoder(seed)
    ref_h, _ = dec.run("exact", bits, prompt, steps)
    out = {}
    for m in methods:
        hs, _ = dec.run(m, bits, prompt, steps)
        out[m] = np.array([rel_err(hs[s], ref_h[s]) for s in range(steps)])
    return out


def table(seeds=(0, 1, 2, 3), bits=(2, 2), steps: int = 1024) -> str:
    rows = []
    ol = [open_loop(s, bits, steps=steps) for s in seeds]
    cl = [closed_loop(s, bits, steps=steps) for s in seeds]
    marks = [m for m in (64, 256, 512, 1024) if m <= steps]
    rows.append("| Method | open loop: attention-weight TV, mean | open loop: output error / value RMS, mean | p95 | "
                + " | ".join(f"closed loop: hidden drift @ step {m}" for m in marks) + " |")
    rows.append("|" + "---|" * (4 + len(marks)))
    for m in METHODS:
        tv = np.concatenate([o[m][0].reshape(-1) for o in ol])
        oe = np.concatenate([o[m][1].reshape(-1) for o in ol])
        drift = [float(np.median([c[m][k - 1] for c in cl])) for k in marks]
        rows.append(f"| {m} | {tv.mean():.4f} | {oe.mean():.4f} | {np.percentile(oe, 95):.4f} | "
                    + " | ".join(f"{x:.4f}" for x in drift) + " |")
    return "\n".join(rows)


if __name__ == "__main__":
    b = tuple(int(x) for x in sys.argv[1].split(",")) if len(sys.argv) > 1 else (2, 2)
    print(f"K/V bits {b}; seeds 0-3; prompt 384 tokens (sink + 2 groups); 1024 pseudo-decode steps "
          f"(8 more groups); 4 query heads, D 128")
    print(table(bits=b))
