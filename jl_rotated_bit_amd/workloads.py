"""Seeded synthetic inputs for the QJL encode/decode workloads.

This module only draws inputs (keys, values, queries) with the shapes and
value distributions of the workloads below and rounds them to bf16 the
way a model's fp32 activations would be stored.  It holds none of the method's
arithmetic: no sketch, no projection, no estimator.  The tests and the bench
feed the same arrays to the HIP library and to the CPU oracle.

Workloads (all d = 128):

* ``small``       - 1 x 1 kv head, 8 query heads, m = 256, 4096 tokens; K, V,
                    q ~ N(0, 1) with 4 outlier channels scaled x10 (the same
                    channels in K, V and q).
* ``gqa32k``      - Llama-3.1-8B-shaped GQA decode: 32 query / 8 kv heads,
                    m = 256, batch 1, 32768 tokens; K, V = z * exp(g) with
                    g ~ N(0, 1) per (kv head, channel) drawn separately for K
                    and V, plus 1% of the (kv head, channel) pairs scaled x20.
* ``tp8``         - one GPU's share of ``gqa32k`` under 8-way tensor
                    parallelism: 1 kv head and its 4 query heads, 32768
                    tokens, the same distributions.
* ``prefill``     - encode throughput: batch 16 x 8192 tokens x 8 kv heads,
                    m = 256, keys drawn like ``gqa32k`` (scales per (kv head,
                    channel), shared by the batch).
* ``long64k``     - batch 1, 8 kv / 32 query heads, m = 512, 65536 cached
                    tokens then 64 decode steps that each append one token.
* ``mha16k``      - LLaMA-2-13B-shaped MHA decode: 40 heads, m = 256, batch 8,
                    16384 tokens; each K and V row is r * u / ||u|| with
                    u ~ N(0, I) and log10 r ~ U(-1, 1).

These stand in for the model caches and evaluation suites the pages measure
on (perplexity corpora, GSM8K, RULER on Mistral/LLaMA models), which are not
available; no item of those suites is reproduced.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

HEAD_DIM = 128
SKETCH_SEED = 42


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (round to nearest, ties to even)."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    # (u + 0x7FFF + lsb) may carry past 32 bits only for NaN payloads; the
    # generators below never produce NaN or Inf.
    return ((u.astype(np.uint64) + 0x7FFF + lsb) >> 16).astype(np.uint16)


@dataclass
class Workload:
    name: str
    B: int
    H_q: int
    H_kv: int
    d: int
    m: int
    N: int                      # tokens attended to by the decode step
    cap: int                    # rows allocated per (batch, kv head)
    keys: np.ndarray            # uint16 [B][H_kv][cap][d]
    values: np.ndarray          # uint16 [B][H_kv][cap][d]
    q: np.ndarray               # float32 [B][H_q][d]
    seed: int = SKETCH_SEED
    steps: list = field(default_factory=list)   # per appended step: (k, v, q)

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv


def _gaussian_with_outliers(rng, shape, d, n_outliers, factor):
    x = rng.standard_normal(shape, dtype=np.float32)
    ch = rng.choice(d, size=n_outliers, replace=False)
    x[..., ch] *= np.float32(factor)
    return x, ch


def _channel_scaled(rng, B, H, n, d, sigma=1.0, outlier_frac=0.01, factor=20.0,
                    chunk_tokens=2048):
    """z * exp(g_{h,c}) with 1% of (head, channel) pairs scaled x factor, as bf16."""
    g = rng.standard_normal((H, d)).astype(np.float32) * np.float32(sigma)
    scale = np.exp(g)
    n_out = int(round(outlier_frac * H * d))
    flat = rng.choice(H * d, size=n_out, replace=False)
    scale.reshape(-1)[flat] *= np.float32(factor)
    out = np.empty((B, H, n, d), dtype=np.uint16)
    for b in range(B):
        for t0 in range(0, n, chunk_tokens):
            t1 = min(n, t0 + chunk_tokens)
            z = rng.standard_normal((H, t1 - t0, d), dtype=np.float32)
            out[b, :, t0:t1] = round_to_bf16_bits(z * scale[:, None, :])
    return out, scale


def _log_uniform_norm_rows(rng, B, H, n, d, chunk_tokens=2048):
    out = np.empty((B, H, n, d), dtype=np.uint16)
    for b in range(B):
        for t0 in range(0, n, chunk_tokens):
            t1 = min(n, t0 + chunk_tokens)
            u = rng.standard_normal((H, t1 - t0, d), dtype=np.float32)
            u /= np.linalg.norm(u, axis=-1, keepdims=True)
            r = np.power(np.float32(10.0), rng.uniform(-1.0, 1.0, (H, t1 - t0, 1)).astype(np.float32))
            out[b, :, t0:t1] = round_to_bf16_bits(u * r)
    return out


def small(N: int = 4096, H_q: int = 8, data_seed: int = 1001) -> Workload:
    rng = np.random.default_rng(data_seed)
    d = HEAD_DIM
    ch = rng.choice(d, size=4, replace=False)
    K = rng.standard_normal((1, 1, N, d), dtype=np.float32)
    V = rng.standard_normal((1, 1, N, d), dtype=np.float32)
    q = rng.standard_normal((1, H_q, d), dtype=np.float32)
    for x in (K, V, q):
        x[..., ch] *= np.float32(10.0)
    return Workload("small", 1, H_q, 1, d, 256, N, N, round_to_bf16_bits(K),
                    round_to_bf16_bits(V), q)


def gqa32k(N: int = 32768, B: int = 1, H_q: int = 32, H_kv: int = 8, m: int = 256,
           data_seed: int = 1002, cap: int | None = None) -> Workload:
    rng = np.random.default_rng(data_seed)
    d = HEAD_DIM
    cap = N if cap is None else cap
    K, _ = _channel_scaled(rng, B, H_kv, cap, d)
    V, _ = _channel_scaled(rng, B, H_kv, cap, d)
    q = rng.standard_normal((B, H_q, d), dtype=np.float32)
    return Workload("gqa32k", B, H_q, H_kv, d, m, N, cap, K, V, q)


def prefill(B: int = 16, n: int = 8192, H_kv: int = 8, m: int = 256,
            data_seed: int = 1003) -> Workload:
    """Keys only (values/queries are empty): the encode-throughput workload."""
    rng = np.random.default_rng(data_seed)
    d = HEAD_DIM
    K, _ = _channel_scaled(rng, B, H_kv, n, d)
    empty = np.zeros((B, H_kv, 0, d), dtype=np.uint16)
    return Workload("prefill", B, H_kv, H_kv, d, m, n, n, K, empty,
                    np.zeros((B, H_kv, d), dtype=np.float32))


def long64k(N0: int = 65536, steps: int = 64, H_q: int = 32, H_kv: int = 8,
            data_seed: int = 1004) -> Workload:
    rng = np.random.default_rng(data_seed)
    d = HEAD_DIM
    cap = N0 + steps
    K, _ = _channel_scaled(rng, 1, H_kv, cap, d)
    V, _ = _channel_scaled(rng, 1, H_kv, cap, d)
    q0 = rng.standard_normal((1, H_q, d), dtype=np.float32)
    per_step = []
    for s in range(steps):
        qs = rng.standard_normal((1, H_q, d), dtype=np.float32)
        # the appended (k, v) of step s live in row N0 + s of K and V
        per_step.append(qs)
    return Workload("long64k", 1, H_q, H_kv, d, 512, N0, cap, K, V, q0, steps=per_step)


def mha16k(N: int = 16384, B: int = 8, H: int = 40, data_seed: int = 1005) -> Workload:
    rng = np.random.default_rng(data_seed)
    d = HEAD_DIM
    K = _log_uniform_norm_rows(rng, B, H, N, d)
    V = _log_uniform_norm_rows(rng, B, H, N, d)
    q = rng.standard_normal((B, H, d), dtype=np.float32)
    return Workload("mha16k", B, H, H, d, 256, N, N, K, V, q)


def gaussian_keys(rng: np.random.Generator, rows: int, d: int = HEAD_DIM,
                  scale: float = 1.0) -> np.ndarray:
    """Plain N(0, scale^2) keys as bf16 bits, [rows][d] (for edge-case tests)."""
    return round_to_bf16_bits(rng.standard_normal((rows, d), dtype=np.float32) * np.float32(scale))


def tp8(data_seed: int = 1006) -> Workload:
    """One GPU's share of ``gqa32k`` under 8-way tensor parallelism: 1 kv
    head and its 4 query heads, 32768 tokens, the same distributions."""
    w = gqa32k(H_q=4, H_kv=1, data_seed=data_seed)
    w.name = "tp8"
    return w


WORKLOADS = {
    "small": small,
    "tp8": tp8,
    "gqa32k": gqa32k,
    "prefill": prefill,
    "long64k": long64k,
    "mha16k": mha16k,
}
