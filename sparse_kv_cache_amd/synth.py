"""Seeded synthetic inputs for the Fathom plane-prefix scan.

This module only draws random numbers; it holds none of the method's
arithmetic (no quantization, no allocation, no scoring).  Both the HIP path
and the CPU oracle consume what it returns, so a parity test feeds the same
bytes to both sides.

Workloads stand in for the pages' Qwen3-8B long-context decode setting
("Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV Caches",
abstract, fourth sentence; "Fathom Makes KV-Cache Scans Query-Adaptive for
Long-Context Decoding", first findings bullet): keys of one layer of a
8-KV-head, 128-channel, GQA-4 model.  Neither the model's weights nor the
pages' task suites are available, so keys are drawn per KV head as

    sigma_c ~ LogNormal(0, 0.5)            (channel scales, float32)
    sigma_c *= 8 for 4 distinct channels   (outlier channels)
    K[i, c] = N(0, 1) * sigma_c            (float32)

and queries as N(0, 1) float32.  Generator: NumPy PCG64 via
``np.random.default_rng(seed)``; heads are drawn in order, then the queries.
Value rows (for the attention over the selected keys) are N(0, 1) float32,
drawn per head from a separate stream.
"""

from __future__ import annotations

import dataclasses
from typing import Iterator, Sequence

import numpy as np

D_DEFAULT = 128
OUTLIER_CHANNELS = 4
OUTLIER_SCALE = np.float32(8.0)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one synthetic decode-step workload (one layer)."""

    name: str
    num_kv_heads: int      # KV heads, sessions x heads flattened
    n: int                 # keys per KV head
    group: int             # query heads per KV head (GQA group)
    budgets: Sequence[int]  # bit budgets B (bits per key per query)
    k: int                 # top-k
    seed: int
    d: int = D_DEFAULT

    @property
    def num_q(self) -> int:
        return self.num_kv_heads * self.group


# The five workloads: tiny, single-head long, the 1M-token Qwen3-8B-shaped
# decode step, a 16-session batch and the host-resident store (same store as
# the 1M-token step, placed in pinned host memory).
WORKLOADS = {
    "tiny": Workload("tiny", 1, 4096, 1, (92,), 64, 0),
    "single_head_long": Workload("single_head_long", 1, 131072, 4, (68, 92, 136, 512), 256, 1),
    "qwen3_8b_1m": Workload("qwen3_8b_1m", 8, 1 << 20, 4, (92,), 2048, 2),
    "multi_session": Workload("multi_session", 16 * 8, 131072, 4, (68, 92, 136), 1024, 3),
    "host_resident": Workload("host_resident", 8, 1 << 20, 4, (68, 92, 136), 2048, 2),
}


def head_keys(rng: np.random.Generator, n: int, d: int = D_DEFAULT) -> np.ndarray:
    """Draw one KV head's keys, float32 [n, d] (see module docstring)."""
    sigma = rng.lognormal(mean=0.0, sigma=0.5, size=d).astype(np.float32)
    outl = rng.choice(d, OUTLIER_CHANNELS, replace=False)
    sigma[outl] = sigma[outl] * OUTLIER_SCALE
    keys = rng.standard_normal((n, d), dtype=np.float32)
    keys *= sigma[None, :]
    return keys


def iter_heads(seed: int, num_kv_heads: int, n: int, d: int = D_DEFAULT) -> Iterator[np.ndarray]:
    """Yield the keys of each KV head in order, then nothing; see ``queries``."""
    rng = np.random.default_rng(seed)
    for _ in range(num_kv_heads):
        yield head_keys(rng, n, d)


def make_inputs(seed: int, num_kv_heads: int, n: int, num_q: int, d: int = D_DEFAULT):
    """Return (keys [H, n, d] float32, q [num_q, d] float32) for small workloads.

    Large workloads should stream heads with ``stream_inputs`` instead.
    """
    rng = np.random.default_rng(seed)
    keys = np.empty((num_kv_heads, n, d), dtype=np.float32)
    for h in range(num_kv_heads):
        keys[h] = head_keys(rng, n, d)
    q = rng.standard_normal((num_q, d), dtype=np.float32)
    return keys, q


def stream_inputs(seed: int, num_kv_heads: int, n: int, num_q: int, d: int = D_DEFAULT):
    """Generator form of ``make_inputs``: yields ("head", h, keys) per head,
    then ("queries", q).  Same bytes as ``make_inputs`` for the same arguments."""
    rng = np.random.default_rng(seed)
    for h in range(num_kv_heads):
        yield "head", h, head_keys(rng, n, d)
    yield "queries", rng.standard_normal((num_q, d), dtype=np.float32)


def head_values(seed: int, h: int, n: int, d: int = D_DEFAULT) -> np.ndarray:
    """Value rows of KV head h for the attention step, float32 [n, d] ~ N(0, 1),
    from a stream of their own (seed, h), so the key and query draws are
    unchanged."""
    return np.random.default_rng([seed, 1 << 20, h]).standard_normal((n, d), dtype=np.float32)


def forced_tie_keys(seed: int, n: int, d: int = D_DEFAULT) -> np.ndarray:
    """Keys with degenerate structure for edge-case tests: one constant
    channel, one pair of duplicated channels, and one channel holding only
    two distinct values."""
    rng = np.random.default_rng(seed)
    keys = head_keys(rng, n, d)
    keys[:, 0] = np.float32(0.75)                       # constant channel
    keys[:, 2] = keys[:, 1]                              # duplicated channel
    keys[:, 3] = np.where(rng.random(n) < 0.5, np.float32(-1.0), np.float32(1.0))
    return keys


def plant_aligned_keys(seed: int, keys: np.ndarray, q: np.ndarray, per_query: int, logit: float) -> np.ndarray:
    """Give attention a peak to find: for each query row g of q [G, d],
    overwrite `per_query` random rows of one head's keys [n, d] with keys
    along that query's direction, scaled so that q_g . k / sqrt(d) = logit,
    plus N(0, 0.1) noise (in place).  Distinct rows per query; returns them,
    int64 [G, per_query].  Only synthetic-input construction: the stand-in for
    the peaked attention of a trained model."""
    rng = np.random.default_rng([seed, 1 << 21])
    n, d = keys.shape
    rows = rng.choice(n, (q.shape[0], per_query), replace=False)
    for g in range(q.shape[0]):
        qg = q[g].astype(np.float64)
        direction = qg * (logit * np.sqrt(d) / float(qg @ qg))
        noise = 0.1 * rng.standard_normal((per_query, d))
        keys[rows[g]] = (direction[None, :] + noise).astype(np.float32)
    return rows
