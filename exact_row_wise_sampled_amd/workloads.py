"""Seeded synthetic score rows for the five evaluation workloads.

This module only draws random inputs; it holds none of the selector's
arithmetic and is shared by the tests, the benchmark and the CPU oracle runs.

Score model (the indexer of "Sample-Guided Exact Top-K Selection for
Long-Context Sparse Attention", Sec. 2.1, Eq. 1): a row score is a weighted sum
over h heads of ReLU(q.k). The pages' real captures are not available, so the
dot products q.k are stand-ins drawn i.i.d. N(0, 1), the head weights w are
drawn U(0, 1) once per row, and the sum is accumulated in float32 from 0 with
one rounded multiply and one rounded add per head (no fused multiply-add).

Every row owns its own PCG64 stream, spawned from SeedSequence(seed), so rows
can be generated in parallel and any single row can be regenerated alone.
Columns at or beyond a row's valid length are filled with garbage bit patterns
(a quarter forced to +inf and a quarter to quiet NaN) so that a selector that
reads past the valid prefix is caught.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

HEADS = 8
POS_INF_BITS = np.uint32(0x7F800000)
NEG_INF_BITS = np.uint32(0xFF800000)
QNAN_BITS = np.uint32(0x7FC00000)


@dataclass
class Workload:
    name: str
    x: np.ndarray          # [M, N] float32, C-contiguous
    ke: np.ndarray         # [M] int32 valid lengths
    k: int                 # requested rank
    seed: int

    @property
    def m(self) -> int:
        return int(self.x.shape[0])

    @property
    def n(self) -> int:
        return int(self.x.shape[1])

    def score_bytes(self) -> int:
        """Bytes of valid scores: sum over rows of 4 * min(max(ke, 0), N)."""
        return int(4 * np.clip(self.ke.astype(np.int64), 0, self.n).sum())


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _row_streams(seed: int, m: int):
    ss = np.random.SeedSequence(seed)
    kids = ss.spawn(m + 1)
    return [np.random.Generator(np.random.PCG64(k)) for k in kids[:m]], \
        np.random.Generator(np.random.PCG64(kids[m]))


def relu_heads(rng: np.random.Generator, length: int, out: np.ndarray) -> None:
    """out[:length] = sum_h w_h * relu(g_h), float32, accumulated head by head."""
    w = rng.random(HEADS, dtype=np.float32)
    acc = out[:length]
    acc[:] = 0.0
    g = np.empty(length, dtype=np.float32)
    t = np.empty(length, dtype=np.float32)
    for h in range(HEADS):
        rng.standard_normal(out=g, dtype=np.float32)
        np.maximum(g, np.float32(0.0), out=g)
        np.multiply(g, w[h], out=t)
        np.add(acc, t, out=acc)


def fill_padding(rng: np.random.Generator, row: np.ndarray, start: int) -> None:
    """Garbage in row[start:]: random bit patterns, 25% +inf, 25% qNaN."""
    n = row.shape[0] - start
    if n <= 0:
        return
    bits = rng.integers(0, 2**32, size=n, dtype=np.uint32)
    sel = rng.random(n)
    bits[sel < 0.25] = POS_INF_BITS
    bits[(sel >= 0.25) & (sel < 0.5)] = QNAN_BITS
    row[start:] = bits.view(np.float32)


def _parallel_rows(m: int, fn) -> None:
    if m <= 2:
        for r in range(m):
            fn(r)
        return
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fn, range(m)))


# ---------------------------------------------------------------- generators

def tiny(seed: int = 1) -> Workload:
    """4 rows of width 8192, ke = [8192, 6000, 3000, 1024], K = 256, N(0,1)."""
    m, n, k = 4, 8192, 256
    ke = np.array([8192, 6000, 3000, 1024], dtype=np.int32)
    x = np.empty((m, n), dtype=np.float32)
    rngs, _ = _row_streams(seed, m)
    for r in range(m):
        x[r, :ke[r]] = rngs[r].standard_normal(int(ke[r]), dtype=np.float32)
        fill_padding(rngs[r], x[r], int(ke[r]))
    return Workload("tiny", x, ke, k, seed)


def decode(seed: int = 2, m: int = 64, n: int = 131072, k: int = 2048,
           lo: int = 32768) -> Workload:
    """Decode-indexer rows: ke ~ U[lo, n] (inclusive), ReLU-weighted 8-head scores."""
    rngs, krng = _row_streams(seed, m)
    ke = krng.integers(lo, n + 1, size=m, dtype=np.int64).astype(np.int32)
    x = np.empty((m, n), dtype=np.float32)

    def row(r):
        relu_heads(rngs[r], int(ke[r]), x[r])
        fill_padding(rngs[r], x[r], int(ke[r]))
    _parallel_rows(m, row)
    return Workload("decode", x, ke, k, seed)


def prefill(seed: int = 3, m: int = 4096, n: int = 65536, k: int = 2048,
            first: int = 61440) -> Workload:
    """Causal prefill window: ke[r] = min(first + r + 1, n)."""
    rngs, _ = _row_streams(seed, m)
    ke = np.minimum(first + np.arange(m, dtype=np.int64) + 1, n).astype(np.int32)
    x = np.empty((m, n), dtype=np.float32)

    def row(r):
        relu_heads(rngs[r], int(ke[r]), x[r])
        fill_padding(rngs[r], x[r], int(ke[r]))
    _parallel_rows(m, row)
    return Workload("prefill", x, ke, k, seed)


def long_rows(seed: int = 4, m: int = 4, n: int = 524288, k: int = 2048,
              spike_density: float = 0.001, spike_sigma: float = 3.0) -> Workload:
    """A few full-width rows with a sparse band of +3 sigma spikes.

    ceil(density * n) distinct positions per row are raised by spike_sigma
    times the row's own standard deviation (computed in float64, rounded to
    float32 once, added in float32).
    """
    rngs, _ = _row_streams(seed, m)
    ke = np.full(m, n, dtype=np.int32)
    x = np.empty((m, n), dtype=np.float32)
    nspk = int(math.ceil(spike_density * n))

    def row(r):
        rng = rngs[r]
        relu_heads(rng, n, x[r])
        sd = np.float32(spike_sigma * float(np.std(x[r].astype(np.float64))))
        pos = rng.choice(n, size=nspk, replace=False)
        x[r, pos] = x[r, pos] + sd
    _parallel_rows(m, row)
    return Workload("long", x, ke, k, seed)


CONSTANT_VALUES = np.array([1.0, 0.0, -0.0, -np.inf, np.inf, 3.4e38, -1.5],
                           dtype=np.float32)


def adversarial(seed: int = 5, m: int = 256, n: int = 262144, k: int = 2048,
                lo: int = 4096) -> Workload:
    """Recovery and tie stress rows, type = r mod 4.

    0: 64 quantized levels, x = level * 0.125 with level ~ U{0..63} (heavy ties)
    1: a ReLU-model row sorted ascending (top values all at the end)
    2: a constant row, value cycling over CONSTANT_VALUES with r // 4
    3: a ReLU-model row where each position independently becomes -inf (30%),
       -0.0 (20%), +0.0 (20%) or a random positive subnormal (1%); then a
       count of +inf cycling over {0, K/2, K, 2K+1} is planted at distinct
       random positions (capped at the valid length).
    """
    rngs, krng = _row_streams(seed, m)
    ke = krng.integers(lo, n + 1, size=m, dtype=np.int64).astype(np.int32)
    x = np.empty((m, n), dtype=np.float32)
    inf_counts = [0, k // 2, k, 2 * k + 1]

    def row(r):
        rng = rngs[r]
        L = int(ke[r])
        t = r % 4
        v = x[r, :L]
        if t == 0:
            lev = rng.integers(0, 64, size=L)
            v[:] = lev.astype(np.float32) * np.float32(0.125)
        elif t == 1:
            relu_heads(rng, L, x[r])
            v.sort()
        elif t == 2:
            v[:] = CONSTANT_VALUES[(r // 4) % len(CONSTANT_VALUES)]
        else:
            relu_heads(rng, L, x[r])
            u = rng.random(L)
            v[u < 0.30] = -np.inf
            v[(u >= 0.30) & (u < 0.50)] = np.float32(-0.0)
            v[(u >= 0.50) & (u < 0.70)] = np.float32(0.0)
            sub = (u >= 0.70) & (u < 0.71)
            nsub = int(sub.sum())
            v[sub] = rng.integers(1, 1 << 23, size=nsub, dtype=np.uint32).view(np.float32)
            cnt = min(inf_counts[(r // 4) % 4], L)
            if cnt:
                v[rng.choice(L, size=cnt, replace=False)] = np.inf
        fill_padding(rng, x[r], L)
    _parallel_rows(m, row)
    return Workload("adversarial", x, ke, k, seed)


CONFIGS = {
    "tiny": tiny,
    "decode": decode,
    "prefill": prefill,
    "long": long_rows,
    "adversarial": adversarial,
}


def make(name: str, **kw) -> Workload:
    return CONFIGS[name](**kw)


def iid_normal(seed: int, m: int, n: int, ke, k: int) -> Workload:
    """Generic i.i.d. N(0,1) rows with the given valid lengths (test helper)."""
    ke = np.asarray(ke, dtype=np.int32)
    rngs, _ = _row_streams(seed, m)
    x = np.empty((m, n), dtype=np.float32)
    for r in range(m):
        L = int(min(max(int(ke[r]), 0), n))
        x[r, :L] = rngs[r].standard_normal(L, dtype=np.float32)
        fill_padding(rngs[r], x[r], L)
    return Workload("iid", x, ke, k, seed)
