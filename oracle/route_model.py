"""CPU model of the selector's route decisions (Phases 1 and 2).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the selector library never does, and
this module imports nothing from the selector package.

The exact Top-K result does not depend on the proposal: the pages build the
method so that sampling decides how much work a row costs, never which indices
it returns.  A wrong view phase, sample rank or boundary therefore leaves the
output exact and only shows in which route each row takes.  This module
computes that route from the definitions of "Sample-Guided Exact Top-K
Selection for Long-Context Sparse Attention", step by step in the pages'
order, with plain numpy:

  * Sec. 4.2, Eqs. 11-14: the row's view is every s-th valid position from the
    row phase a_r = pi_s(r mod s), with pi_s the bit reversal of log2(s) bits;
    each view value is projected to the 11-bit coarse key
    c(x) = kappa16(fp16_rne(x)) >> 5 and histogrammed.
  * Eq. 15: tau0 = the first bin whose inclusive prefix reaches q = ceil(K~/s),
    K~ = ceil(primary_quarters * K / 4) (1.5K in the pages); with the nested
    secondary target, tau1 from q1 = ceil(K~1/s), K~1 = ceil(band_quarters *
    K / 4).  A view with fewer than q1 samples (q without the secondary
    target) is unusable and the row goes to the exact coarse route directly
    (Sec. 5.2).
  * Sec. 4.3, Eqs. 16-19: the complete-row count C(tau0) = #{i < L : c(x_i) <=
    tau0}.  C(tau0) >= K certifies the primary tail; otherwise, when the
    secondary boundary is recorded and lies deeper, the band tau0 < c <= tau1
    is added and C(tau1) >= K certifies it (Sec. 6.4 "Conditional rescue");
    otherwise the row enters exact coarse recovery.  With tau1 == tau0 the
    band is empty and the row goes to exact recovery.
  * Sec. 4.5, Eq. 27: a KV-split row sums the counts of disjoint segments,
    which is the same complete-row count, so the route does not depend on the
    mapping.

The coarse key here is numpy's IEEE round-to-nearest-even float32 -> float16
conversion; the comparison with an inclusive FP32 cutoff that the pages use
in the scan (Sec. 5.3) is, by the pages' own argument, the same predicate as
c(x) <= tau, so this model counts with c(x) directly.

Rows of length L <= K take the sentinel layout (Sec. 2.1).

A caller-supplied proposal (a cutoff carried over from the previous decode
step, the GVR page's temporal guess) replaces the view's boundary in a plan
that has a view: the row admits every value whose descending key is at most
the proposal's, certifies it by the same complete-row count, and on underfill
goes to exact coarse recovery (there is no secondary boundary).  A NaN
proposal means none.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

ROUTES = ("sentinel", "primary", "band", "exact_underfill", "exact_direct")


def coarse_keys(x: np.ndarray) -> np.ndarray:
    """c(x) = kappa16(fp16_rne(x)) >> 5 of float32 values (Sec. 4.2, Eq. 11).

    kappa16 maps an FP16 bit pattern h to h ^ 0x7FFF when the sign is clear
    and leaves it as is when set, so a larger value gets a smaller key."""
    with np.errstate(over="ignore"):   # 65520 and up round to infinity
        h = np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16).astype(np.uint32)
    k16 = np.where(h & 0x8000, h, h ^ 0x7FFF)
    return (k16 >> 5).astype(np.int64)


def desc_keys(x: np.ndarray) -> np.ndarray:
    """Descending sortable keys of float32 values: the bit pattern with every
    bit but the sign flipped when the sign is clear, as is when set, so a
    larger value gets a smaller key and +0 ranks above -0."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return np.where(b & 0x80000000, b, b ^ 0x7FFFFFFF).astype(np.int64)


def row_phase(r: int, s: int) -> int:
    """a_r = pi_s(r mod s): the log2(s) low bits of the row index, reversed."""
    bits = int(round(math.log2(s)))
    if 1 << bits != s:
        raise ValueError("stride must be a power of two")
    if bits == 0:
        return 0
    return int(format(r % s, "0%db" % bits)[::-1], 2)


def sample_rank(k: int, s: int, quarters: int) -> int:
    """q = ceil(K~ / s) with K~ = ceil(quarters * K / 4)."""
    target = -(-quarters * k // 4)
    return -(-target // s)


@dataclass
class Policy:
    """The parts of a plan that decide routes: view stride (0 = no view),
    whether the secondary boundary is recorded, and the two targets."""
    stride: int
    dual: bool = True
    primary_quarters: int = 6
    band_quarters: int = 7


@dataclass
class RowRoute:
    route: str
    L: int
    n_view: int = 0
    q: int = 0
    q1: int = 0
    tau0: int = -1
    tau1: int = -1
    c0: int = 0   # C(tau0)
    c1: int = 0   # C(tau1) (equal to c0 without a secondary boundary)
    hinted: bool = False  # a proposal replaced the view


def first_bin_reaching(hist: np.ndarray, target: int) -> int:
    """min{b : sum_{b' <= b} hist[b'] >= target} (Eq. 15)."""
    return int(np.searchsorted(np.cumsum(hist), target, side="left"))


def route_row(x_row: np.ndarray, L: int, r: int, k: int, pol: Policy,
              hint: float | None = None) -> RowRoute:
    """The route row r (index within the call, length L) takes under `pol`,
    with an optional proposed cutoff `hint` (NaN or None: no proposal)."""
    if L <= k:
        return RowRoute("sentinel", L)
    if pol.stride == 0:
        return RowRoute("exact_direct", L)
    if hint is not None and not np.isnan(hint):
        hk = int(desc_keys(np.array([hint], dtype=np.float32))[0])
        c0 = int(np.count_nonzero(desc_keys(x_row[:L]) <= hk))
        rr = RowRoute("primary" if c0 >= k else "exact_underfill", L, c0=c0, c1=c0)
        rr.hinted = True
        return rr
    s = pol.stride
    a = row_phase(r, s)
    view = x_row[a:L:s]
    q = sample_rank(k, s, pol.primary_quarters)
    q1 = sample_rank(k, s, pol.band_quarters) if pol.dual else q
    rr = RowRoute("exact_direct", L, n_view=len(view), q=q, q1=q1)
    if len(view) < q1:
        return rr
    hist = np.bincount(coarse_keys(view), minlength=2048)
    rr.tau0 = first_bin_reaching(hist, q)
    rr.tau1 = first_bin_reaching(hist, q1)
    row_c = coarse_keys(x_row[:L])
    rr.c0 = int(np.count_nonzero(row_c <= rr.tau0))
    rr.c1 = int(np.count_nonzero(row_c <= rr.tau1)) if pol.dual else rr.c0
    if rr.c0 >= k:
        rr.route = "primary"
    elif pol.dual and rr.tau1 > rr.tau0 and rr.c1 >= k:
        rr.route = "band"
    else:
        rr.route = "exact_underfill"
    return rr


def route_rows(x: np.ndarray, ke, k: int, pol: Policy, m_live: int | None = None, hints=None):
    """Per-row routes of rows r < min(m_live, M); lengths clamped to [0, N]."""
    m, n = x.shape
    live = m if m_live is None else max(0, min(int(m_live), m))
    ke = np.asarray(ke)
    return [route_row(x[r], int(min(max(int(ke[r]), 0), n)), r, k, pol,
                      None if hints is None else float(hints[r])) for r in range(live)]


def route_counts(x: np.ndarray, ke, k: int, pol: Policy, m_live: int | None = None,
                 hints=None) -> dict:
    """Rows per route, plus `hinted`: rows whose proposal replaced the view."""
    counts = {name: 0 for name in ROUTES}
    counts["hinted"] = 0
    for rr in route_rows(x, ke, k, pol, m_live, hints):
        counts[rr.route] += 1
        counts["hinted"] += int(rr.hinted)
    return counts
