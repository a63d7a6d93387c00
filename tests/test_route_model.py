"""Pins of the CPU route model (oracle/route_model.py) against closed forms,
brute force and the finite-population statistics of the paper's Sec. 3.2
(Eq. 8), independent of the model's own histogram-prefix code."""
import math

import numpy as np
import pytest
from scipy.stats import hypergeom

from exact_row_wise_sampled_amd import workloads
from oracle import route_model as rm


def test_coarse_key_landmarks():
    # Sec. 4.2, Eq. 11 on the FP16 landmarks: +inf has FP16 pattern 0x7C00,
    # the largest finite FP16 (65504) 0x7BFF, and 65520 rounds up to +inf.
    vals = np.array([np.inf, 65520.0, 65519.0, 65504.0, 0.0, -0.0, -np.inf, 1.0, -1.0],
                    dtype=np.float32)
    c = rm.coarse_keys(vals)
    assert c.tolist() == [0x03FF >> 5, 0x03FF >> 5, 0x0400 >> 5, 0x0400 >> 5,
                          0x7FFF >> 5, 0x8000 >> 5, 0xFC00 >> 5,
                          (0x7FFF ^ 0x3C00) >> 5, 0xBC00 >> 5]
    assert c[0] == 31 and c[4] == 1023 and c[5] == 1024 and c[6] == 2016


def test_coarse_key_monotone_and_bin_width():
    # c never increases with the value; every non-NaN FP16 value lands in
    # bins 31..2016 and each bin between holds 32 consecutive FP16 patterns.
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, size=1 << 20, dtype=np.uint32)
    x = bits.view(np.float32)
    x = np.sort(x[~np.isnan(x)])
    c = rm.coarse_keys(x)
    assert np.all(np.diff(c) <= 0)
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    h = h[~np.isnan(h)].astype(np.float32)
    ch = rm.coarse_keys(h)
    assert ch.min() == 31 and ch.max() == 2016
    counts = np.bincount(ch, minlength=2048)
    assert counts[32:1023].tolist() == [32] * (1023 - 32)
    assert counts[1025:2016].tolist() == [32] * (2016 - 1025)


@pytest.mark.parametrize("s", [64, 128])
def test_phase_blocks_use_every_residue(s):
    # Eq. 13: each block of s consecutive rows uses every phase once.
    for start in (0, s, 7 * s):
        assert sorted(rm.row_phase(r, s) for r in range(start, start + s)) == list(range(s))
    assert rm.row_phase(1, s) == s // 2
    assert rm.row_phase(3, s) == s // 2 + s // 4
    assert rm.row_phase(s - 1, s) == s - 1


def test_sample_ranks():
    # 1.5K and 1.75K targets (Sec. 4.2; Sec. 6.4) at K = 2048 and K = 256.
    assert [rm.sample_rank(2048, 128, q) for q in (6, 7)] == [24, 28]
    assert [rm.sample_rank(2048, 64, q) for q in (6, 7)] == [48, 56]
    assert [rm.sample_rank(256, 128, q) for q in (6, 7)] == [3, 4]
    assert [rm.sample_rank(256, 64, q) for q in (6, 7)] == [6, 7]
    assert rm.sample_rank(5, 64, 6) == 1          # ceil(ceil(7.5) / 64)


@pytest.mark.parametrize("seed", range(6))
def test_boundaries_match_sorted_view(seed):
    # Brute force: tau0 is the coarse key of the q-th largest view value, and
    # the admitted count covers every value at or above it (Sec. 4.3).
    rng = np.random.default_rng(seed)
    s = int(rng.choice([64, 128]))
    k = int(rng.choice([64, 256, 2048]))
    L = int(rng.integers(k + 1, 70000))
    r = int(rng.integers(0, 1000))
    x = rng.standard_normal(L, dtype=np.float32)
    if seed % 2:
        x = np.round(x * 8).astype(np.float32) / np.float32(8)   # heavy ties
    pol = rm.Policy(s, True, 6, 9)
    rr = rm.route_row(x, L, r, k, pol)
    a = rm.row_phase(r, s)
    view = np.sort(x[a::s])[::-1]
    assert rr.n_view == len(view) == math.ceil((L - a) / s)
    if rr.route == "exact_direct":
        assert len(view) < rr.q1
        return
    v_q, v_q1 = view[rr.q - 1], view[rr.q1 - 1]
    assert rr.tau0 == rm.coarse_keys(np.array([v_q]))[0]
    assert rr.tau1 == rm.coarse_keys(np.array([v_q1]))[0]
    assert rr.c0 >= np.count_nonzero(x >= v_q)
    assert rr.c1 >= np.count_nonzero(x >= v_q1)


def _aliased_row(s: int, nv: int, a: int, k: int, extra_at: int | None):
    """View positions a + j*s hold 1000 - 20 j (one value per coarse bin: the
    FP16 bins are 16 wide in [512, 1024)); all other positions hold -1, except
    that k of them repeat view value number `extra_at` (0-based)."""
    L = nv * s
    x = np.full(L, -1.0, dtype=np.float32)
    x[a::s] = (1000.0 - 20.0 * np.arange(nv)).astype(np.float32)
    if extra_at is not None:
        others = np.setdiff1d(np.arange(L), np.arange(a, L, s))[:k]
        x[others] = np.float32(1000.0 - 20.0 * extra_at)
    return x, L


@pytest.mark.parametrize("s", [64, 128])
def test_routes_closed_forms(s):
    k = 256
    pol = rm.Policy(s, True, 6, 12)          # q = ceil(384/s), q1 = ceil(768/s)
    q, q1 = rm.sample_rank(k, s, 6), rm.sample_rank(k, s, 12)
    assert q1 > q
    r = 5
    a = rm.row_phase(r, s)
    nv = 24
    # Only the view's own values are large: C(tau0) = q and C(tau1) = q1.
    x, L = _aliased_row(s, nv, a, k, None)
    rr = rm.route_row(x, L, r, k, pol)
    assert (rr.route, rr.c0, rr.c1) == ("exact_underfill", q, q1)
    # K copies of view value q1 - 1 elsewhere: the band certifies.
    x, L = _aliased_row(s, nv, a, k, q1 - 1)
    rr = rm.route_row(x, L, r, k, pol)
    assert (rr.route, rr.c0, rr.c1) == ("band", q, q1 + k)
    # Primary-only policy: the same row has no band to fall back on.
    assert rm.route_row(x, L, r, k, rm.Policy(s, False, 6, 12)).route == "exact_underfill"
    # K copies of view value q - 1: the primary boundary certifies.
    x, L = _aliased_row(s, nv, a, k, q - 1)
    rr = rm.route_row(x, L, r, k, pol)
    assert (rr.route, rr.c0) == ("primary", q + k)
    # A constant row admits everything at its one bin.
    rr = rm.route_row(np.full(L, 3.0, dtype=np.float32), L, r, k, pol)
    assert (rr.route, rr.c0) == ("primary", L)
    # Sentinel, no view, unusable view.
    assert rm.route_row(x, k, r, k, pol).route == "sentinel"
    assert rm.route_row(x, L, r, k, rm.Policy(0)).route == "exact_direct"
    short = (q1 - 1) * s
    assert rm.route_row(x, short, r, k, pol).route == "exact_direct"
    assert rm.route_row(x, short, r, k, rm.Policy(s, False, 6, 12)).route != "exact_direct"


def test_counts_respect_live_rows_and_clamping():
    w = workloads.iid_normal(11, 6, 5000, [5000, 9000, -3, 100, 4000, 5000], 256)
    c = rm.route_counts(w.x, w.ke, 256, rm.Policy(64), m_live=5)
    assert sum(c.values()) == 5
    assert c["sentinel"] == 2            # ke = -3 and ke = 100
    zero = {name: 0 for name in rm.ROUTES}
    zero["hinted"] = 0
    assert rm.route_counts(w.x, w.ke, 256, rm.Policy(64), m_live=0) == zero


def _view_ranks(x, L, r, s, q):
    """J_a(q): the complete-row rank of the q-th largest view value."""
    a = rm.row_phase(r, s)
    v = np.sort(x[a:L:s])[::-1][q - 1]
    return int(np.count_nonzero(x[:L] >= v)), len(x[a:L:s])


def test_view_rank_statistics_eq8():
    # Eq. 8 (Sec. 3.2): for exchangeable rows the rank of the q-th view value
    # has mean q(L+1)/(n+1) and the stated variance; the frequency of J < K
    # is the hypergeometric tail P(#view values among the top K-1 >= q).
    # Every underfilled row has J < K (C(tau0) >= J).
    m, L, k, s = 1200, 32768, 2048, 128
    w = workloads.iid_normal(23, m, L, [L] * m, k)
    pol = rm.Policy(s, False, 6, 7)
    q = rm.sample_rank(k, s, 6)
    J = np.empty(m)
    routes = rm.route_rows(w.x, w.ke, k, pol)
    for r in range(m):
        J[r], n = _view_ranks(w.x[r], L, r, s, q)
        if routes[r].route != "primary":
            assert J[r] < k
    mean = q * (L + 1) / (n + 1)
    var = q * (n - q + 1) * (L + 1) * (L - n) / ((n + 1) ** 2 * (n + 2))
    se = math.sqrt(var / m)
    assert abs(J.mean() - mean) < 4 * se
    assert 0.8 < J.var() / var < 1.2
    p = hypergeom.sf(q - 1, L, k - 1, n)
    hits = int(np.count_nonzero(J < k))
    assert abs(hits - m * p) < 4 * math.sqrt(m * p * (1 - p)) + 2
    under = sum(rr.route != "primary" for rr in routes)
    assert under <= hits


def test_desc_keys_order():
    # Descending keys: larger values get smaller keys, +0 above -0, and the
    # FP32 landmarks at their closed-form patterns.
    v = np.array([np.inf, 3.0, 1.0, 1e-45, 0.0, -0.0, -1e-45, -1.0, -np.inf], dtype=np.float32)
    kk = rm.desc_keys(v)
    assert np.all(np.diff(kk) > 0)
    assert kk[0] == 0x7F800000 ^ 0x7FFFFFFF and kk[4] == 0x7FFFFFFF and kk[5] == 0x80000000
    assert kk[-1] == 0xFF800000


def test_hinted_routes_closed_forms():
    # A proposal replaces the view (plans with a view only): the row admits
    # every value at or above it; the count certifies it or the row goes to
    # exact recovery (no band).
    rng = np.random.default_rng(3)
    k, L = 256, 20000
    x = rng.permutation(np.arange(L, dtype=np.float32) * np.float32(0.5))   # distinct values
    vk = np.sort(x)[::-1][k - 1]
    pol = rm.Policy(128, True, 6, 10)
    rr = rm.route_row(x, L, 7, k, pol, float(vk))
    assert (rr.route, rr.c0, rr.hinted) == ("primary", k, True)
    rr = rm.route_row(x, L, 7, k, pol, float(vk) + 0.25)          # one value short
    assert (rr.route, rr.c0) == ("exact_underfill", k - 1)
    rr = rm.route_row(x, L, 7, k, pol, float(-np.inf))
    assert (rr.route, rr.c0) == ("primary", L)
    assert not rm.route_row(x, L, 7, k, pol, float("nan")).hinted   # no proposal: the view
    assert rm.route_row(x, L, 7, k, rm.Policy(0), float(vk)).route == "exact_direct"
    assert rm.route_row(x, k, 7, k, pol, float(vk)).route == "sentinel"
    z = np.full(L, -0.0, dtype=np.float32)
    z[: k + 5] = 0.0                                               # +0 ranks above -0
    assert rm.route_row(z, L, 7, k, pol, 0.0).c0 == k + 5
    c = rm.route_counts(np.stack([x, x]), [L, L], k, pol, hints=[float(vk), float("nan")])
    assert c["hinted"] == 1 and c["primary"] + c["band"] + c["exact_underfill"] == 2
