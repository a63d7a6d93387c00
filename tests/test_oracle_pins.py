"""Pins for the CPU oracle, independent of the oracle's own code.

The oracle (oracle/topk_oracle.c) sorts each valid prefix with qsort.  These
tests fix its answers against things other than itself:
  * hand-worked rows of the operator contract (tests/golden/contract_cases.json,
    "Sample-Guided Exact Top-K Selection ...", Sec. 2.1 and Eq. 30);
  * a brute-force counting definition in pure Python on tiny rows, for every K;
  * closed-form rows (constant, ascending, descending, +inf floods, L <= K);
  * numpy's own sort of the same values (a different library routine);
  * the checker: it accepts the oracle's answers and tie swaps, and rejects
    planted mistakes.
"""
import json
import math
import os
import struct

import numpy as np
import pytest

from oracle import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "contract_cases.json")


def f32(v):
    if isinstance(v, str):
        return np.float32(float(v))
    return np.float32(v)


def bits(v):
    return struct.unpack("<I", struct.pack("<f", float(v)))[0]


def rank_gt(a, b):
    """a ranks strictly above b: numerically larger, or +0.0 against -0.0."""
    if a > b:
        return True
    if a == b == 0.0:
        return math.copysign(1.0, a) > 0 > math.copysign(1.0, b)
    return False


def brute(row, K):
    """Counting definition: the K-th value v has #{x > v} < K <= #{x >= v}."""
    vals = [float(v) for v in row]
    for v in vals:
        above = sum(1 for u in vals if rank_gt(u, v))
        same = sum(1 for u in vals if bits(u) == bits(v))
        if above < K <= above + same:
            strict = {i for i, u in enumerate(vals) if rank_gt(u, v)}
            ties = {i for i, u in enumerate(vals) if bits(u) == bits(v)}
            return v, strict, ties
    raise AssertionError("no K-th value found")


def run_oracle(rows, K, n=None):
    n = n or max(len(r) for r in rows)
    x = np.zeros((len(rows), n), dtype=np.float32)
    ke = np.zeros(len(rows), dtype=np.int32)
    for i, r in enumerate(rows):
        x[i, :len(r)] = np.asarray(r, dtype=np.float32)
        ke[i] = len(r)
    return x, ke, oracle.topk(x, ke, K)


def assert_matches(res, r, row, K):
    L = len(row)
    if L <= K:
        assert list(res.sel_idx[r]) == list(range(L)) + [-1] * (K - L)
        return
    v, strict, ties = brute(row, K)
    ns = int(res.n_strict[r])
    idx = [int(i) for i in res.sel_idx[r]]
    assert ns == len(strict)
    assert set(idx[:ns]) == strict
    assert len(set(idx)) == K
    assert set(idx[ns:]) <= ties
    assert all(int(b) == bits(v) for b in res.sel_bits[r][ns:])
    want = sorted([bits(row[i]) for i in strict] + [bits(v)] * (K - ns))
    assert sorted(int(b) for b in res.sel_bits[r]) == want


def test_golden_contract_cases():
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        row = [f32(v) for v in c["row"]][: c["L"]]
        K = c["K"]
        x = np.zeros((1, max(len(c["row"]), 1)), dtype=np.float32)
        x[0, :len(c["row"])] = [f32(v) for v in c["row"]]
        ke = np.array([c["L"]], dtype=np.int32)
        res = oracle.topk(x, ke, K)
        idx = [int(i) for i in res.sel_idx[0]]
        if "sentinel" in c:
            assert idx == c["sentinel"], c
            continue
        ns = int(res.n_strict[0])
        assert set(idx[:ns]) == set(c["strict"]), c
        assert ns == len(c["strict"])
        assert set(idx[ns:]) <= set(c["ties"]) and len(idx[ns:]) == c["take"], c
        assert int(res.sel_bits[0][K - 1]) == bits(f32(c["kth"])), c
        # the checker accepts every valid tie choice
        for alt in c["ties"]:
            out = list(c["strict"]) + [alt] + [t for t in c["ties"] if t != alt][: c["take"] - 1]
            out = out[:K]
            assert oracle.check_row(np.array(out), x[0], c["L"], K, res.sel_bits[0],
                                    res.sel_idx[0], ns) is None, (c, out)


SPECIALS = [0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45, 3e-39, -3e-39, 1.0, -1.0, 2.0,
            65504.0, 65520.0, 3.4e38, -3.4e38, 0.5]


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_every_k(seed):
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(1, 48))
    kind = seed % 3
    if kind == 0:
        row = rng.standard_normal(L).astype(np.float32)
    elif kind == 1:
        row = rng.integers(-3, 4, size=L).astype(np.float32)  # heavy ties
    else:
        row = np.array(rng.choice(SPECIALS, size=L), dtype=np.float32)
    for K in range(1, L + 2):
        _, _, res = run_oracle([row], K)
        assert_matches(res, 0, list(row), K)


def test_brute_force_medium_rows():
    rng = np.random.default_rng(7)
    rows = [np.array(rng.choice(SPECIALS + [0.25, -0.25], size=300), dtype=np.float32),
            rng.integers(0, 5, size=257).astype(np.float32),
            rng.standard_normal(512).astype(np.float32)]
    for K in (1, 2, 50, 128, 256, 299):
        _, _, res = run_oracle(rows, K)
        for r, row in enumerate(rows):
            assert_matches(res, r, list(row), K)


def test_closed_forms():
    K = 16
    L = 100
    const = np.full(L, 2.5, dtype=np.float32)
    asc = np.arange(L, dtype=np.float32) * np.float32(0.5) - 7
    desc = asc[::-1].copy()
    infs = np.concatenate([np.full(K + 3, np.inf, dtype=np.float32),
                           np.arange(L - K - 3, dtype=np.float32)])
    x, ke, res = run_oracle([const, asc, desc, infs], K)
    # constant row: nothing strictly above, K copies of the value
    assert res.n_strict[0] == 0
    assert (res.sel_bits[0] == bits(2.5)).all()
    # ascending distinct row: exactly the last K positions
    assert set(res.sel_idx[1]) == set(range(L - K, L))
    assert res.n_strict[1] == K - 1
    # descending: the first K positions
    assert set(res.sel_idx[2]) == set(range(K))
    # at least K copies of +inf: K times +inf, none strictly above
    assert res.n_strict[3] == 0
    assert (res.sel_bits[3] == 0x7F800000).all()
    assert set(res.sel_idx[3]) <= set(range(K + 3))


def test_length_clamping_and_live_rows():
    K = 4
    x = np.arange(40, dtype=np.float32).reshape(4, 10)
    ke = np.array([-5, 3, 99, 10], dtype=np.int32)
    res = oracle.topk(x, ke, K, m_live=3)
    assert res.rows == 3
    assert list(res.lengths) == [0, 3, 10]
    assert list(res.sel_idx[0]) == [-1] * 4
    assert list(res.sel_idx[1]) == [0, 1, 2, -1]
    assert set(res.sel_idx[2]) == {6, 7, 8, 9}
    assert oracle.topk(x, ke, K, m_live=0).rows == 0
    assert oracle.topk(x, ke, K, m_live=-3).rows == 0


def test_padded_columns_never_read():
    # values past ke must not influence the answer
    K = 3
    x = np.zeros((2, 12), dtype=np.float32)
    x[:, :6] = [1, 5, 2, 8, 3, 4]
    x[0, 6:] = np.inf
    x[1, 6:] = np.nan
    res = oracle.topk(x, np.array([6, 6], dtype=np.int32), K)
    assert set(res.sel_idx[0]) == {1, 3, 5} == set(res.sel_idx[1])


def test_against_numpy_sort():
    rng = np.random.default_rng(11)
    M, N, K = 12, 3000, 64
    x = rng.standard_normal((M, N)).astype(np.float32)
    x[3] = np.round(x[3] * 4) / 4          # ties
    x[5, ::7] = np.inf
    x[6, ::3] = -np.inf
    ke = rng.integers(K + 1, N + 1, size=M).astype(np.int32)
    res = oracle.topk(x, ke, K)
    for r in range(M):
        L = ke[r]
        top = np.sort(x[r, :L].astype(np.float64))[::-1][:K]
        got = x[r, res.sel_idx[r]].astype(np.float64)
        assert np.array_equal(np.sort(got)[::-1], top)
        assert oracle.check_row(res.sel_idx[r], x[r], int(L), K, res.sel_bits[r],
                                res.sel_idx[r], int(res.n_strict[r])) is None


def test_threads_agree():
    rng = np.random.default_rng(5)
    x = rng.integers(0, 50, size=(20, 900)).astype(np.float32)
    ke = rng.integers(0, 900, size=20).astype(np.int32)
    a = oracle.topk(x, ke, 100, threads=1)
    b = oracle.topk(x, ke, 100, threads=7)
    assert np.array_equal(a.sel_bits, b.sel_bits)
    assert np.array_equal(a.sel_idx, b.sel_idx)
    assert np.array_equal(a.n_strict, b.n_strict)


def test_checker_rejects_planted_mistakes():
    rng = np.random.default_rng(9)
    N, K = 500, 20
    x = rng.standard_normal((1, N)).astype(np.float32)
    x[0, 10] = x[0, 11] = x[0, 12] = np.float32(9.0)  # ties above everything
    res = oracle.topk(x, np.array([N], dtype=np.int32), K)
    good = res.sel_idx[0].copy()
    chk = lambda out: oracle.check_row(out, x[0], N, K, res.sel_bits[0], res.sel_idx[0],
                                       int(res.n_strict[0]))
    assert chk(good) is None
    assert chk(good[::-1].copy()) is None                 # order is free
    unselected = np.setdiff1d(np.arange(N), good)
    worst = unselected[np.argmin(x[0, unselected])]
    bad = good.copy(); bad[-1] = worst
    assert "multiset" in chk(bad)                        # smaller value swapped in
    bad = good.copy(); bad[1] = bad[0]
    assert "duplicate" in chk(bad)
    bad = good.copy(); bad[2] = N
    assert "range" in chk(bad)
    bad = good.copy(); bad[0] = -1
    assert "range" in chk(bad)
    # sentinel rows
    L = 5
    res2 = oracle.topk(x, np.array([L], dtype=np.int32), K)
    ok = np.array(list(range(L)) + [-1] * (K - L))
    chk2 = lambda out: oracle.check_row(out, x[0], L, K, res2.sel_bits[0], res2.sel_idx[0],
                                        int(res2.n_strict[0]))
    assert chk2(ok) is None
    bad = ok.copy(); bad[L] = 0
    assert chk2(bad) is not None
    bad = ok.copy(); bad[0], bad[1] = bad[1], bad[0]
    assert chk2(bad) is not None


def test_checker_strict_set_with_equal_multiset():
    # Two positions hold the same bits: swapping a strictly-above index for a
    # different index with the same value keeps the multiset, so the strict-set
    # rule is what catches it only when values differ; build a case where the
    # K-th value ties and a strict index is dropped for a tie of lower rank.
    x = np.array([[5, 5, 4, 4, 4, 1]], dtype=np.float32)
    K = 3
    res = oracle.topk(x, np.array([6], dtype=np.int32), K)
    assert res.n_strict[0] == 2
    chk = lambda out: oracle.check_row(np.array(out), x[0], 6, K, res.sel_bits[0],
                                       res.sel_idx[0], int(res.n_strict[0]))
    assert chk([0, 1, 3]) is None
    assert chk([0, 1, 4]) is None
    assert chk([0, 2, 3]) is not None


# ------------------------------------------------- c(x) reference (Eq. 11)

def _numpy_coarse(bits: np.ndarray) -> np.ndarray:
    """c(x) from numpy's own IEEE round-to-nearest-even float32 -> float16
    conversion (a software routine, independent of the host's F16C unit)."""
    with np.errstate(over="ignore"):
        h = bits.view(np.float32).astype(np.float16).view(np.uint16).astype(np.uint32)
    return (np.where(h & 0x8000, h, h ^ 0x7FFF) >> 5).astype(np.uint16)


def _windows() -> list[tuple[int, int]]:
    """Pattern ranges around every place the conversion changes regime: the
    signed zeros, the binary16 subnormal/normal boundary and smallest
    subnormal, the overflow threshold 65520 (and 65504 below it), the
    infinities and the first NaN patterns, and the ends of the pattern space."""
    centers = [0x00000000, 0x33000000, 0x33800000, 0x387FE000, 0x38800000, 0x3F800000,
               0x477FE000, 0x477FF000, 0x47800000, 0x7F800000, 0xFFFFFFFF - 4096]
    out = []
    for c in centers:
        for sign in (0, 0x80000000):
            lo = max(0, min((c | sign) - 4096, (1 << 32) - 8192))
            out.append((lo, 8192))
    return out


def test_coarse_check_matches_numpy_fp16():
    """The C reference behind the exhaustive device pin of c(x) agrees with
    numpy's conversion on every boundary window and 4M random patterns."""
    try:
        for start, n in _windows():
            bits = (np.arange(n, dtype=np.uint64) + start).astype(np.uint32)
            keep = (bits & 0x7FFFFFFF) <= 0x7F800000
            want = _numpy_coarse(bits)
            want[~keep] = 0   # NaN patterns are skipped by the checker
            assert oracle.coarse_check(start, want) == (0, None), hex(start)
        rng = np.random.default_rng(17)
        for _ in range(4):
            start = int(rng.integers(0, (1 << 32) - (1 << 20)))
            bits = (np.arange(1 << 20, dtype=np.uint64) + start).astype(np.uint32)
            assert oracle.coarse_check(start, _numpy_coarse(bits))[0] == 0
    except RuntimeError as e:
        pytest.skip(str(e))


def test_coarse_check_finds_planted_mismatches():
    """One flipped key is counted and located; NaN patterns are not compared."""
    try:
        start = 0x47000000
        bits = (np.arange(1 << 16, dtype=np.uint64) + start).astype(np.uint32)
        got = _numpy_coarse(bits)
        got[777] ^= 1
        got[40000] += 3
        assert oracle.coarse_check(start, got) == (2, start + 777)
        nan_start = 0x7F800001
        assert oracle.coarse_check(nan_start, np.full(4096, 123, dtype=np.uint16)) == (0, None)
        # +inf: 0x7C00 ^ 0x7FFF = 0x03FF -> 31, and 65520 rounds up to +inf;
        # just below 65520 rounds to 65504 = 0x7BFF -> 0x0400 -> 32
        got = _numpy_coarse(np.array([0x7F800000, 0x477FF000, 0x477FEFFF], dtype=np.uint32))
        assert got.tolist() == [31, 31, 32]
    except RuntimeError as e:
        pytest.skip(str(e))
