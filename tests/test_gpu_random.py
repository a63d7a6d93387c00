"""Seeded randomized parity sweep of the HIP selector against the CPU oracle.

Each case draws a shape, a length mix, K, a value structure and a plan (the
automatic one or a forced family / view / band / primary / split / worker
setting), runs the selector through the C ABI and checks the oracle's exact
criterion (value multiset bit-identical, every index strictly above the K-th
value selected, distinct in-range indices, sentinel layout, rows >= M_live
untouched), and that the route counters equal the CPU route model's counts.
Sizes keep the oracle to seconds.
"""
import numpy as np
import pytest

from tests.gpu_util import assert_exact, assert_routes, auto_plan, note, run_topk

pytestmark = pytest.mark.gpu

N_CASES = 160


def _values(rng, kind: str, m: int, n: int) -> np.ndarray:
    if kind == "normal":
        x = rng.standard_normal((m, n), dtype=np.float32)
    elif kind == "relu":
        g = rng.standard_normal((8, m, n), dtype=np.float32)
        w = rng.random((m, 8), dtype=np.float32)
        x = np.zeros((m, n), dtype=np.float32)
        for h in range(8):
            x = x + w[:, h:h + 1] * np.maximum(g[h], np.float32(0))
    elif kind == "levels":                      # heavy ties
        x = (rng.integers(0, 16, size=(m, n)).astype(np.float32) * np.float32(0.25))
    elif kind == "constant":
        vals = np.array([1.0, 0.0, -0.0, -np.inf, np.inf, 3.4e38, -1.5], dtype=np.float32)
        x = np.repeat(vals[rng.integers(0, len(vals), size=m)][:, None], n, axis=1)
    elif kind == "sorted":
        x = np.sort(rng.standard_normal((m, n), dtype=np.float32), axis=1)
        if rng.random() < 0.5:
            x = x[:, ::-1].copy()
    else:                                       # specials planted into normal rows
        x = rng.standard_normal((m, n), dtype=np.float32)
        for v, frac in ((np.inf, 0.002), (-np.inf, 0.05), (0.0, 0.05), (-0.0, 0.05),
                        (np.float32(1e-40), 0.01), (np.float32(-1e-42), 0.01)):
            mask = rng.random((m, n)) < frac
            x[mask] = v
    return np.ascontiguousarray(x, dtype=np.float32)


def _lengths(rng, m: int, n: int, k: int) -> np.ndarray:
    mix = rng.integers(0, 3)
    if mix == 0:
        ke = rng.integers(0, n + 1, size=m)
    elif mix == 1:
        ke = np.full(m, n)
    else:   # around K, plus the edges
        cands = np.array([0, 1, max(k - 1, 0), k, k + 1, 2 * k + 3, n, n - 1, n // 2])
        ke = rng.choice(np.clip(cands, 0, n), size=m)
    return ke.astype(np.int32)


def _plan(rng, t):
    if rng.random() < 0.35:
        return None, "auto"
    fam = t.FAMILY_PERSISTENT if rng.random() < 0.5 else t.FAMILY_KVSPLIT
    stride = int(rng.choice([0, 64, 128]))
    dual = int(stride != 0 and rng.random() < 0.7)
    prim = int(rng.integers(5, 9))
    band = int(rng.integers(prim + 1, 13))
    if fam == t.FAMILY_PERSISTENT:
        plan = t.make_plan(fam, stride, dual, workers=int(rng.integers(1, 40)),
                           band_quarters=band, primary_quarters=prim)
    else:
        plan = t.make_plan(fam, stride, dual, splits=int(rng.integers(1, 24)),
                           min_segment=int(rng.choice([512, 1024, 4096, 8192])),
                           band_quarters=band, primary_quarters=prim)
    return plan, "fam%d s%d dual%d P%d W%d q%d/%d" % (plan.family, plan.stride, plan.dual,
                                                     plan.splits, plan.workers, prim, band)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_case(case):
    from exact_row_wise_sampled_amd import topkf as t
    rng = np.random.default_rng(1000 + case)
    n = int(rng.choice([700, 3000, 9000, 20000, 70000, 150000]))
    m = int(rng.integers(1, 24 if n <= 20000 else 8))
    k = int(rng.choice([1, 7, 64, 256, 1000, 2048]))
    kind = str(rng.choice(["normal", "relu", "levels", "constant", "sorted", "special"]))
    x = _values(rng, kind, m, n)
    ke = _lengths(rng, m, n, k)
    m_live = int(rng.integers(0, m + 1)) if rng.random() < 0.2 else None
    plan, pname = _plan(rng, t)
    note("random case %d: M=%d N=%d K=%d %s live=%s plan %s" % (case, m, n, k, kind, m_live, pname))
    out, st, _ = run_topk(x, ke, k, m_live=m_live, plan=plan, stats=True)
    assert_exact(out, x, ke, k, m_live=m_live)
    assert_routes(st, x, ke, k, plan if plan is not None else auto_plan(m, n), m_live=m_live)
