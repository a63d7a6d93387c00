"""Route parity: which route each row takes (Phases 1-2 of "Sample-Guided
Exact Top-K Selection for Long-Context Sparse Attention", Secs. 4.2-4.3 and
Sec. 6.4 "Conditional rescue") must equal the CPU route model's prediction.

The output of the selector is exact whatever the proposal does, so these
counts are what pins the view phase, the sample ranks q and q1, the boundary
search and the admitted-count certification on the device.  The workloads are
the evaluation shapes (prefill cut to its first 1024 rows); the plans are the
automatic one and forced variants of stride, secondary boundary, targets and
mapping, including tight targets that drive many rows into band rescue and
exact recovery (those runs also check exactness against the oracle).
"""
import pytest

from exact_row_wise_sampled_amd import workloads as W
from tests.gpu_util import assert_exact, assert_routes, auto_plan, note, run_topk

pytestmark = pytest.mark.gpu

_CACHE = {}


def _workload(name):
    if name not in _CACHE:
        _CACHE.clear()
        _CACHE[name] = W.prefill(m=1024) if name == "prefill1024" else W.make(name)
    return _CACHE[name]


def _plans(t):
    P, K = t.FAMILY_PERSISTENT, t.FAMILY_KVSPLIT
    return {
        "pages-default": t.make_plan(P, 128, 1, workers=96, band_quarters=7, primary_quarters=6),
        "s64-primary-only": t.make_plan(P, 64, 0, workers=96, primary_quarters=6),
        "kv-s128-dual": t.make_plan(K, 128, 1, splits=8, min_segment=4096, band_quarters=10,
                                    primary_quarters=6),
        "tight-kv": t.make_plan(K, 128, 1, splits=4, min_segment=8192, band_quarters=5,
                                primary_quarters=4),
        "tight-persistent": t.make_plan(P, 64, 1, workers=128, band_quarters=5,
                                        primary_quarters=4),
    }


WORKLOADS = ["tiny", "decode", "long", "adversarial", "prefill1024"]
PLANS = ["auto", "pages-default", "s64-primary-only", "kv-s128-dual", "tight-kv",
         "tight-persistent"]


@pytest.mark.parametrize("plan_name", PLANS)
@pytest.mark.parametrize("name", WORKLOADS)
def test_routes_match_model(name, plan_name):
    from exact_row_wise_sampled_amd import topkf as t
    w = _workload(name)
    plan = auto_plan(w.m, w.n) if plan_name == "auto" else _plans(t)[plan_name]
    note("routes %s plan %s (%s)" % (name, plan_name, plan))
    out, st, _ = run_topk(w.x, w.ke, w.k, plan=plan, stats=True)
    want = assert_routes(st, w.x, w.ke, w.k, plan)
    note("routes %s" % want)
    if plan_name.startswith("tight") and name in ("decode", "prefill1024", "tiny"):
        assert_exact(out, w.x, w.ke, w.k)
