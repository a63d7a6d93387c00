"""Caller-supplied proposals (topk_filtered_hinted): a per-row cutoff carried
over from a previous decode step replaces the view's boundary, as the GVR
page's temporal guess does; the complete-row count certifies it and an
underfilled row takes the exact coarse route.  Outputs must be exact whatever
the hint, and the route counters must match the CPU route model's (including
the number of rows whose proposal replaced the view)."""
import numpy as np
import pytest

from exact_row_wise_sampled_amd import workloads as W
from tests.gpu_util import assert_exact, assert_routes, auto_plan, dev, note

pytestmark = pytest.mark.gpu


def _run(x, ke, k, hints, plan):
    import torch
    from exact_row_wise_sampled_amd import topkf as t
    d = dev()
    m, n = x.shape
    xd = torch.from_numpy(x).to(d)
    ke_d = torch.from_numpy(ke.astype(np.int32)).to(d)
    out = torch.full((m, k), -7, dtype=torch.int32, device=d)
    nvr = torch.tensor([m], dtype=torch.int32, device=d)
    h = torch.from_numpy(hints.astype(np.float32)).to(d)
    sel = t.Selector(m, n, device=d, plan=plan)
    rs = torch.zeros(t.ROUTE_COUNT, dtype=torch.int32, device=d)
    sel(xd, ke_d, out, nvr, k, route_stats=rs, hint=h)
    torch.cuda.synchronize()
    assert int(sel.counters.sum().item()) == 0
    return out.cpu().numpy(), dict(zip(t.ROUTE_NAMES, rs.cpu().numpy().tolist()))


def _kth(x, ke, k, rank):
    """Each row's value at 1-based rank `rank` (clamped to its length), by a
    full sort; NaN (no proposal) for rows with L <= K."""
    h = np.full(x.shape[0], np.nan, dtype=np.float32)
    for r in range(x.shape[0]):
        L = int(min(max(ke[r], 0), x.shape[1]))
        if L > k:
            h[r] = np.sort(x[r, :L])[::-1][min(rank, L) - 1]
    return h


def _plans(t):
    P, K = t.FAMILY_PERSISTENT, t.FAMILY_KVSPLIT
    return {
        "kv-primary": t.make_plan(K, 128, 0, splits=8, min_segment=4096, primary_quarters=8),
        "kv-dual": t.make_plan(K, 128, 1, splits=4, min_segment=4096, band_quarters=10,
                               primary_quarters=6),
        "persistent-dual": t.make_plan(P, 128, 1, workers=40, band_quarters=10, primary_quarters=7),
        "persistent-s64": t.make_plan(P, 64, 0, workers=17, primary_quarters=6),
        "no-view": t.make_plan(P, 0, 0, workers=9),
    }


@pytest.mark.parametrize("plan_name", ["auto", "kv-primary", "kv-dual", "persistent-dual",
                                       "persistent-s64", "no-view"])
def test_hints_exact_and_routes(plan_name):
    from exact_row_wise_sampled_amd import topkf as t
    w = W.decode(seed=21, m=48, n=65536, lo=2000)
    x, ke, k = w.x, w.ke.copy(), w.k
    ke[:4] = [3000, 2100, 4000, 1000]                    # views too short for q1; a sentinel row
    rng = np.random.default_rng(5)
    hk = _kth(x, ke, k, int(1.25 * k))                   # a useful proposal: rank 1.25K
    hk_tight = _kth(x, ke, k, k)                         # exactly the K-th value: certifies
    hints = hk.copy()
    sel = rng.random(x.shape[0])
    hints[sel < 0.2] = np.nan                            # no proposal: the view
    hints[(sel >= 0.2) & (sel < 0.4)] = hk_tight[(sel >= 0.2) & (sel < 0.4)]
    over = (sel >= 0.4) & (sel < 0.55)                   # one value short: exact recovery
    hints[over] = np.nextafter(hk_tight[over], np.float32(np.inf))
    hints[sel >= 0.95] = -np.inf                         # admits the whole row
    plan = auto_plan(x.shape[0], x.shape[1]) if plan_name == "auto" else _plans(t)[plan_name]
    note("hinted rows plan %s (%s)" % (plan_name, plan))
    out, st = _run(x, ke, k, hints, plan)
    assert_exact(out, x, ke, k)
    want = assert_routes(st, x, ke, k, plan, hints=hints)
    note("routes %s" % want)
    if plan.stride:
        assert want["hinted"] > 0 and want["exact_underfill"] > 0


def test_hints_on_long_and_tied_rows():
    """Few long rows (KV-split) and tied rows with proposals at and around the
    K-th value."""
    from exact_row_wise_sampled_amd import topkf as t
    w = W.long_rows()
    x, ke, k = w.x.copy(), w.ke, w.k
    x[1] = np.round(x[1] * 2) / 2                          # heavy ties at the boundary
    x[2] = np.float32(1.25)                                # every value tied
    hints = _kth(x, ke, k, k)
    hints[3] = np.nan
    for name, plan in (("auto", auto_plan(x.shape[0], x.shape[1])),
                       ("kv-dual", _plans(t)["kv-dual"])):
        note("hinted long rows plan %s" % name)
        out, st = _run(x, ke, k, hints, plan)
        assert_exact(out, x, ke, k)
        assert_routes(st, x, ke, k, plan, hints=hints)
