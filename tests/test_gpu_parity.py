"""Parity of the HIP selector with the CPU oracle, through the C ABI.

Exactness is the set-valued criterion of "Sample-Guided Exact Top-K Selection
..." Eq. 30: bit-identical selected value multiset, every index strictly above
the K-th value selected, K distinct in-range indices (or the sentinel layout
when L <= K).  No floating-point tolerance: the selector is exact.
"""
import numpy as np
import pytest

from exact_row_wise_sampled_amd import workloads as W
from tests.gpu_util import aliased_rows, assert_exact, note, run_topk

pytestmark = pytest.mark.gpu


def topkf():
    from exact_row_wise_sampled_amd import topkf as t
    return t


# ------------------------------------------------------------ full workloads

@pytest.mark.parametrize("name", ["tiny", "decode", "long", "adversarial"])
def test_workload_auto_plan(name):
    w = W.make(name)
    note("workload %s M=%d N=%d K=%d auto plan" % (name, w.m, w.n, w.k))
    out, st, _ = run_topk(w.x, w.ke, w.k, stats=True)
    assert_exact(out, w.x, w.ke, w.k)
    note("routes %s" % st)


def test_workload_prefill_auto_plan():
    w = W.make("prefill")
    note("workload prefill M=%d N=%d auto plan" % (w.m, w.n))
    out, st, _ = run_topk(w.x, w.ke, w.k, stats=True)
    assert_exact(out, w.x, w.ke, w.k)
    note("routes %s" % st)


@pytest.mark.parametrize("m,n", [(64, 65536), (4, 65536), (128, 131072), (32, 131072),
                                 (48, 131072), (40, 131072)])
def test_planner_kvsplit_shapes_auto_plan(m, n):
    """Shapes whose automatic plan is KV-split with 4, 5, 6 or 8 parts (about
    one part per CU): ragged decode-model rows with ke ~ U[N/2, N], the first row cut
    to a length of 3 mod 4 and the last to exactly K + 1 (both shorter than
    the generated length, so every valid score is a generated one)."""
    t = topkf()
    w = W.decode(seed=50 + m, m=m, n=n, lo=n // 2)
    ke = w.ke.copy()
    ke[0] = (int(ke[0]) // 4) * 4 - 1
    ke[-1] = w.k + 1
    plan = t.plan_for(m, n, 256)
    assert plan.family == t.FAMILY_KVSPLIT, plan
    note("planner KV shape M=%d N=%d splits=%d" % (m, n, plan.splits))
    out, st, _ = run_topk(w.x, ke, w.k, stats=True)
    assert_exact(out, w.x, ke, w.k)
    note("routes %s" % st)


@pytest.mark.parametrize("m,n", [(64, 10240), (1024, 8193)])
def test_planner_view_just_past_register_rows(m, n):
    """Rows just past the 8192 scores the exact route keeps in registers take
    the view on the automatic plan."""
    t = topkf()
    w = W.decode(seed=70 + m, m=m, n=n, lo=n // 2)
    plan = t.plan_for(m, n, 256)
    assert plan.family == t.FAMILY_PERSISTENT and plan.stride == 128, plan
    note("planner view shape M=%d N=%d" % (m, n))
    out, st, _ = run_topk(w.x, w.ke, w.k, stats=True)
    assert_exact(out, w.x, w.ke, w.k)
    note("routes %s" % st)


# -------------------------------------------------------- forced mappings

def plans():
    t = topkf()
    P, K = t.FAMILY_PERSISTENT, t.FAMILY_KVSPLIT
    return {
        "pers-exact": t.make_plan(P, 0, 0, workers=7),
        "pers-s64": t.make_plan(P, 64, 0, workers=5),
        "pers-s64-dual": t.make_plan(P, 64, 1, workers=16),
        "pers-s128": t.make_plan(P, 128, 0, workers=3),
        "pers-s128-dual": t.make_plan(P, 128, 1, workers=64),
        "kv-s128-dual-p4": t.make_plan(K, 128, 1, splits=4, min_segment=1024),
        "kv-s64-p3": t.make_plan(K, 64, 0, splits=3, min_segment=4096),
        "kv-s128-dual-p16": t.make_plan(K, 128, 1, splits=16, min_segment=512),
        "kv-exact-p2": t.make_plan(K, 0, 0, splits=2, min_segment=4096),
    }


PLAN_NAMES = ["pers-exact", "pers-s64", "pers-s64-dual", "pers-s128", "pers-s128-dual",
              "kv-s128-dual-p4", "kv-s64-p3", "kv-s128-dual-p16", "kv-exact-p2"]


@pytest.mark.parametrize("plan_name", PLAN_NAMES)
def test_mixed_rows_every_plan(plan_name):
    """Ragged i.i.d. and adversarial rows spanning several tiles and a ragged tail."""
    k = 256
    n = 20000
    lens = [0, 1, k - 1, k, k + 1, 300, 1000, 2047, 4097, 8191, 12345, 19999, 20000, 20000,
            5000, 17001]
    w = W.iid_normal(31, len(lens), n, lens, k)
    adv = W.adversarial(seed=9, m=8, n=n, k=k, lo=2 * k)
    x = np.concatenate([w.x, adv.x])
    ke = np.concatenate([w.ke, adv.ke]).astype(np.int32)
    note("mixed rows plan %s" % plan_name)
    out, st, _ = run_topk(x, ke, k, plan=plans()[plan_name])
    assert_exact(out, x, ke, k)
    assert sum(st.values()) - st["spill"] == len(ke)


@pytest.mark.parametrize("plan_name", PLAN_NAMES)
def test_decode_shape_every_plan(plan_name):
    w = W.decode(seed=12, m=24, n=65536, lo=3000)
    note("decode-like rows plan %s" % plan_name)
    out, st, _ = run_topk(w.x, w.ke, w.k, plan=plans()[plan_name])
    assert_exact(out, w.x, w.ke, w.k)


@pytest.mark.parametrize("k", [1, 2, 7, 100, 2047, 2048])
def test_rank_values(k):
    w = W.iid_normal(40 + k, 6, 30000, [30000, 29999, 12000, 5000, k + 1, k], k)
    for name in ("pers-exact", "pers-s128-dual", "kv-s128-dual-p4"):
        note("rank K=%d plan %s" % (k, name))
        out, _, _ = run_topk(w.x, w.ke, k, plan=plans()[name])
        assert_exact(out, w.x, w.ke, k)


# ------------------------------------------------------------ forced routes

def test_route_primary_certified():
    t = topkf()
    w = W.iid_normal(5, 8, 65536, [65536] * 8, 2048)
    plan = t.make_plan(t.FAMILY_PERSISTENT, 128, 1, workers=4)
    out, st, _ = run_topk(w.x, w.ke, 2048, plan=plan)
    assert_exact(out, w.x, w.ke, 2048)
    assert st["primary"] >= 6, st


@pytest.mark.parametrize("family", ["persistent", "kvsplit"])
def test_route_band_rescue(family):
    t = topkf()
    k, s, n = 512, 128, 40000
    x, ke = aliased_rows(s, k, n, 6, "band", seed=1)
    if family == "persistent":
        plan = t.make_plan(t.FAMILY_PERSISTENT, s, 1, workers=3)
    else:
        plan = t.make_plan(t.FAMILY_KVSPLIT, s, 1, splits=4, min_segment=2048)
    note("band rescue %s" % family)
    out, st, _ = run_topk(x, ke, k, plan=plan)
    assert_exact(out, x, ke, k)
    assert st["band"] == 6, st


@pytest.mark.parametrize("family", ["persistent", "kvsplit"])
@pytest.mark.parametrize("dual", [0, 1])
def test_route_exact_recovery(family, dual):
    t = topkf()
    k, s, n = 512, 64, 40000
    x, ke = aliased_rows(s, k, n, 5, "exact", seed=2)
    if family == "persistent":
        plan = t.make_plan(t.FAMILY_PERSISTENT, s, dual, workers=2)
    else:
        plan = t.make_plan(t.FAMILY_KVSPLIT, s, dual, splits=3, min_segment=2048)
    note("exact recovery %s dual=%d" % (family, dual))
    out, st, _ = run_topk(x, ke, k, plan=plan)
    assert_exact(out, x, ke, k)
    assert st["exact_underfill"] == 5, st


def test_route_unusable_view_goes_exact():
    t = topkf()
    k = 2048
    # |V| = ceil(L / 128) < q1 = 28 for L < 3457
    w = W.iid_normal(8, 4, 8192, [2100, 3000, 3400, 2049], k)
    plan = t.make_plan(t.FAMILY_PERSISTENT, 128, 1, workers=4)
    out, st, _ = run_topk(w.x, w.ke, k, plan=plan)
    assert_exact(out, w.x, w.ke, k)
    assert st["exact_direct"] == 4, st


def test_spill_rows_constant_and_quantized():
    """Frontiers far beyond on-chip capacity: every value in one coarse bin."""
    t = topkf()
    k, n = 2048, 200000
    x = np.empty((4, n), dtype=np.float32)
    x[0] = 1.0
    x[1] = -0.0
    x[2] = np.float32(0.125) * np.random.default_rng(3).integers(0, 4, size=n).astype(np.float32)
    x[3] = np.inf
    ke = np.array([n, n - 5, n - 77, 150001], dtype=np.int32)
    for name, plan in (("pers", t.make_plan(t.FAMILY_PERSISTENT, 128, 1, workers=2)),
                       ("kv", t.make_plan(t.FAMILY_KVSPLIT, 128, 1, splits=8, min_segment=4096)),
                       ("exact", t.make_plan(t.FAMILY_PERSISTENT, 0, 0, workers=4))):
        note("spill rows plan %s" % name)
        out, st, _ = run_topk(x, ke, k, plan=plan)
        assert_exact(out, x, ke, k)


def test_tied_candidates_shortcut_boundary():
    """Rows whose candidates all share one key take the direct tie fill; a
    single differing value (above, or +0 against -0) must still be separated."""
    t = topkf()
    k, n = 2048, 100000
    rng = np.random.default_rng(11)
    x = np.empty((6, n), dtype=np.float32)
    x[0] = 1.0                                   # all candidates tied
    x[1] = 1.0
    x[1, rng.integers(0, n)] = 2.0               # one value above the tie
    x[2] = 1.0
    x[2, rng.integers(0, n)] = 0.5               # one value below: not a candidate
    x[3] = -0.0
    x[3, rng.choice(n, 10, replace=False)] = 0.0  # +0 ranks above -0
    x[4] = -np.inf
    x[4, rng.choice(n, 3000, replace=False)] = np.float32(3.4e38)
    x[5] = np.float32(-1.5)
    ke = np.array([n, n - 3, n, n - 1000, n, 70001], dtype=np.int32)
    for name, plan in (("kv-p8", t.make_plan(t.FAMILY_KVSPLIT, 128, 1, splits=8, min_segment=4096)),
                       ("kv-p3", t.make_plan(t.FAMILY_KVSPLIT, 64, 0, splits=3, min_segment=4096))):
        note("tied candidate rows plan %s" % name)
        out, st, _ = run_topk(x, ke, k, plan=plan, stats=True)
        assert_exact(out, x, ke, k)
        note("routes %s" % st)


def kv_part_counts(sel, m_cap: int, n: int, splits: int) -> np.ndarray:
    """The per-part (primary, band) candidate counts a KV-split scan stored in
    the workspace: after M_cap regions of 2 (n + 128) eight-byte pairs, two
    words per part and row."""
    base = 16 * m_cap * (n + 128)
    words = sel.workspace[base:base + 8 * m_cap * splits].cpu().numpy().view(np.uint32)
    return words.reshape(m_cap, splits, 2)


def test_kv_flood_rows_store_at_most_k_copies():
    """Constant, signed-zero and +inf-flood rows over several parts: each part
    stores the first bulk batches of its flood key that reach K copies and
    counts the rest out, and the answer stays exact (any K equal keys at the
    boundary, Sec. 4.4).  Two interleaved floods and a dense run of distinct
    values in one coarse bin take the same scan form and must stay exact."""
    t = topkf()
    k, n = 2048, 262144
    rng = np.random.default_rng(21)
    x = np.empty((8, n), dtype=np.float32)
    x[0] = 1.0                                    # constant
    x[1] = -0.0                                   # -0 flood with a few +0 above it
    x[1, rng.choice(n, 40, replace=False)] = 0.0
    x[2] = 0.0                                    # +0 flood
    x[3] = np.inf                                 # +inf flood
    x[4] = -np.inf                                # a few finite values above a -inf flood
    x[4, rng.choice(n, 1500, replace=False)] = rng.random(1500).astype(np.float32)
    x[5] = np.float32(0.5)                        # a tie flood after a run of distinct values
    x[5, :3000] = rng.random(3000).astype(np.float32) + np.float32(1.0)
    x[6] = np.where(rng.random(n) < 0.5, np.float32(1.0), np.float32(2.0))  # two floods interleaved
    x[7] = np.float32(1.0) + np.float32(0.03) * rng.random(n).astype(np.float32)  # one coarse bin, distinct
    ke = np.array([n, n - 3, 200001, n - 77, n, 150004, n - 9, n], dtype=np.int32)
    for name, P in (("kv-p4", 4), ("kv-p8", 8)):
        plan = t.make_plan(t.FAMILY_KVSPLIT, 128, 0, splits=P, min_segment=4096)
        note("flood rows plan %s" % name)
        out, st, sel = run_topk(x, ke, k, plan=plan, stats=True)
        assert_exact(out, x, ke, k)
        cnt = kv_part_counts(sel, x.shape[0], n, P)
        # bulk copies: K plus one batch; partial and mixed batches: a few per
        # wave and segment end; plus the distinct run of row 5
        bound = k + 8 * 256 + 2 * 512
        for r in (0, 1, 2, 3, 4):
            assert int(cnt[r, :, 0].max()) <= bound, (r, cnt[r, :, 0])
            assert int(cnt[r, :, 0].sum()) >= k, (r, cnt[r, :, 0])
        assert int(cnt[5, :, 0].max()) <= bound + 3000, cnt[5, :, 0]
        note("routes %s" % st)


def test_kv_finisher_slot_layouts():
    """The KV-split finisher maps each part's candidates to fixed register
    slots when no part holds more than its share, and searches the part
    offsets otherwise.  Rows whose tail sits in one segment (ascending,
    descending, a block of large values in the middle) force the search;
    i.i.d. rows take the direct map; both with and without the band."""
    t = topkf()
    k, n = 2048, 65536
    rng = np.random.default_rng(12)
    x = rng.standard_normal((8, n), dtype=np.float32)
    x[0] = np.sort(x[0])                          # tail in the last segment
    x[1] = np.sort(x[1])[::-1]                    # tail in the first segment
    x[2, 30000:34000] += np.float32(6.0)          # tail inside one middle segment
    x[3, ::8] += np.float32(4.0)                  # tail spread evenly
    ke = np.array([n, n, n, n, n - 5, 40000, 20000, n], dtype=np.int32)
    plans = (("kv-p8-primary", t.make_plan(t.FAMILY_KVSPLIT, 128, 0, splits=8, min_segment=4096,
                                           primary_quarters=8)),
             ("kv-p8-dual", t.make_plan(t.FAMILY_KVSPLIT, 128, 1, splits=8, min_segment=4096,
                                        band_quarters=10, primary_quarters=6)),
             ("kv-p16-tight", t.make_plan(t.FAMILY_KVSPLIT, 64, 1, splits=16, min_segment=2048,
                                          band_quarters=6, primary_quarters=4)))
    for name, plan in plans:
        note("kv finisher slot layouts plan %s" % name)
        out, st, _ = run_topk(x, ke, k, plan=plan, stats=True)
        assert_exact(out, x, ke, k)
        note("routes %s" % st)


def test_small_boundary_group_with_ties():
    """When the boundary digit group shrinks to at most 64 entries, one wave
    orders it by full key; copies of the K-th value straddling the boundary
    must be split exactly (some selected, the rest not)."""
    t = topkf()
    k, n = 2048, 70000
    rng = np.random.default_rng(13)
    x = rng.standard_normal((6, n), dtype=np.float32)
    for r, copies in enumerate((3, 9, 40, 63, 64, 200)):
        v = np.sort(x[r])[::-1][k - 1]              # the K-th value
        pos = rng.choice(n, copies, replace=False)
        x[r, pos] = v                                # ties across the boundary
    ke = np.full(6, n, dtype=np.int32)
    for name, plan in (("persistent", t.make_plan(t.FAMILY_PERSISTENT, 128, 1, workers=6,
                                                  band_quarters=10, primary_quarters=7)),
                       ("kv-p4", t.make_plan(t.FAMILY_KVSPLIT, 128, 0, splits=4,
                                             min_segment=4096, primary_quarters=8)),
                       ("exact", t.make_plan(t.FAMILY_PERSISTENT, 0, 0, workers=3))):
        note("small boundary group plan %s" % name)
        out, _, _ = run_topk(x, ke, k, plan=plan)
        assert_exact(out, x, ke, k)


def test_cooperative_exact_route():
    """KV-split without a view: each part histograms its segment, the row's
    histograms merge in the counter buffer, the parts commit and collect the
    boundary bin, one workgroup per row refines.  Long i.i.d., ascending,
    constant and tied rows, short and sentinel rows, clamped live rows; the
    counters (including the merged histograms) must be zero after each call,
    and a second call on the same buffers must be exact too."""
    import torch
    from tests.gpu_util import dev
    t = topkf()
    k, n = 2048, 300000
    rng = np.random.default_rng(14)
    x = rng.standard_normal((8, n), dtype=np.float32)
    x[1] = np.sort(x[1])                                   # tail in the last segment
    x[2] = np.float32(0.75)                                # every value tied
    x[3] = np.round(x[3] * 4).astype(np.float32) / 4       # heavy ties
    x[4, rng.choice(n, 5000, replace=False)] = np.inf      # +inf flood beyond K
    ke = np.array([n, n - 7, 250000, n, 123457, 3000, 1500, n], dtype=np.int32)
    for name, plan in (("kvx-p8", t.make_plan(t.FAMILY_KVSPLIT, 0, 0, splits=8, min_segment=4096)),
                       ("kvx-p32", t.make_plan(t.FAMILY_KVSPLIT, 0, 0, splits=32, min_segment=8192)),
                       ("kvx-p3", t.make_plan(t.FAMILY_KVSPLIT, 0, 0, splits=3, min_segment=1024))):
        note("cooperative exact route plan %s" % name)
        out, st, _ = run_topk(x, ke, k, plan=plan, stats=True)
        assert_exact(out, x, ke, k)
        assert st["exact_direct"] == 7 and st["sentinel"] == 1, st   # ke = 1500 <= K
        out, st, _ = run_topk(x, ke, k, m_live=5, plan=plan, stats=True)
        assert_exact(out, x, ke, k, m_live=5)
    # Two calls on one set of buffers, the second with other rows.
    plan = t.make_plan(t.FAMILY_KVSPLIT, 0, 0, splits=16, min_segment=4096)
    d = dev()
    sel = t.Selector(8, n, device=d, plan=plan)
    for trial in range(2):
        xt = x if trial == 0 else rng.standard_normal((8, n), dtype=np.float32)
        xd = torch.from_numpy(xt).to(d)
        ke_d = torch.from_numpy(ke).to(d)
        o = torch.full((8, k), -7, dtype=torch.int32, device=d)
        nvr = torch.tensor([8], dtype=torch.int32, device=d)
        note("cooperative exact route reuse, call %d" % trial)
        sel(xd, ke_d, o, nvr, k)
        torch.cuda.synchronize()
        assert int(sel.counters.sum().item()) == 0
        assert_exact(o.cpu().numpy(), xt, ke, k)
