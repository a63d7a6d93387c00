"""Host-side checks of the C ABI library: it loads, exports what include/topkf.h
declares, and its host-only planner behaves.  No GPU compute is launched."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "topkf.h")
LIB = os.path.join(ROOT, "exact_row_wise_sampled_amd", "libtopkf.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\*?\s+\*?\s*([A-Za-z_]\w*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libtopkf.so is not built; run __graft_entry__.build()")
    return ctypes.CDLL(LIB)


def test_header_declares_the_api():
    names = declared_functions()
    for want in ("topk_filtered_workspace_size", "topk_filtered", "topkf_status_string",
                 "topkf_plan_for", "topkf_plan_workspace_size", "topk_filtered_debug",
                 "topkf_coarse_keys", "topkf_read_probe", "topkf_coarse_cutoffs",
                 "topk_filtered_hinted", "topk_filtered_hinted_debug"):
        assert want in names, names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True,
                         text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings():
    from exact_row_wise_sampled_amd import topkf
    assert topkf.status_string(0) == "ok"
    assert "workspace" in topkf.status_string(3)
    assert topkf.status_string(99) == "unknown status"


def test_planner_maps_workload_shapes():
    from exact_row_wise_sampled_amd import topkf
    cus = 256
    tiny = topkf.plan_for(4, 8192, cus)
    assert tiny.family == topkf.FAMILY_PERSISTENT and tiny.stride == 0 and tiny.workers == 4
    prefill = topkf.plan_for(4096, 65536, cus)
    assert prefill.family == topkf.FAMILY_PERSISTENT and prefill.stride == 128
    assert prefill.workers == 2 * cus and prefill.dual == 1
    decode = topkf.plan_for(64, 131072, cus)
    assert decode.family == topkf.FAMILY_KVSPLIT and decode.stride == 128
    assert decode.splits * 64 >= cus
    long_ = topkf.plan_for(4, 524288, cus)
    assert long_.family == topkf.FAMILY_KVSPLIT
    assert long_.splits <= 524288 // long_.min_segment
    mid = topkf.plan_for(1024, 32768, cus)
    assert mid.stride == 128 and mid.family == topkf.FAMILY_PERSISTENT
    assert topkf.plan_for(1024, 12288, cus).stride == 128
    assert topkf.plan_for(1024, 8193, cus).stride == 128
    assert topkf.plan_for(1024, 8192, cus).stride == 0
    # Few rows: one workgroup per row unless the rows are long
    # (N >= 1024 * max(M, 64)).
    for m, n, fam in ((64, 65536, topkf.FAMILY_KVSPLIT), (4, 65536, topkf.FAMILY_KVSPLIT),
                      (4, 32768, topkf.FAMILY_PERSISTENT), (128, 65536, topkf.FAMILY_PERSISTENT),
                      (64, 32768, topkf.FAMILY_PERSISTENT),
                      (4, 131072, topkf.FAMILY_KVSPLIT), (128, 131072, topkf.FAMILY_KVSPLIT),
                      (128, 262144, topkf.FAMILY_KVSPLIT), (256, 65536, topkf.FAMILY_KVSPLIT),
                      (256, 262144, topkf.FAMILY_KVSPLIT), (512, 262144, topkf.FAMILY_PERSISTENT)):
        pl = topkf.plan_for(m, n, cus)
        assert pl.family == fam, (m, n, pl)
        if fam == topkf.FAMILY_PERSISTENT:
            assert pl.workers == min(m, 2 * cus)
    assert long_.splits == 32 and decode.splits == 4
    # parts: half the pool over the rows, at least min(4, 2 pool / M), within
    # the 16K-column segment floor
    assert topkf.plan_for(32, 131072, cus).splits == 8
    assert topkf.plan_for(128, 262144, cus).splits == 4
    assert topkf.plan_for(256, 262144, cus).splits == 4
    assert topkf.plan_for(384, 131072, cus).splits == 3
    assert topkf.plan_for(4, 65536, cus).splits == 4
    # rounded down, so that the grid does not just exceed the CU count
    assert topkf.plan_for(48, 131072, cus).splits == 5
    assert topkf.plan_for(40, 131072, cus).splits == 6
    assert decode.dual == 0 and decode.primary_quarters == 8
    assert prefill.primary_quarters == 8 and prefill.band_quarters == 10


def test_planner_is_deterministic_and_validates():
    from exact_row_wise_sampled_amd import topkf
    a = topkf.plan_for(300, 200000, 256).as_dict()
    b = topkf.plan_for(300, 200000, 256).as_dict()
    assert a == b
    with pytest.raises(topkf.TopkfError):
        topkf.plan_for(-1, 100, 256)
    with pytest.raises(topkf.TopkfError):
        topkf.plan_for(10, 0, 256)
    with pytest.raises(topkf.TopkfError):
        topkf.plan_for(10, 100, 0)


def test_workspace_sizes_follow_the_plan():
    from exact_row_wise_sampled_amd import topkf
    n = 100000
    pers = topkf.make_plan(topkf.FAMILY_PERSISTENT, 128, 1, workers=10)
    cb, wb = topkf.plan_workspace_size(pers, 77, n)
    assert cb == 4 * (64 + 2 * 77)
    sl = n + 128                         # slice of (index, key) pairs
    assert wb == 10 * 2 * sl * 8         # two slices per worker
    kv = topkf.make_plan(topkf.FAMILY_KVSPLIT, 64, 0, splits=8)
    cb, wb = topkf.plan_workspace_size(kv, 5, n)
    assert wb == 5 * (2 * sl * 8 + 4 * 8 * 4)  # two slices per row, four words per part
    assert cb == 4 * (64 + 2 * 5)
    kvx = topkf.make_plan(topkf.FAMILY_KVSPLIT, 0, 0, splits=8)   # cooperative exact route
    cb, wb = topkf.plan_workspace_size(kvx, 5, n)
    assert cb == 4 * (64 + 2 * 5 + 5 * 2048)  # plus one coarse histogram per row
    assert wb == 5 * (2 * sl * 8 + 4 * 8 * 4)
    for bad in (topkf.make_plan(7, 128), topkf.make_plan(1, 32), topkf.make_plan(1, 64, dual=2),
                topkf.make_plan(1, 64, workers=0), topkf.make_plan(2, 64, splits=0),
                topkf.make_plan(2, 64, splits=257),
                topkf.make_plan(2, 64, splits=2, min_segment=0),
                topkf.make_plan(1, 64, 1, workers=2, band_quarters=6),
                topkf.make_plan(1, 64, 0, workers=2, primary_quarters=3),
                topkf.make_plan(1, 128, 1, workers=2, primary_quarters=7, band_quarters=7)):
        with pytest.raises(topkf.TopkfError):
            topkf.plan_workspace_size(bad, 5, n)


def test_hinted_entry_rejects_a_null_hint(lib):
    # Argument check before any device access: a null proposal array with rows.
    c = ctypes
    f = lib.topk_filtered_hinted
    f.restype = c.c_int32
    f.argtypes = [c.c_void_p, c.c_int64, c.c_int64, c.c_int64, c.c_void_p, c.c_void_p,
                  c.c_void_p, c.c_int32, c.c_void_p, c.c_void_p, c.c_size_t, c.c_void_p,
                  c.c_size_t, c.c_void_p]
    fake = 0x1000
    assert f(fake, 4, 100, 100, fake, fake, fake, 8, None, fake, 1 << 20, fake, 1 << 20,
             None) == 1
