"""ABI behaviour on the GPU: argument errors, counter restoration, live-row
bounds, length clamping, padded pitches, graph capture and replay."""
import numpy as np
import pytest

from exact_row_wise_sampled_amd import workloads as W
from tests.gpu_util import assert_exact, dev, note, run_topk

pytestmark = pytest.mark.gpu


def T():
    from exact_row_wise_sampled_amd import topkf
    return topkf


def test_argument_errors():
    import torch
    t = T()
    d = dev()
    x = torch.zeros((4, 100), dtype=torch.float32, device=d)
    ke = torch.full((4,), 100, dtype=torch.int32, device=d)
    out = torch.zeros((4, 8), dtype=torch.int32, device=d)
    nvr = torch.tensor([4], dtype=torch.int32, device=d)
    cb, wb = t.topk_filtered_workspace_size(4, 100)
    cnt = torch.zeros(cb, dtype=torch.uint8, device=d)
    ws = torch.empty(wb, dtype=torch.uint8, device=d)
    lib = t._lib
    st = torch.cuda.current_stream().cuda_stream
    call = lambda **kw: lib.topk_filtered(
        kw.get("x", x.data_ptr()), kw.get("m", 4), kw.get("n", 100), kw.get("stride", 100),
        kw.get("ke", ke.data_ptr()), kw.get("out", out.data_ptr()), kw.get("nvr", nvr.data_ptr()),
        kw.get("k", 8), kw.get("cnt", cnt.data_ptr()), kw.get("cb", cb), kw.get("ws", ws.data_ptr()),
        kw.get("wb", wb), st)
    assert call() == 0
    assert call(k=0) == 1 and call(k=2049) == 1
    assert call(stride=99) == 1 and call(n=0) == 1 and call(m=-1) == 1
    assert call(x=None) == 1 and call(ke=None) == 1 and call(out=None) == 1
    assert call(nvr=None) == 1 and call(cnt=None) == 1
    assert call(cb=cb - 1) == 3 and call(wb=wb - 1) == 3
    assert call(m=0, x=None, ke=None, out=None, nvr=None, cnt=None) == 0
    torch.cuda.synchronize()
    assert int(cnt.sum()) == 0


def test_live_rows_and_length_clamping():
    k = 64
    x = W.iid_normal(3, 10, 5000, [5000] * 10, k).x
    ke = np.array([-3, 0, 64, 65, 5000, 9999, 4999, 100, 2, 70], dtype=np.int32)
    for m_live in (0, 1, 6, 10, 11, -5):
        note("live rows %d" % m_live)
        out, _, _ = run_topk(x, ke, k, m_live=m_live)
        assert_exact(out, x, ke, k, m_live=m_live)


@pytest.mark.parametrize("pad", [1, 3, 4, 37])
def test_padded_and_unaligned_pitch(pad):
    w = W.decode(seed=21, m=9, n=30001, lo=2000)
    for name, plan in (("auto", None),
                       ("kv", T().make_plan(T().FAMILY_KVSPLIT, 64, 1, splits=5, min_segment=1000)),
                       ("pers", T().make_plan(T().FAMILY_PERSISTENT, 128, 1, workers=3))):
        note("pitch pad %d plan %s" % (pad, name))
        out, _, _ = run_topk(w.x, w.ke, w.k, stride_pad=pad, plan=plan)
        assert_exact(out, w.x, w.ke, w.k)


def test_counters_zero_after_every_call_and_reuse():
    import torch
    t = T()
    d = dev()
    w = W.decode(seed=5, m=16, n=65536, lo=4096)
    x = torch.from_numpy(w.x).to(d)
    ke = torch.from_numpy(w.ke).to(d)
    out = torch.zeros((w.m, w.k), dtype=torch.int32, device=d)
    nvr = torch.tensor([w.m], dtype=torch.int32, device=d)
    for plan in (None, t.make_plan(t.FAMILY_PERSISTENT, 128, 1, workers=5),
                 t.make_plan(t.FAMILY_KVSPLIT, 128, 1, splits=7, min_segment=2048)):
        sel = t.Selector(w.m, w.n, device=d, plan=plan)
        for rep in range(5):
            sel(x, ke, out, nvr, w.k)
            torch.cuda.synchronize()
            assert int(sel.counters.sum()) == 0
            assert_exact(out.cpu().numpy(), w.x, w.ke, w.k)


def test_graph_capture_and_replay_with_mutated_inputs():
    """Live rows and lengths stay on the device, so one captured call serves
    every replay; the counters return to zero after each replay."""
    import torch
    t = T()
    d = dev()
    m, n, k = 32, 65536, 2048
    rng = np.random.default_rng(77)
    # every column valid, so any mutated length selects from real scores
    w = W.decode(seed=8, m=m, n=n, lo=n)
    x = torch.from_numpy(w.x).to(d)
    ke = torch.from_numpy(w.ke).to(d)
    out = torch.full((m, k), -7, dtype=torch.int32, device=d)
    nvr = torch.tensor([m], dtype=torch.int32, device=d)
    for plan in (None, t.make_plan(t.FAMILY_PERSISTENT, 64, 1, workers=6)):
        sel = t.Selector(m, n, device=d, plan=plan)
        s = torch.cuda.Stream(device=d)
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            sel(x, ke, out, nvr, k, stream=s)   # warm-up outside the graph
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            sel(x, ke, out, nvr, k, stream=s)
        for rep in range(6):
            new_ke = rng.integers(0, n + 1, size=m).astype(np.int32)
            new_ke[:3] = [k, k + 1, 0]
            live = int(rng.integers(0, m + 1)) if rep % 2 else m
            ke.copy_(torch.from_numpy(new_ke))
            nvr.fill_(live)
            out.fill_(-7)
            torch.cuda.synchronize()
            note("graph replay %d live=%d" % (rep, live))
            g.replay()
            torch.cuda.synchronize()
            assert int(sel.counters.sum()) == 0
            assert_exact(out.cpu().numpy(), w.x, new_ke, k, m_live=live)


def test_nan_in_padding_never_read():
    # workloads fill columns past ke with NaN/+inf garbage; the adversarial
    # rows also end well before N.  Explicitly plant +inf right after ke.
    w = W.decode(seed=30, m=12, n=40000, lo=5000)
    for r in range(w.m):
        w.x[r, w.ke[r]:w.ke[r] + 64] = np.inf
    out, _, _ = run_topk(w.x, w.ke, w.k)
    assert_exact(out, w.x, w.ke, w.k)


def test_coarse_keys_match_ieee_fp16():
    """Eq. 11 on the device against numpy's IEEE round-to-nearest-even FP16."""
    import torch
    t = T()
    d = dev()
    rng = np.random.default_rng(1)
    bits = np.concatenate([
        rng.integers(0, 2**32, size=1 << 22, dtype=np.uint64).astype(np.uint32),
        np.arange(0x477FE000, 0x47800100, dtype=np.uint32),        # around 65504..65536
        np.arange(0x33000000 - 4096, 0x33000000 + 4096, dtype=np.uint32),  # fp16 min subnormal
        np.arange(0x387FF000, 0x38801000, dtype=np.uint32),        # fp16 min normal
        np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 1, 0x80000001], dtype=np.uint32),
    ])
    bits = bits[(bits & 0x7F800000) != 0x7F800000 | ((bits & 0x007FFFFF) == 0)]
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    xd = torch.from_numpy(x.copy()).to(d)
    kd = torch.empty(x.size, dtype=torch.int16, device=d)
    t.coarse_keys(xd, kd)
    torch.cuda.synchronize()
    got = kd.cpu().numpy().view(np.uint16).astype(np.uint32)
    with np.errstate(over="ignore"):
        h = x.astype(np.float16).view(np.uint16).astype(np.uint32)
    k16 = np.where(h & 0x8000, h, h ^ 0x7FFF)
    want = k16 >> 5
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, "first mismatch x=%r got %d want %d" % (x[bad[0]], got[bad[0]], want[bad[0]])
    assert want[x == np.inf].tolist() == [31] * int((x == np.inf).sum())


def test_coarse_keys_exhaustive():
    """Eq. 11 on the device for every float32 bit pattern (NaNs excluded), in
    chunks of 2^28, against the C oracle's IEEE round-to-nearest-even binary16
    conversion on the host CPU (itself pinned to numpy's conversion)."""
    import torch
    from oracle import oracle
    t = T()
    d = dev()
    chunk = 1 << 28
    base = torch.arange(chunk, dtype=torch.int64, device=d)
    kd = torch.empty(chunk, dtype=torch.int16, device=d)
    host = torch.empty(chunk, dtype=torch.int16, pin_memory=True)
    for c in range((1 << 32) // chunk):
        start = c * chunk
        v = base + start
        pats = torch.where(v >= 1 << 31, v - (1 << 32), v).to(torch.int32)
        del v
        t.coarse_keys(pats.view(torch.float32), kd)
        host.copy_(kd)
        torch.cuda.synchronize()
        del pats
        try:
            bad, first = oracle.coarse_check(start, host.numpy().view(np.uint16))
        except RuntimeError as e:
            pytest.skip(str(e))
        note("coarse keys patterns [%#010x, %#010x): %d mismatches" % (start, start + chunk, bad))
        assert bad == 0, "first mismatch at pattern %#010x" % first


def test_read_probe():
    """The streaming-read reference: validates alignment and size, reads a
    buffer without writing its sink for ordinary data."""
    import torch
    from exact_row_wise_sampled_amd import topkf
    from tests.gpu_util import dev
    d = dev()
    x = torch.ones(1 << 20, dtype=torch.float32, device=d)
    sink = torch.zeros(1, dtype=torch.int32, device=d)
    topkf.read_probe(x, sink)
    topkf.read_probe(x[:4], sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    with pytest.raises(topkf.TopkfError):
        topkf.read_probe(x[1:5], sink)   # 4-byte offset: not 16-byte aligned
    with pytest.raises(topkf.TopkfError):
        topkf.read_probe(x[:3], sink)    # 12 bytes: not a multiple of 16


def test_cutoff_table_matches_search_and_ieee():
    """The compile-time cutoff table T(tau) equals the device's search over
    the hardware FP16 conversion for every coarse bin, and numpy's IEEE FP16
    conversion confirms it is the last key of bin <= tau (paper Sec. 4.3)."""
    import torch
    from exact_row_wise_sampled_amd import topkf
    from tests.gpu_util import dev
    d = dev()
    table = torch.zeros(2048, dtype=torch.int32, device=d)
    search = torch.zeros(2048, dtype=torch.int32, device=d)
    topkf.coarse_cutoffs(table, search)
    torch.cuda.synchronize()
    tab = table.cpu().numpy().view(np.uint32)
    sea = search.cpu().numpy().view(np.uint32)
    assert np.array_equal(tab, sea), np.nonzero(tab != sea)[0][:10]

    def coarse_of_keys(k):
        k = k.astype(np.uint32)
        b = np.where(k & np.uint32(0x80000000), k, k ^ np.uint32(0x7FFFFFFF)).astype(np.uint32)
        with np.errstate(over="ignore"):
            h = b.view(np.float32).astype(np.float16).view(np.uint16).astype(np.uint32)
        return np.where(h & 0x8000, h, h ^ 0x7FFF) >> 5

    tau = np.arange(2048, dtype=np.uint32)
    none = tab == 0x007FFFFE          # even +inf lies above tau
    full = tab == 0xFF800000          # every non-NaN value is admitted
    assert np.all(coarse_of_keys(np.array([0x007FFFFF]))[0] > tau[none])
    mid = ~none & ~full
    assert np.all(coarse_of_keys(tab[mid]) <= tau[mid])
    assert np.all(coarse_of_keys(tab[mid] + 1) > tau[mid])
    assert np.all(coarse_of_keys(tab[full]) <= tau[full])
    assert np.all(np.diff(tab.astype(np.int64)) >= 0)   # monotone in tau
