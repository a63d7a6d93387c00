"""topk_filtered_noalloc (the entry point for callers that cannot allocate):
called through the C ABI twice in a row, the second time on a smaller input,
and checked against topk_filtered on the same inputs (both exact against the
CPU oracle, with the same selected value multiset per row); the worker
narrowing when the automatic plan's workspace exceeds the library's device
array; and the size limits, which return an error without launching."""
import numpy as np
import pytest

from exact_row_wise_sampled_amd import workloads as W
from oracle import oracle
from tests.gpu_util import dev, note

pytestmark = pytest.mark.gpu


def T():
    from exact_row_wise_sampled_amd import topkf
    return topkf


def _both(w, canary=-7):
    """Runs topk_filtered_noalloc, then topk_filtered, on the same device input."""
    import torch
    t = T()
    d = dev()
    x = torch.from_numpy(w.x).to(d)
    ke = torch.from_numpy(w.ke).to(d)
    nvr = torch.tensor([w.m], dtype=torch.int32, device=d)
    out_na = torch.full((w.m, w.k), canary, dtype=torch.int32, device=d)
    out_ref = torch.full((w.m, w.k), canary, dtype=torch.int32, device=d)
    t.topk_filtered_noalloc(x, ke, out_na, nvr, w.k)
    sel = t.Selector(w.m, w.n, device=d)
    sel(x, ke, out_ref, nvr, w.k)
    torch.cuda.synchronize()
    assert int(sel.counters.sum().item()) == 0
    return out_na.cpu().numpy(), out_ref.cpu().numpy()


def _check_pair(w, out_na, out_ref):
    res = oracle.topk(w.x, w.ke, w.k)
    fails = oracle.check_rows(out_na, w.x, res)
    assert not fails, "noalloc: " + "\n".join(fails)
    fails = oracle.check_rows(out_ref, w.x, res)
    assert not fails, "topk_filtered: " + "\n".join(fails)
    for r in range(w.m):
        L = int(min(max(int(w.ke[r]), 0), w.n))
        if L <= w.k:
            assert np.array_equal(out_na[r], out_ref[r])
            continue
        bits = w.x[r, :L].view(np.uint32)
        assert np.array_equal(np.sort(bits[out_na[r]]), np.sort(bits[out_ref[r]])), r


def test_noalloc_two_calls_second_smaller():
    # first a KV-split shape (decode rows), then a smaller persistent one
    w1 = W.decode(seed=71, m=64, n=131072)
    note("noalloc decode 64 x 131072")
    _check_pair(w1, *_both(w1))
    w2 = W.prefill(seed=72, m=8, n=32768, first=30000)
    note("noalloc prefill 8 x 32768")
    _check_pair(w2, *_both(w2))


def test_noalloc_narrowed_workers_then_smaller():
    # 1024 rows of 64K: the automatic plan's 512 workers need more workspace
    # than the device array holds, so fewer workers take the rows
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan = T().plan_for(1024, 65536, cus)
    _, wb = T().plan_workspace_size(plan, 1024, 65536)
    assert wb > T().NOALLOC_SCRATCH_BYTES - (1 << 20)
    w1 = W.prefill(seed=73, m=1024, n=65536)
    note("noalloc prefill 1024 x 65536 (narrowed pool)")
    _check_pair(w1, *_both(w1))
    w2 = W.adversarial(seed=74, m=32, n=40000, lo=100)
    note("noalloc adversarial 32 x 40000")
    _check_pair(w2, *_both(w2))
    w3 = W.tiny(seed=75)
    note("noalloc tiny")
    _check_pair(w3, *_both(w3))


def test_noalloc_limits_and_errors():
    import torch
    t = T()
    d = dev()
    lib = t._lib
    st = torch.cuda.current_stream().cuda_stream
    x = torch.zeros((4, 100), dtype=torch.float32, device=d)
    ke = torch.full((4,), 100, dtype=torch.int32, device=d)
    out = torch.zeros((4, 8), dtype=torch.int32, device=d)
    nvr = torch.tensor([4], dtype=torch.int32, device=d)

    def call(**kw):
        return lib.topk_filtered_noalloc(
            kw.get("x", x.data_ptr()), kw.get("m", 4), kw.get("n", 100), kw.get("stride", 100),
            kw.get("ke", ke.data_ptr()), kw.get("out", out.data_ptr()),
            kw.get("nvr", nvr.data_ptr()), kw.get("k", 8), st)
    assert call(k=0) == 1 and call(k=2049) == 1
    assert call(stride=99) == 1 and call(n=0) == 1 and call(m=-1) == 1
    assert call(x=None) == 1 and call(ke=None) == 1 and call(out=None) == 1
    assert call(nvr=None) == 1
    assert call(m=0, x=None, ke=None, out=None, nvr=None) == 0
    # beyond the device array: too many rows for the counter part, a row too
    # wide for one worker's workspace (pointers are not read: nothing launches)
    assert call(m=131041, n=16, stride=16) == 3
    assert call(m=1, n=16711553, stride=16711553) == 3
    assert call() == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    for r in range(4):  # all-zero rows: any 8 distinct valid indices
        assert o[r].min() >= 0 and o[r].max() < 100 and np.unique(o[r]).size == 8
