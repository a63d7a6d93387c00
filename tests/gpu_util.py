"""Shared helpers of the GPU tests: run the HIP selector through the C ABI on
host-generated inputs and compare with the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np

from oracle import oracle


def dev():
    import torch
    return torch.device("cuda:0")


def note(msg: str) -> None:
    """Names the case about to run on the GPU (flushed, so it survives a crash)."""
    print("[gpu] " + msg, flush=True)
    sys.stdout.flush()


def run_topk(x: np.ndarray, ke: np.ndarray, k: int, m_live: int | None = None, plan=None,
             stats: bool = False, x_dev=None, canary: int = -7, stride_pad: int = 0):
    """Runs topk_filtered (or the debug entry with `plan`) and returns (out, stats, sel).

    stride_pad > 0 stores the rows at a pitch of N + stride_pad elements.
    """
    import torch
    from exact_row_wise_sampled_amd import topkf
    d = dev()
    m, n = x.shape
    if x_dev is None:
        if stride_pad:
            buf = torch.empty((m, n + stride_pad), dtype=torch.float32, device=d)
            buf[:, :n] = torch.from_numpy(x).to(d)
            buf[:, n:] = float("nan")
            x_dev = buf[:, :n]
        else:
            x_dev = torch.from_numpy(np.ascontiguousarray(x)).to(d)
    ke_d = torch.from_numpy(np.ascontiguousarray(ke, dtype=np.int32)).to(d)
    out = torch.full((m, k), canary, dtype=torch.int32, device=d)
    nvr = torch.tensor([m if m_live is None else m_live], dtype=torch.int32, device=d)
    sel = topkf.Selector(m, n, device=d, plan=plan)
    rs = torch.zeros(topkf.ROUTE_COUNT, dtype=torch.int32, device=d) if (stats or plan) else None
    sel(x_dev, ke_d, out, nvr, k, route_stats=rs)
    torch.cuda.synchronize()
    counters_zero = int(sel.counters.sum().item()) == 0
    assert counters_zero, "counters not returned to zero"
    st = None
    if rs is not None:
        st = dict(zip(topkf.ROUTE_NAMES, rs.cpu().numpy().tolist()))
    return out.cpu().numpy(), st, sel


def assert_exact(out: np.ndarray, x: np.ndarray, ke: np.ndarray, k: int, m_live=None,
                 res=None, canary: int = -7) -> None:
    m = x.shape[0]
    if res is None:
        res = oracle.topk(x, ke, k, m_live=m_live)
    fails = oracle.check_rows(out, x, res)
    assert not fails, "\n".join(fails)
    # rows at or beyond M_live are untouched
    if res.rows < m:
        assert (out[res.rows:] == canary).all(), "rows >= M_live were written"


def assert_routes(st: dict, x: np.ndarray, ke: np.ndarray, k: int, plan, m_live=None,
                  hints=None) -> dict:
    """The selector's route counters equal the CPU route model's counts for
    every exclusive route and for the rows whose proposal replaced the view
    (the spill counter is an extra, capacity-dependent tally and is not
    modelled).  `plan` is the plan the call ran with, `hints` its proposals."""
    from oracle import route_model as rm
    pol = rm.Policy(int(plan.stride), bool(plan.dual), int(plan.primary_quarters),
                    int(plan.band_quarters))
    want = rm.route_counts(x, ke, k, pol, m_live=m_live, hints=hints)
    got = {name: int(st[name]) for name in want}
    assert got == want, "routes: selector %s, model %s" % (got, want)
    return want


def auto_plan(m: int, n: int):
    """The plan the library picks on this device for an (M_cap, N) call."""
    import torch
    from exact_row_wise_sampled_amd import topkf
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return topkf.plan_for(m, n, cus)


def view_phase(row: int, s: int) -> int:
    """The row's view residue: log2(s)-bit reversal of row mod s (Eq. 13 reading)."""
    b = s.bit_length() - 1
    r = row % s
    return int(format(r, "0%db" % b)[::-1], 2)


def aliased_rows(s: int, k: int, n: int, m: int, kind: str, seed: int = 0):
    """Rows whose view (residue a_r) sees a misleading tail.

    'band':  q view entries at 100, the next q1-q view entries at 50, and
             enough 50s elsewhere that the secondary boundary certifies.
    'exact': q view entries at 100 and q1-q at 50, all other values small, so
             both boundaries underfill and exact recovery must run.
    """
    rng = np.random.default_rng(seed)
    cdiv = lambda a, b: -(-a // b)
    q = cdiv(cdiv(3 * k, 2), s)
    q1 = cdiv(cdiv(7 * k, 4), s)
    x = (rng.standard_normal((m, n)) * 0.1).astype(np.float32)
    for r in range(m):
        a = view_phase(r, s)
        view = np.arange(a, n, s)
        x[r, view[:q]] = 100.0 + rng.random(q).astype(np.float32)
        x[r, view[q:q1]] = 50.0 + rng.random(q1 - q).astype(np.float32)
        if kind == "band":
            others = np.setdiff1d(np.arange(n), view)
            pick = rng.choice(others, size=2 * k, replace=False)
            x[r, pick] = 50.0 + rng.random(2 * k).astype(np.float32)
    ke = np.full(m, n, dtype=np.int32)
    return x, ke
