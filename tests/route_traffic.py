"""Forced-route inputs for the score-read counters of "Sample-Guided Exact
Top-K Selection for Long-Context Sparse Attention", Sec. 4.6 (Table 2 "Score
reads", Eq. 29).  Not a test: run it under rocprofv3 with FETCH_SIZE (then
WRITE_SIZE) to measure the HBM bytes each route reads per valid score, e.g.

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT -o pmc -- \
        python3 tests/route_traffic.py --case band --copy-probe

Every case is 512 rows x 65536 columns (all valid), K = 2048, one persistent
workgroup per row, the view at s = 128 with the pages' K~ = 1.5K / K~1 = 1.75K
boundaries; rows are built so that each one takes the named route (the
route counters of the first call are printed to confirm it):

  primary              i.i.d. N(0, 0.1) rows, certified at tau0      1 + 1/s
  band                 the view's tail misleads tau0, tau1 certifies 2 + 1/s
  exact_after_band     both boundaries underfill (dual plan)         4 + 1/s
  exact_after_primary  tau0 underfills, no band (plan without it)    3 + 1/s
  direct_exact         the plan without a view: exact coarse route   2

Reads of the view (1/s of the row's values, but one cache line per sample)
come from lines the scans read again, so on the counters they show up only
through the L2 hit rate.  --copy-probe runs one plain 256 MiB device copy
first: the calibration reference for the counters.
"""
from __future__ import annotations

import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

CASES = {
    # name: (aliased-row kind or None for i.i.d. rows, stride, dual)
    "primary": (None, 128, 1),
    "band": ("band", 128, 1),
    "exact_after_band": ("exact", 128, 1),
    "exact_after_primary": ("exact", 128, 0),
    "direct_exact": (None, 0, 0),
}
EXPECTED_READS = {"primary": "1 + 1/s", "band": "2 + 1/s", "exact_after_band": "4 + 1/s",
                  "exact_after_primary": "3 + 1/s", "direct_exact": "2"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--case", required=True, choices=sorted(CASES))
    ap.add_argument("--rows", type=int, default=512)
    ap.add_argument("--cols", type=int, default=65536)
    ap.add_argument("--calls", type=int, default=8)
    ap.add_argument("--copy-probe", action="store_true")
    args = ap.parse_args()

    import numpy as np
    import torch

    from exact_row_wise_sampled_amd import topkf
    from tests.gpu_util import aliased_rows

    dev = torch.device("cuda:0")
    if args.copy_probe:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    kind, s, dual = CASES[args.case]
    k, m, n = 2048, args.rows, args.cols
    if kind is None:
        rng = np.random.default_rng(3)
        x = (rng.standard_normal((m, n)) * 0.1).astype(np.float32)
        ke = np.full(m, n, dtype=np.int32)
    else:
        x, ke = aliased_rows(128, k, n, m, kind, seed=4)
    plan = topkf.make_plan(topkf.FAMILY_PERSISTENT, s, dual, workers=m)
    xd = torch.from_numpy(x).to(dev)
    ked = torch.from_numpy(ke).to(dev)
    out = torch.empty((m, k), dtype=torch.int32, device=dev)
    nvr = torch.tensor([m], dtype=torch.int32, device=dev)
    sel = topkf.Selector(m, n, device=dev, plan=plan)
    rs = torch.zeros(topkf.ROUTE_COUNT, dtype=torch.int32, device=dev)
    sel(xd, ked, out, nvr, k, route_stats=rs)
    torch.cuda.synchronize()
    routes = {name: v for name, v in zip(topkf.ROUTE_NAMES, rs.cpu().tolist()) if v}
    for _ in range(args.calls):
        sel(xd, ked, out, nvr, k)
    torch.cuda.synchronize()
    print(json.dumps({"case": args.case, "rows": m, "cols": n, "k": k, "stride": s, "dual": dual,
                      "score_bytes": int(4 * ke.astype(np.int64).sum()), "calls": args.calls + 1,
                      "routes_first_call": routes, "expected_reads": EXPECTED_READS[args.case]}),
          flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
