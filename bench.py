"""Throughput of the exact row-wise Top-K selector on one MI355X.

One step is one topk_filtered call over one batch of synthetic score rows
(every phase of the selector runs inside it).  Inputs are resident in HBM
before timing starts.  Calls are captured in a HIP graph over R rotated copies
of the batch (R chosen so the copies span at least twice the 256 MB
last-level cache, so replays stream from HBM), then replayed.  The timed
region is exactly --steps calls, bracketed by device synchronisation, timed
with HIP events on the stream the graph runs on.

Prints one JSON line: effective score-row GB/s (sum over rows of 4*ke bytes per
second) with rows/s, the roofline of the selector kernel and the CPU oracle's
rate on the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20

DESCRIPTIONS = {
    "tiny": "tiny: M=4, N=8192, ke=[8192,6000,3000,1024], K=256, iid N(0,1)",
    "decode": "decode indexer: M=64, N=131072, ke~U[32768,131072], K=2048, "
              "8-head ReLU-weighted scores",
    "prefill": "causal prefill: M=4096, N=65536, ke=min(61440+r+1,N), K=2048, "
               "8-head ReLU-weighted scores",
    "long": "few long rows: M=4, N=524288, ke=N, K=2048, ReLU scores + 0.1% +3sigma spikes",
    "adversarial": "adversarial: M=256, N=262144, ke~U[4096,N], K=2048, ties/sorted/"
                   "constant/+-inf rows",
}


def algorithmic_bytes(ke, n: int, k: int, stride: int) -> int:
    """Bytes the selector must move per call: one complete read of every valid
    row, the 1/s view, and the K int32 outputs per row."""
    total = 0
    for L in ke:
        L = min(max(int(L), 0), n)
        if L > k:
            view = math.ceil(L / stride) if stride else 0
            total += 4 * L + 4 * view
        total += 4 * k
    return total


def measured_traffic(config: str):
    """HBM bytes per call from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    (profiles/hbm_traffic.json, calibrated against a plain device copy), or None
    when they were taken on a different kernel source than the one built here."""
    import hashlib
    src = os.path.join(ROOT, "exact_row_wise_sampled_amd", "csrc", "topkf.hip")
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        rec = json.load(open(path))
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256_16") != digest:
        return None
    cfg = rec.get("configs", {}).get(config)
    return None if cfg is None else int(cfg["traffic_bytes"])


def stream_read_reference(dev, nbytes: int = 1 << 30) -> float:
    """GB/s of the library's plain 128-bit streaming-read kernel over nbytes
    (topkf_read_probe, the same loads the selector streams with): the
    achievable-bandwidth reference for the selector's score-row GB/s."""
    import torch
    from exact_row_wise_sampled_amd import topkf
    x = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    for _ in range(3):
        topkf.read_probe(x, sink)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        topkf.read_probe(x, sink)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    del x
    return nbytes / (ms * 1e-3) / 1e9


def cpu_baseline(w, seconds: float) -> dict:
    """The CPU oracle (complete sort per row, threaded over rows) on the same batch."""
    from oracle import oracle
    threads = oracle.default_threads()
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.topk(w.x, w.ke, w.k, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 10000:
            break
    per_call = el / reps
    return {"value": round(w.score_bytes() / per_call / 1e9, 4), "unit": "GB/s",
            "rows_per_s": round(w.m / per_call, 1), "cores": threads, "kind": "oracle",
            "sample": "whole %s batch (%d rows) x %d repetitions, %.1f s wall on %d threads "
                      "(%.0f thread-seconds)" % (w.name, w.m, reps, el, threads, el * threads)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--config", default="decode", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall time of the CPU oracle baseline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch every call directly instead of replaying a HIP graph "
                         "(for hardware-counter runs)")
    ap.add_argument("--no-ref", action="store_true", help="skip the streaming-read reference")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one plain 256 MiB device copy first, the calibration "
                         "reference for FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the selector has no multi-GPU path "
              "(rows are independent; see the sharding note in DESIGN.md)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from exact_row_wise_sampled_amd import topkf, workloads

    dev = torch.device("cuda:0")
    if args.copy_probe:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w = workloads.make(args.config)
    m, n, k = w.m, w.n, w.k
    plan = topkf.plan_for(m, n, torch.cuda.get_device_properties(dev).multi_processor_count)
    x_bytes = m * n * 4
    copies = max(2, math.ceil(2 * MALL_BYTES / x_bytes))
    base = torch.from_numpy(w.x).to(dev)
    xs = [base] + [base.clone() for _ in range(copies - 1)]
    ke = torch.from_numpy(w.ke).to(dev)
    nvr = torch.tensor([m], dtype=torch.int32, device=dev)
    outs = [torch.empty((m, k), dtype=torch.int32, device=dev) for _ in range(copies)]
    sel = topkf.Selector(m, n, device=dev)
    torch.cuda.synchronize()

    if not args.no_check:
        from oracle import oracle
        sel(xs[-1], ke, outs[-1], nvr, k)
        torch.cuda.synchronize()
        res = oracle.topk(w.x, w.ke, k)
        fails = oracle.check_rows(outs[-1].cpu().numpy(), w.x, res)
        if fails:
            print("bench: output differs from the oracle: %s" % fails, file=sys.stderr)
            return 1
        print("bench: %s output matches the oracle (%d rows)" % (w.name, m), file=sys.stderr,
              flush=True)

    stream = torch.cuda.Stream(device=dev)
    stream.wait_stream(torch.cuda.current_stream())

    def one_pass():
        for i in range(copies):
            sel(xs[i], ke, outs[i], nvr, k, stream=stream)

    with torch.cuda.stream(stream):
        one_pass()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    if args.eager:
        replay = one_pass
    else:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            one_pass()
        torch.cuda.synchronize()
        replay = graph.replay

    reps_warm = max(1, math.ceil(args.warmup / copies))
    reps = max(1, math.ceil(args.steps / copies))
    steps = reps * copies
    with torch.cuda.stream(stream):
        for _ in range(reps_warm):
            replay()
    torch.cuda.synchronize()
    if int(sel.counters.sum().item()) != 0:
        print("bench: counters not zero after replays", file=sys.stderr)
        return 1

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        ev0.record(stream)
        for _ in range(reps):
            replay()
        ev1.record(stream)
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / steps

    score_bytes = w.score_bytes()
    gbs = score_bytes / (ms_step * 1e-3) / 1e9
    alg = algorithmic_bytes(w.ke, n, k, plan.stride)
    achieved = alg / (ms_step * 1e-3) / 1e9
    kernels = (["persistent_kernel<%d,%s>" % (plan.stride, "true" if plan.dual else "false")]
               if plan.family == 1 else
               ["kvsplit_scan_kernel<%d,%s>" % (plan.stride, "true" if plan.dual else "false"),
                "kvsplit_finish_kernel<%d,%s>" % (plan.stride, "true" if plan.dual else "false")])
    traffic = measured_traffic(args.config)
    line = {
        "metric": "score-row GB/s and rows/s vs HBM peak, K=2048, ragged rows up to 512K",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "rows_per_s": round(m / (ms_step * 1e-3), 1),
        "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
        "n_gpus": 1,
        "steps": steps,
        "warmup": reps_warm * copies,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": DESCRIPTIONS[args.config], "M": m, "N": n, "K": k,
                   "score_bytes": score_bytes, "rotated_copies": copies,
                   "plan": plan.as_dict()},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": alg,
                     "kernels": kernels,
                     "timing": "achieved = algorithmic bytes / ms_per_step; one call runs "
                               "every listed kernel"},
    }
    if not args.no_ref:
        ref = stream_read_reference(dev)
        line["stream_read_ref_gbs"] = round(ref, 1)
        line["stream_read_ref_frac"] = round(gbs / ref, 4)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
