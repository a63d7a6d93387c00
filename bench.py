"""Throughput of the exact row-wise Top-K selector on one MI355X.

One step is one topk_filtered call over one batch of synthetic score rows
(every phase of the selector runs inside it).  Inputs are resident in HBM
before timing starts.  Timing follows the protocol of "Sample-Guided Exact
Top-K Selection for Long-Context Sparse Attention", Sec. 6.1 ("Timing
protocol"): calls are captured in HIP graphs and replayed on one stream,
each call on the next of R rotated copies of the batch (R chosen so the
copies span at least twice the 256 MB last-level cache, so calls stream from
HBM); after the warm-up calls, the timed calls are split into rounds (seven
by default), each round's mean per-call time is taken from HIP events on
the graphs' stream, and the per-call time is the median of the round means.
Exactly --warmup calls run before and exactly --steps calls inside the timed
region.  The defaults (--warmup 110, --steps 700) are the pages' 10 warm-ups
plus two 50-call conditioning sweeps, and seven rounds of 100 calls; a round
holds at least 10 calls (fewer rounds when --steps is small), since every
graph launch adds a gap on the GPU.  Right before the warm-up calls the GPU
streams a separate 256 MiB buffer through the library's read probe for about
20 ms, and the probe, the warm-up and the timed calls are queued back to back
with no host synchronisation between them: the first ~10 ms of load after a
pause run several per cent slower on this GPU (measured: 236 then 232 us per
prefill call over the first 40 calls, 223 us afterwards), and the pages'
conditioning sweeps serve the same purpose.

The headline line is the causal-prefill workload (4096 rows of about 64K
scores, the largest of the five configurations); the same line carries every
configuration's figures under "per_config", each timed with the same
protocol and checked against the CPU oracle outside the timed region.

Prints one JSON line: effective score-row GB/s (sum over rows of 4*ke bytes per
second) with rows/s, the roofline of the selector kernel and the CPU oracle's
rate on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
CPU_SHARE = 16  # host threads one GPU's share of the host may use
MIN_ROUND_CALLS = 10  # calls per timed round (one graph launch each) at the least
CONDITION_MS = 20.0  # GPU time of streaming reads right before each warm-up

_probe = {}


def condition(dev, stream) -> None:
    """Queues about CONDITION_MS of plain streaming reads of a separate 256 MiB
    buffer (topkf_read_probe) on `stream`, without waiting for them."""
    import torch
    from exact_row_wise_sampled_amd import topkf
    if "x" not in _probe:
        _probe["x"] = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        _probe["sink"] = torch.zeros(1, dtype=torch.int32, device=dev)
        _probe["calls"] = None
    x, sink = _probe["x"], _probe["sink"]
    if _probe["calls"] is None:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        for _ in range(20):
            topkf.read_probe(x, sink, stream=stream)
        e0.record(stream)
        for _ in range(20):
            topkf.read_probe(x, sink, stream=stream)
        e1.record(stream)
        stream.synchronize()
        per = max(e0.elapsed_time(e1) / 20, 1e-3)
        _probe["calls"] = max(1, int(CONDITION_MS / per))
    for _ in range(_probe["calls"]):
        topkf.read_probe(x, sink, stream=stream)

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
ORDER = ("prefill", "decode", "long", "adversarial", "tiny")


def algorithmic_bytes(ke, n: int, k: int, stride: int, parts: int = 1) -> int:
    """Bytes the selector must move per call: one complete read of every valid
    row, its 1/s view (read by each of the `parts` workgroups that split the
    row), and the K int32 outputs per row."""
    total = 0
    for L in ke:
        L = min(max(int(L), 0), n)
        if L > k:
            view = math.ceil(L / stride) if stride else 0
            total += 4 * L + 4 * view * max(1, parts)
        total += 4 * k
    return total


def source_digest() -> str:
    """Digest of the kernel source's code: its lines with // comments and
    surrounding blanks removed, empty lines dropped (an edit of comments alone
    keeps the digest)."""
    src = os.path.join(ROOT, "exact_row_wise_sampled_amd", "csrc", "topkf.hip")
    code = []
    for line in open(src, encoding="utf-8"):
        cut = line.split("//", 1)[0].strip()
        if cut:
            code.append(cut)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def measured_traffic(config: str):
    """HBM bytes per call from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    (profiles/hbm_traffic.json, calibrated against a plain device copy), or None
    when they were taken on a different kernel source than the one built here."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        rec = json.load(open(path))
        digest = source_digest()
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256_16") != digest:
        return None
    return rec.get("configs", {}).get(config)


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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def usable_cpus() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def oracle_rate(w, rows: int, seconds: float, threads: int) -> dict:
    """The CPU oracle (complete sort of every valid prefix, threaded over rows)
    on the first `rows` rows of the batch, repeated for about `seconds`."""
    import numpy as np
    from oracle import oracle
    x = np.ascontiguousarray(w.x[:rows])
    ke = np.ascontiguousarray(w.ke[:rows])
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.topk(x, ke, w.k, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 10000:
            break
    per_batch = el / reps
    sb = int(4 * np.clip(ke.astype(np.int64), 0, w.n).sum())
    return {"value": round(sb / per_batch / 1e9, 4), "unit": "GB/s",
            "rows_per_s": round(rows / per_batch, 1), "threads": threads,
            "sample": "%d of %d %s rows x %d repetitions, %.1f s wall" % (
                rows, w.m, w.name, reps, el)}


def cpu_baseline(w, seconds: float, small: dict) -> dict:
    """The oracle on the host cores this process may use (at most one GPU's
    share of the host), on a bounded sample of the headline batch; plus
    one-thread figures on the small workloads."""
    threads = max(1, min(usable_cpus(), CPU_SHARE))
    rows = w.m
    if w.name == "prefill":
        rows = min(w.m, 64 * threads)  # about 0.6 s of sorting per repetition
    r = oracle_rate(w, rows, seconds, threads)
    out = {"value": r["value"], "unit": "GB/s", "rows_per_s": r["rows_per_s"],
           "cores": threads, "kind": "oracle",
           "sample": r["sample"] + " on %d threads" % threads,
           "host_cpus": os.cpu_count(), "usable_cpus": usable_cpus(),
           "cpu_model": cpu_model(),
           "note": "threads = the cores this process may use, capped at the %d-thread "
                   "host share of one GPU" % CPU_SHARE}
    one = {}
    for name, wl in small.items():
        r1 = oracle_rate(wl, wl.m, min(3.0, seconds), 1)
        one[name] = {"value": r1["value"], "unit": "GB/s", "rows_per_s": r1["rows_per_s"],
                     "sample": r1["sample"]}
    if one:
        out["one_thread"] = one
    return out


class Runner:
    """Timed calls of one workload: R rotated copies of the batch in HBM, calls
    captured in HIP graphs (one graph per run of consecutive calls, each call on
    the next copy), replayed on one stream."""

    def __init__(self, w, dev, eager: bool):
        import torch
        from exact_row_wise_sampled_amd import topkf
        self.w = w
        self.dev = dev
        self.eager = eager
        m, n = w.m, w.n
        self.copies = max(2, math.ceil(2 * MALL_BYTES / (m * n * 4)))
        base = torch.from_numpy(w.x).to(dev)
        self.xs = [base] + [base.clone() for _ in range(self.copies - 1)]
        self.ke = torch.from_numpy(w.ke).to(dev)
        self.nvr = torch.tensor([m], dtype=torch.int32, device=dev)
        self.outs = [torch.empty((m, w.k), dtype=torch.int32, device=dev)
                     for _ in range(self.copies)]
        self.sel = topkf.Selector(m, n, device=dev)
        self.stream = torch.cuda.Stream(device=dev)
        self.dev = dev
        self.pos = 0  # copy the next call reads
        self.graphs = {}
        torch.cuda.synchronize()

    def call(self, i: int) -> None:
        self.sel(self.xs[i], self.ke, self.outs[i], self.nvr, self.w.k, stream=self.stream)

    def _graph(self, start: int, n: int):
        import torch
        key = (start, n)
        g = self.graphs.get(key)
        if g is None:
            self.stream.wait_stream(torch.cuda.current_stream())
            # one eager pass of the same calls before capture
            with torch.cuda.stream(self.stream):
                for j in range(n):
                    self.call((start + j) % self.copies)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=self.stream):
                for j in range(n):
                    self.call((start + j) % self.copies)
            torch.cuda.synchronize()
            self.graphs[key] = g
        return g

    def prepare(self, n: int):
        """Returns a launcher of the next n calls (a captured graph, or eager calls)."""
        start = self.pos
        self.pos = (self.pos + n) % self.copies
        if n == 0:
            return lambda: None
        if self.eager:
            def run():
                for j in range(n):
                    self.call((start + j) % self.copies)
            return run
        return self._graph(start, n).replay

    def check(self) -> list:
        """Checks one call's output against the CPU oracle (outside any timing)."""
        import torch
        from oracle import oracle
        self.call(self.copies - 1)
        torch.cuda.synchronize()
        res = oracle.topk(self.w.x, self.w.ke, self.w.k)
        return oracle.check_rows(self.outs[-1].cpu().numpy(), self.w.x, res)

    def time(self, warmup: int, steps: int, rounds: int) -> dict:
        """Conditioning reads, warmup calls, then exactly `steps` timed calls in
        `rounds` rounds (at most one round per 10 calls), all queued back to
        back on one stream."""
        import torch
        rounds = max(1, min(rounds, steps // MIN_ROUND_CALLS))
        sizes = [steps // rounds + (1 if j < steps % rounds else 0) for j in range(rounds)]
        warm = self.prepare(warmup)
        launchers = [self.prepare(s) for s in sizes]
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(rounds + 1)]
        torch.cuda.synchronize()
        with torch.cuda.stream(self.stream):
            condition(self.dev, self.stream)
            warm()
            ev[0].record(self.stream)
            for j in range(rounds):
                launchers[j]()
                ev[j + 1].record(self.stream)
        torch.cuda.synchronize()
        means = [ev[j].elapsed_time(ev[j + 1]) / sizes[j] for j in range(rounds)]
        total = ev[0].elapsed_time(ev[rounds])
        if int(self.sel.counters.sum().item()) != 0:
            raise RuntimeError("counters not returned to zero after the timed calls")
        return {"ms_median": statistics.median(means), "ms_mean": total / steps,
                "round_ms": means, "round_sizes": sizes}


def measure(name: str, dev, cus: int, args, w=None) -> dict:
    from exact_row_wise_sampled_amd import topkf, workloads
    if w is None:
        w = workloads.make(name)
    plan = topkf.plan_for(w.m, w.n, cus)
    r = Runner(w, dev, args.eager)
    exact = None
    if not args.no_check:
        fails = r.check()
        if fails:
            raise RuntimeError("%s: output differs from the oracle: %s" % (name, fails))
        exact = True
        print("bench: %s output matches the oracle (%d rows)" % (name, w.m), file=sys.stderr,
              flush=True)
    t = r.time(args.warmup, args.steps, args.rounds)
    ms = t["ms_median"]
    sb = w.score_bytes()
    parts = plan.splits if plan.family == topkf.FAMILY_KVSPLIT else 1
    alg = algorithmic_bytes(w.ke, w.n, w.k, plan.stride, parts)
    gbs = sb / (ms * 1e-3) / 1e9
    ach = alg / (ms * 1e-3) / 1e9
    tr = measured_traffic(name)
    d = {"workload": DESCRIPTIONS[name], "M": w.m, "N": w.n, "K": w.k, "score_bytes": sb,
         "us_per_call": round(ms * 1e3, 3), "us_per_call_mean": round(t["ms_mean"] * 1e3, 3),
         "round_us": [round(v * 1e3, 3) for v in t["round_ms"]], "round_calls": t["round_sizes"],
         "gbs": round(gbs, 2), "rows_per_s": round(w.m / (ms * 1e-3), 1),
         "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
         "algorithmic_bytes": alg, "achieved_gbs": round(ach, 2),
         "roofline_frac": round(ach / HBM_PEAK_GBS, 4),
         "traffic_bytes": None if tr is None else int(tr["traffic_bytes"]),
         "read_per_score_byte": None if tr is None else round(tr["read_bytes"] / sb, 4),
         "rotated_copies": r.copies, "plan": plan.as_dict(), "exact": exact}
    del r
    import torch
    torch.cuda.empty_cache()
    return {"summary": d, "workload": w, "plan": plan}


def kernels_of(plan) -> list:
    from exact_row_wise_sampled_amd import topkf
    s, dl = plan.stride, "true" if plan.dual else "false"
    if plan.family == topkf.FAMILY_PERSISTENT:
        return ["persistent_kernel<%d,%s,false>" % (s, dl)]
    if s == 0:
        return ["kvx_hist_kernel", "kvx_cut_kernel", "kvx_classify_kernel", "kvx_finish_kernel"]
    return ["kvsplit_scan_kernel<%d,%s,false>" % (s, dl),
            "kvsplit_finish_kernel<%d,%s,false>" % (s, dl)]


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=700, help="timed calls per configuration")
    ap.add_argument("--warmup", type=int, default=110,
                    help="untimed calls before the timed ones (warm-up and conditioning)")
    ap.add_argument("--rounds", type=int, default=7,
                    help="timed calls are split into this many rounds; per-call time = median "
                         "of the round means")
    ap.add_argument("--config", default="prefill", choices=sorted(DESCRIPTIONS),
                    help="the headline configuration")
    ap.add_argument("--only", action="store_true",
                    help="time the headline configuration alone (no per_config entries)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall time of the CPU oracle baseline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch every call directly instead of replaying HIP graphs "
                         "(for hardware-counter runs)")
    ap.add_argument("--no-ref", action="store_true", help="skip the streaming-read reference")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one plain 256 MiB device copy first, the calibration "
                         "reference for FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the selector has no multi-GPU path "
              "(rows are independent and would be sharded in contiguous blocks; see the "
              "sharding note in DESIGN.md)", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("bench.py: --steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch

    from exact_row_wise_sampled_amd import workloads

    dev = torch.device("cuda:0")
    if args.copy_probe:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cus = torch.cuda.get_device_properties(dev).multi_processor_count

    names = [args.config] if args.only else [args.config] + [c for c in ORDER if c != args.config]
    results = {}
    for name in names:
        results[name] = measure(name, dev, cus, args)
        s = results[name]["summary"]
        print("bench: %-11s %9.3f us/call  %8.1f GB/s  frac %.4f" % (
            name, s["us_per_call"], s["gbs"], s["roofline_frac"]), file=sys.stderr, flush=True)
    head = results[args.config]
    h = head["summary"]
    ms = h["us_per_call"] * 1e-3
    tr = measured_traffic(args.config)
    line = {
        "metric": "score-row GB/s and rows/s vs HBM peak, K=2048, ragged rows up to 512K",
        "value": h["gbs"],
        "unit": "GB/s",
        "rows_per_s": h["rows_per_s"],
        "hbm_peak_frac": h["hbm_peak_frac"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "ms_per_step_mean": round(h["us_per_call_mean"] * 1e-3, 6),
        "timing": "median over %d rounds of the mean per-call time (HIP events on the graphs' "
                  "stream); %s; each configuration's warm-up follows %.0f ms of streaming reads "
                  "of a separate buffer, queued back to back" % (
                      len(h["round_calls"]), "eager launches" if args.eager else "HIP graph replays",
                      CONDITION_MS),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": DESCRIPTIONS[args.config], "M": h["M"], "N": h["N"], "K": h["K"],
                   "score_bytes": h["score_bytes"], "rotated_copies": h["rotated_copies"],
                   "plan": h["plan"]},
        "roofline": {"bound": "hbm", "achieved": h["achieved_gbs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": h["roofline_frac"],
                     "traffic": None if tr is None else int(tr["traffic_bytes"]),
                     "algorithmic_bytes_per_launch": h["algorithmic_bytes"],
                     "kernels": kernels_of(head["plan"]),
                     "timing": "achieved = algorithmic bytes per call / per-call time; one call "
                               "runs every listed kernel"},
    }
    if not args.only:
        line["per_config"] = {n: results[n]["summary"] for n in names}
    if not args.no_ref:
        ref = stream_read_reference(dev)
        line["stream_read_ref_gbs"] = round(ref, 1)
        line["stream_read_ref_frac"] = round(h["gbs"] / ref, 4)
    if not args.no_cpu:
        small = {}
        if not args.only:
            small = {n: results[n]["workload"] for n in ("tiny", "decode") if n in results}
        line["cpu_baseline"] = cpu_baseline(head["workload"], args.cpu_seconds, small)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
