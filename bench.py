"""Throughput of the fused propose + dyadic24 + verify step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 5] [--no-cpu]

One step is one dspark_fused call over the whole batch of a configuration
(5 draft rows + 6 target rows per request, V = 129280), inputs resident in
HBM.  Prints one JSON line: rows/s, the roofline of the row kernel (HIP
events on the launch stream; algorithmic bytes per launch / mean launch
time against 8 TB/s), the HBM traffic measured by rocprofv3 counters when a
matching profile is committed, and the CPU oracle timed on a bounded sample
of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "rows/sec at V=129280 (propose+dyadic24+verify); achieved HBM GB/s vs peak"
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "vocab_wide_draft_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def _code_tokens(src: str) -> str:
    """C++ source without its comments, whitespace runs folded to one space:
    edits to comments or layout leave the kernels, and so the hash, as they
    were.  (The sources hold no string literal with // or /* in it.)"""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp", ".inc")):
            with open(os.path.join(CSRC, name), encoding="utf-8") as f:
                h.update(name.encode() + _code_tokens(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from committed rocprofv3 counters, or None when
    there is none for this workload or the kernel sources changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload)
    if not e or e.get("kernel_source_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(w, max_seconds: float):
    """The oracle (single-threaded numpy + Python integers) on the first
    requests of the same workload until about max_seconds have passed."""
    from oracle import dyadic24 as O
    t0 = time.perf_counter()
    n = 0
    while n < w.R and (time.perf_counter() - t0) < max_seconds:
        tk = None if w.topk is None else w.topk[n * 5:(n + 1) * 5].tolist()
        dr = None if w.draws is None else w.draws[n * 5:(n + 1) * 5].tolist()
        O.request(w.draft[n * 5:(n + 1) * 5], w.target[n * 6:(n + 1) * 6], w.dtype, w.mode, topk=tk, draws=dr)
        n += 1
    el = time.perf_counter() - t0
    return {"value": round(11 * n / el, 3), "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} requests ({11 * n} rows) of {w.name}, {el:.1f} s single-threaded on "
                      f"{platform.processor() or platform.machine()} ({os.cpu_count()} host cores present)"}


def copy_probe(nbytes: int, reps: int):
    """A plain device-to-device copy of known size, for scaling counters."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=5, help="workload 1..5 (default: the R=1024 mixed batch)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-probe", type=int, default=0, help="only run a plain copy of this many bytes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): this step shards by request with no "
              "exchange, and multi-GPU runs are not part of this build", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe, 10)
        return

    import numpy as np
    import torch

    from vocab_wide_draft_amd import binding as B
    from vocab_wide_draft_amd import workloads as W

    w = W.make(args.config)
    dev = torch.device("cuda:0")

    def up(a):
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    d, t = up(w.draft), up(w.target)
    draws = None if w.draws is None else torch.from_numpy(w.draws.view(np.int32)).to(dev)
    mode = B.SAMPLED if w.mode == "sampled" else B.GREEDY
    with_q = w.topk is not None
    out = B.fused(d, t, mode, topk=w.topk, k_max=1024 if with_q else 0, draws=draws, with_q=with_q)
    for _ in range(max(args.warmup - 1, 0)):
        B.fused(d, t, mode, draws=draws, out=out)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s, e in evs:
        s.record(stream)
        B.fused(d, t, mode, draws=draws, out=out)
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [s.elapsed_time(e) for s, e in evs]
    mean_launch = sum(launch_ms) / len(launch_ms)
    ms_per_step = wall * 1e3 / args.steps
    st = out["status"].cpu().numpy()
    rows = w.rows
    alg = w.algorithmic_bytes()
    achieved = alg / (mean_launch * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(rows / (ms_per_step * 1e-3), 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": w.name, "R": w.R, "V": w.V, "rows": rows, "logits": w.dtype, "mode": w.mode,
                   "requests_per_s": round(w.R / (ms_per_step * 1e-3), 1),
                   "rows_failed": int((st != 0).sum()), "parallelism": "single GPU, one workgroup per row"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic(w.name),
                     "algorithmic_bytes": alg, "kernel_ms": round(mean_launch, 4)},
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
