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
WIRE_WORKLOAD = "wire_check_r1024_mixed_q"
STOCHASTIC_WORKLOAD = "stochastic_verify_r1024_targets"


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


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (Linux), else what
    platform reports."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


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
                      f"{cpu_model()} ({os.cpu_count()} host cores present)"}


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


def _tensors(o, pre=""):
    """(name, tensor) pairs of an output dict, nested dicts included."""
    import torch
    for k, v in o.items():
        if isinstance(v, torch.Tensor):
            yield pre + k, v
        elif isinstance(v, dict):
            yield from _tensors(v, pre + k + ".")


def _timed(fn, steps, warmup):
    """Mean HIP-event duration (ms) of fn on the current stream, and the wall
    time per call (ms) between two synchronisations."""
    import torch
    for _ in range(warmup):
        fn()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s, e in evs:
        s.record(stream)
        fn()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return sum(s.elapsed_time(e) for s, e in evs) / steps, wall * 1e3 / steps


def wire_bench(args):
    """Receiver-side check of the q rows of the R = 1024 mixed workload in
    the wire form: dense rows of V binary32 values, sparse rows of (id,
    value) pairs, each with its sampled token.  The q, tokens and wire values
    are made once by the library; the timed step is the check alone."""
    import numpy as np
    import torch

    from vocab_wide_draft_amd import binding as B
    from vocab_wide_draft_amd import workloads as W

    w = W.make(5)
    dev = torch.device("cuda:0")
    d = torch.from_numpy(w.draft.view(np.int16)).view(torch.bfloat16).to(dev)
    t = torch.from_numpy(w.target.view(np.int16)).view(torch.bfloat16).to(dev)
    draws = torch.from_numpy(w.draws.view(np.int32)).to(dev)
    out = B.fused(d, t, B.SAMPLED, topk=w.topk, k_max=1024, draws=draws)
    q = out["q"]
    dense_w = B.q_encode(q["dense"])
    sp_w = B.q_encode(q["sp_cnt"])
    tok = out["sample"]
    del d, t
    torch.cuda.synchronize()
    n = w.draft.shape[0]
    topk = np.asarray(w.topk)
    lens = q["sp_len"].cpu().numpy()
    n_dense = int((topk == 0).sum())
    alg = n_dense * w.V * 4 + int(lens[topk != 0].sum()) * 8 + n * 16

    topk_dev = torch.from_numpy(topk.astype(np.int32)).to(dev)

    def check():
        return B.q_validate(w.V, topk=topk_dev, k_max=1024, dense=dense_w, sp_ids=q["sp_ids"], sp_val=sp_w,
                            sp_len=q["sp_len"], tokens=tok)

    kernel_ms, ms_per_step = _timed(check, args.steps, args.warmup)
    st = check()["status"].cpu().numpy()
    dense_rows = q["dense"][torch.from_numpy(topk == 0).to(dev)].contiguous()
    enc_out = torch.empty(dense_rows.shape, dtype=torch.float32, device=dev)
    enc_ms, _ = _timed(lambda: B.q_encode(dense_rows, out=enc_out), args.steps, args.warmup)
    enc_bytes = dense_rows.numel() * 8
    # a plain device copy of the same bytes (torch's copy kernel), as the
    # practical read + write ceiling beside the encoder
    src_f = dense_rows.view(torch.float32)
    copy_ms, _ = _timed(lambda: enc_out.copy_(src_f), args.steps, args.warmup)
    del dense_rows, enc_out, src_f
    d = torch.from_numpy(w.draft.view(np.int16)).view(torch.bfloat16).to(dev)
    mrg_ms, _ = _timed(lambda: B.margin(d), args.steps, args.warmup)
    mrg_bytes = n * w.V * 2 + n * 4
    achieved = alg / (kernel_ms * 1e-3) / 1e9
    res = {
        "metric": "q rows checked per second (wire form, receiver side)",
        "value": round(n / (ms_per_step * 1e-3), 1),
        "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u32", "data": "synthetic",
        "config": {"workload": "wire check of the R=1024 mixed workload's q", "rows": n, "dense_rows": n_dense,
                   "V": w.V, "rows_refused": int((st != 0).sum())},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic(WIRE_WORKLOAD),
                     "algorithmic_bytes": alg, "kernel_ms": round(kernel_ms, 4)},
        "encode": {"rows": n_dense, "kernel_ms": round(enc_ms, 4), "bytes": enc_bytes,
                   "achieved_GBs": round(enc_bytes / (enc_ms * 1e-3) / 1e9, 1),
                   "plain_copy_GBs": round(enc_bytes / (copy_ms * 1e-3) / 1e9, 1)},
        "margin": {"rows": n, "kernel_ms": round(mrg_ms, 4), "bytes": mrg_bytes,
                   "achieved_GBs": round(mrg_bytes / (mrg_ms * 1e-3) / 1e9, 1)},
    }
    if not args.no_cpu:
        from oracle import q_wire as Q
        hw, ht = dense_w.cpu().numpy(), tok.cpu().numpy()
        t0 = time.perf_counter()
        done = 0
        for r in range(n):
            if topk[r] != 0:
                continue
            Q.check_dense(hw[r], w.V, token=int(ht[r]))
            done += 1
            if time.perf_counter() - t0 > args.cpu_seconds:
                break
        el = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(done / el, 3), "unit": "rows/s", "cores": 1, "kind": "oracle",
                               "sample": f"{done} dense rows of the same q, oracle.q_wire.check_dense"}
    print(json.dumps(res), flush=True)


def _mixed_step_outputs():
    """The R = 1024 mixed workload on the device and one fused step of it
    (made before any timed region): target rows, the sampled drafts, their
    statuses and q."""
    import numpy as np
    import torch

    from vocab_wide_draft_amd import binding as B
    from vocab_wide_draft_amd import workloads as W

    w = W.make(5)
    dev = torch.device("cuda:0")
    d = torch.from_numpy(w.draft.view(np.int16)).view(torch.bfloat16).to(dev)
    t = torch.from_numpy(w.target.view(np.int16)).view(torch.bfloat16).to(dev)
    draws = torch.from_numpy(w.draws.view(np.int32)).to(dev)
    f = B.fused(d, t, B.SAMPLED, topk=w.topk, k_max=1024, draws=draws)
    dtok = f["sample"].view(w.R, 5).clone()
    dst = f["status"].view(w.R, 5).clone()
    return w, t, dtok, dst, f["q"]


def stochastic_bench(args):
    """Stochastic verification of the R = 1024 mixed workload: each of the
    6,144 target rows gets an exact inverse-CDF draw from its p with its own
    64-bit draw, and the workload's sampled drafts are checked against those
    draws."""
    import numpy as np

    from vocab_wide_draft_amd import binding as B

    w, t, dtok, dst, _ = _mixed_step_outputs()
    rng = np.random.default_rng(0xD5A1F00D)
    tdr = rng.integers(0, 2**63, (w.R, 6), dtype=np.uint64) * np.uint64(2)
    tdraws = B.u64_draws(tdr, t.device)
    out = B.verify_stochastic(t, dtok, tdraws, draft_status=dst)
    kernel_ms, ms_per_step = _timed(lambda: B.verify_stochastic(t, dtok, tdraws, draft_status=dst, out=out),
                                    args.steps, args.warmup)
    n = 6 * w.R
    alg = n * w.V * 2 + n * 16 + w.R * 32
    achieved = alg / (kernel_ms * 1e-3) / 1e9
    acc = out["accept_len"].cpu().numpy()
    res = {
        "metric": "target rows verified per second (stochastic verification)",
        "value": round(n / (ms_per_step * 1e-3), 1), "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int256", "data": "synthetic",
        "config": {"workload": "stochastic verification of the R=1024 mixed workload", "R": w.R, "V": w.V,
                   "target_rows": n, "mean_accept_len": round(float(acc.mean()), 3),
                   "requests_refused": int((out["req_status"].cpu().numpy() != 0).sum())},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic(STOCHASTIC_WORKLOAD),
                     "algorithmic_bytes": alg, "kernel_ms": round(kernel_ms, 4)},
    }
    if not args.no_cpu:
        from oracle import dyadic24 as O
        ht, hs = dtok.cpu().numpy(), dst.cpu().numpy()
        t0 = time.perf_counter()
        done = 0
        for r in range(w.R):
            O.verify_stochastic(list(ht[r]), list(hs[r]), w.target[6 * r:6 * r + 6], "bf16",
                                [int(u) for u in tdr[r]])
            done += 1
            if time.perf_counter() - t0 > args.cpu_seconds:
                break
        el = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(6 * done / el, 3), "unit": "rows/s", "cores": 1, "kind": "oracle",
                               "sample": f"first {done} requests ({6 * done} target rows), oracle.verify_stochastic"}
    print(json.dumps(res), flush=True)


def ratio_bench(args):
    """Probability-ratio verification of the R = 1024 mixed workload's
    sampled drafts against its target rows, with the drafts' dyadic q (dense,
    k = 32 and k = 1024 rows).  Algorithmic bytes per request: the target
    rows it reads (up to the position that ends it), and the q row of a
    rejected position (4 B per dense count, 8 B per sparse entry)."""
    import numpy as np

    from oracle import dyadic24 as O  # noqa: F401  (cpu_baseline leg below)
    from vocab_wide_draft_amd import binding as B

    w, t, dtok, dst, qd = _mixed_step_outputs()
    rng = np.random.default_rng(0xD5A1F00E)
    ad = rng.integers(0, 2**63, (w.R, 5), dtype=np.uint64) * np.uint64(2)
    fd = rng.integers(0, 2**63, w.R, dtype=np.uint64) * np.uint64(2) + np.uint64(1)
    adv, fdv = B.u64_draws(ad, t.device), B.u64_draws(fd, t.device)
    out = B.verify_ratio(t, dtok, qd, adv, fdv, draft_status=dst)
    kernel_ms, ms_per_step = _timed(lambda: B.verify_ratio(t, dtok, qd, adv, fdv, draft_status=dst, out=out),
                                    args.steps, args.warmup)
    acc = out["accept_len"].cpu().numpy()
    rst = out["req_status"].cpu().numpy()
    hs = dst.cpu().numpy()
    lens = qd["sp_len"].cpu().numpy()
    topk = np.asarray(w.topk)
    alg = 0
    for r in range(w.R):
        if rst[r] != 0:
            continue
        i = int(acc[r])
        alg += (i + 1) * w.V * 2 + 5 * 8 + 8 + 12
        j = 5 * r + i
        if i < 5 and hs[r, i] == 0:  # ended by a rejection: the residual reads q
            alg += w.V * 4 if topk[j] == 0 else int(lens[j]) * 8
    achieved = alg / (kernel_ms * 1e-3) / 1e9
    res = {
        "metric": "requests verified per second (probability-ratio verification)",
        "value": round(w.R / (ms_per_step * 1e-3), 1), "unit": "requests/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int256", "data": "synthetic",
        "config": {"workload": "ratio verification of the R=1024 mixed workload", "R": w.R, "V": w.V,
                   "mean_accept_len": round(float(acc[rst == 0].mean()), 3),
                   "requests_refused": int((rst != 0).sum())},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "algorithmic_bytes": alg, "kernel_ms": round(kernel_ms, 4)},
    }
    if not args.no_cpu:
        from oracle import ratio as RT
        hq = {k: (v.cpu().numpy() if v is not None and hasattr(v, "cpu") else v) for k, v in qd.items()}
        ht = dtok.cpu().numpy()
        t0 = time.perf_counter()
        done = 0
        for r in range(w.R):
            qs = []
            for i in range(5):
                j = 5 * r + i
                if topk[j] == 0:
                    qs.append((np.arange(w.V), hq["dense"][j].view(np.uint32)))
                else:
                    n = int(hq["sp_len"][j])
                    qs.append((hq["sp_ids"][j, :n], hq["sp_cnt"][j, :n].view(np.uint32)))
            RT.verify_ratio(list(ht[r]), list(hs[r]), qs, w.target[6 * r:6 * r + 6], "bf16",
                            [int(u) for u in ad[r]], int(fd[r]))
            done += 1
            if time.perf_counter() - t0 > args.cpu_seconds:
                break
        el = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(done / el, 3), "unit": "requests/s", "cores": 1, "kind": "oracle",
                               "sample": f"first {done} requests, oracle.ratio.verify_ratio"}
    print(json.dumps(res), flush=True)


def sharded_bench(args):
    """The vocabulary-sharded propose emulated on one GPU over the 5,120
    draft rows of the R = 1024 mixed workload, two shards per row (64,640
    ids each).  Algorithmic bytes are one read of the rows; the emulator
    reads each shard twice (maximum, then exact sum), as a rank would not
    have to if its shard stayed on chip."""
    import numpy as np
    import torch

    from vocab_wide_draft_amd import binding as B
    from vocab_wide_draft_amd import workloads as W

    w = W.make(5)
    dev = torch.device("cuda:0")
    d = torch.from_numpy(w.draft.view(np.int16)).view(torch.bfloat16).to(dev)
    G = 2
    kernel_ms, ms_per_step = _timed(lambda: B.sharded_propose(d, G), args.steps, args.warmup)
    n = d.shape[0]
    alg = n * w.V * 2 + n * 20
    achieved = alg / (kernel_ms * 1e-3) / 1e9
    st = B.sharded_propose(d, G)["status"].cpu().numpy()
    # beside it: the sharded q (dense rows with global tickets, sparse rows
    # from merged shard top-k) and the shard-then-token sample of every row
    draws = torch.from_numpy(w.draws.view(np.int32)).to(dev)
    qo = B.sharded_q(d, G, topk=w.topk, k_max=1024, draws=draws)
    q_ms, _ = _timed(lambda: B.sharded_q(d, G, draws=draws, out=qo), args.steps, args.warmup)
    topk = np.asarray(w.topk)
    lens = qo["sp_len"].cpu().numpy()
    q_bytes = alg + int((topk == 0).sum()) * w.V * 4 + int(lens[topk != 0].sum()) * 8 + n * 4
    q_rows_refused = int((qo["status"].cpu().numpy() != 0).sum())
    res = {
        "metric": "draft rows proposed per second (vocabulary-sharded, emulated on one GPU)",
        "value": round(n / (ms_per_step * 1e-3), 1), "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": {"workload": "sharded propose of the R=1024 mixed workload's draft rows", "rows": n, "V": w.V,
                   "shards": G, "rows_refused": int((st != 0).sum())},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "algorithmic_bytes": alg, "kernel_ms": round(kernel_ms, 4)},
        "sharded_q": {"rows": n, "shards": G, "kernel_ms": round(q_ms, 4), "algorithmic_bytes": q_bytes,
                      "achieved_GBs": round(q_bytes / (q_ms * 1e-3) / 1e9, 1), "rows_refused": q_rows_refused},
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=5, help="workload 1..5 (default: the R=1024 mixed batch)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--graph", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the step captured as one HIP graph (default); the faster launch mode is "
                         "the reported step")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--also", default=None,
                    help="comma-separated workloads measured after the main one and reported under 'also' "
                         "(default: 4 when --config is 5; an empty string for none)")
    ap.add_argument("--copy-probe", type=int, default=0, help="only run a plain copy of this many bytes")
    ap.add_argument("--op", choices=["step", "wire", "stochastic", "ratio", "sharded"], default="step",
                    help="step: the fused propose/q/sample/verify step; wire: the receiver's check of the "
                         "workload's q in the FP32 wire form (and the sender's encoding, reported beside it); "
                         "stochastic: stochastic verification of the workload's sampled drafts; "
                         "ratio: probability-ratio verification of them with their q; "
                         "sharded: the vocabulary-sharded propose (two shards per row) of its draft rows")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): this step shards by request with no "
              "exchange, and multi-GPU runs are not part of this build", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe, 10)
        return
    if args.op == "wire":
        wire_bench(args)
        return
    if args.op == "stochastic":
        stochastic_bench(args)
        return
    if args.op == "ratio":
        ratio_bench(args)
        return
    if args.op == "sharded":
        sharded_bench(args)
        return

    res, w = step_line(args.config, args)
    also = [4] if args.also is None and args.config == 5 else [int(c) for c in (args.also or "").split(",") if c]
    if also:
        # the other configuration the bandwidth bar applies to, measured in the same run
        res["also"] = {}
        for c in also:
            r, _ = step_line(c, args)
            res["also"][r["config"]["workload"]] = {
                "ms_per_step": r["ms_per_step"], "rows_per_s": r["value"], "launch": r["config"]["launch"],
                "frac": r["roofline"]["frac"], "achieved": r["roofline"]["achieved"],
                "algorithmic_bytes": r["roofline"]["algorithmic_bytes"], "kernel_ms": r["roofline"]["kernel_ms"],
                "traffic": r["roofline"]["traffic"], "rows_failed": r["config"]["rows_failed"]}
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def step_line(cfg: int, args):
    """The bench line of one workload's fused step (without the CPU baseline),
    and the workload."""
    import numpy as np
    import torch

    from vocab_wide_draft_amd import binding as B
    from vocab_wide_draft_amd import workloads as W

    w = W.make(cfg)
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

    def eager():
        B.fused(d, t, mode, draws=draws, out=out)

    graph = None
    if args.graph:
        # the whole step captured once into a HIP graph and replayed: one
        # submission per step instead of one per kernel
        torch.cuda.synchronize()
        ref = {k: v.clone() for k, v in _tensors(out)}
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            eager()
        graph.replay()
        torch.cuda.synchronize()
        now = dict(_tensors(out))
        for k, v in ref.items():
            if not torch.equal(now[k], v):
                raise RuntimeError(f"graph replay differs from the eager step in {k}")
    # both launch modes timed over the same number of steps; the faster one is
    # the reported step, the other is kept beside it
    times = {"eager": _timed(eager, args.steps, max(args.warmup - 1, 0))}
    if graph is not None:
        times["hip graph"] = _timed(graph.replay, args.steps, max(args.warmup - 1, 0))
    launch = min(times, key=lambda k: times[k][1])
    mean_launch, ms_per_step = times[launch]
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
                   "rows_failed": int((st != 0).sum()), "launch": launch,
                   "ms_per_step_by_launch": {k: round(v[1], 4) for k, v in times.items()},
                   "parallelism": "single GPU; bf16 rows: one workgroup per row; streamed dense rows: "
                                  "vocabulary shards per row, a workgroup per shard and pass"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic(w.name),
                     "algorithmic_bytes": alg, "kernel_ms": round(mean_launch, 4)},
    }
    return res, w




if __name__ == "__main__":
    main()
