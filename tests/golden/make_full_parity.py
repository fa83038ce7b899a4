"""Writes tests/golden/full_c<n>.npz: the oracle's outputs for every row and
request of the five workloads at full size (V = 129280), for the full-size
parity test.  It calls only oracle/ (and the seeded input generator, which
holds none of the method's arithmetic):

    python tests/golden/make_full_parity.py [cfg ...] [--jobs N]

Per draft row: status, argmax, confidence (binary32), sample, sparse length
(-1 for a dense row, 0 for no q) and a 64-bit digest of its q (dense: the V
counts as little-endian uint32; sparse: the len ids as little-endian int32,
then their counts as little-endian uint32; the first 8 bytes of SHA-256,
little-endian).  Per target row: status and argmax.  Per request: status,
accept length, bonus.  The file records the configuration, its seed and the
SHA-256 of the oracle and generator sources it was made from.
"""
from __future__ import annotations

import argparse
import hashlib
import multiprocessing as mp
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle import dyadic24 as O  # noqa: E402
from vocab_wide_draft_amd import workloads as W  # noqa: E402

SOURCES = [os.path.join(ROOT, "oracle", "dyadic24.py"), os.path.join(ROOT, "vocab_wide_draft_amd", "workloads.py")]


def sources_hash() -> str:
    h = hashlib.sha256()
    for p in SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def q_digest(ids, counts, dense: bool, V: int) -> int:
    """64-bit digest of one row's q, as described in the module docstring."""
    if dense:
        b = np.asarray(counts, dtype="<u4").tobytes()
        assert len(b) == 4 * V
    else:
        b = np.asarray(ids, dtype="<i4").tobytes() + np.asarray(counts, dtype="<u4").tobytes()
    return int.from_bytes(hashlib.sha256(b).digest()[:8], "little")


_W = None


def _one_request(r):
    w = _W
    tk = None if w.topk is None else w.topk[r * 5:(r + 1) * 5].tolist()
    dr = None if w.draws is None else w.draws[r * 5:(r + 1) * 5].tolist()
    ref = O.request(w.draft[r * 5:(r + 1) * 5], w.target[r * 6:(r + 1) * 6], w.dtype, w.mode, topk=tk, draws=dr)
    rows = []
    for i in range(5):
        d = ref["draft"][i]
        k = None if tk is None else tk[i]
        if k is None:
            ln, dig = 0, 0
        elif k == 0:
            counts = d["counts"] if d["status"] == O.ST_OK else np.zeros(w.V, np.int64)
            ln, dig = -1, q_digest(None, counts, True, w.V)
        else:
            ln, dig = len(d["ids"]), q_digest(d["ids"], d["counts"], False, w.V)
        rows.append((d["status"], d["argmax"], float(d["conf"]), d["sample"], ln, dig))
    return r, rows, ref["target_status"], ref["target_argmax"], (ref["req_status"], ref["accept_len"], ref["bonus"])


def make(cfg: int, jobs: int) -> str:
    global _W
    t0 = time.time()
    _W = w = W.make(cfg)
    n, R = w.R * 5, w.R
    out = {
        "d_status": np.zeros(n, np.int32), "d_argmax": np.zeros(n, np.int32), "d_conf": np.zeros(n, np.float32),
        "d_sample": np.zeros(n, np.int32), "d_len": np.zeros(n, np.int32), "d_digest": np.zeros(n, np.uint64),
        "t_status": np.zeros(R * 6, np.int32), "t_argmax": np.zeros(R * 6, np.int32),
        "r_status": np.zeros(R, np.int32), "r_accept": np.zeros(R, np.int32), "r_bonus": np.zeros(R, np.int32),
    }
    with mp.get_context("fork").Pool(jobs) as pool:
        for r, rows, ts, ta, rq in pool.imap_unordered(_one_request, range(R), chunksize=4):
            for i, (st, am, cf, sm, ln, dg) in enumerate(rows):
                j = r * 5 + i
                out["d_status"][j], out["d_argmax"][j], out["d_conf"][j] = st, am, cf
                out["d_sample"][j], out["d_len"][j], out["d_digest"][j] = sm, ln, dg
            out["t_status"][r * 6:(r + 1) * 6] = ts
            out["t_argmax"][r * 6:(r + 1) * 6] = ta
            out["r_status"][r], out["r_accept"][r], out["r_bonus"][r] = rq
    out["meta_config"] = np.array(cfg, np.int32)
    out["meta_seed"] = np.array(W.SEED_BASE + cfg, np.int64)
    out["meta_V"] = np.array(w.V, np.int32)
    out["meta_sources_sha256"] = np.array(sources_hash())
    path = os.path.join(HERE, f"full_c{cfg}.npz")
    np.savez_compressed(path, **out)
    print(f"config {cfg}: {R} requests in {time.time() - t0:.0f} s -> {path}", flush=True)
    return path


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("cfgs", type=int, nargs="*", default=[1, 2, 3, 4, 5])
    ap.add_argument("--jobs", type=int, default=os.cpu_count() or 1)
    a = ap.parse_args()
    for c in a.cfgs:
        make(c, a.jobs)
