"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
HIP path through the binding, and compare with the CPU oracle row by row."""
from __future__ import annotations

import numpy as np
import torch

from oracle import dyadic24 as O
from vocab_wide_draft_amd import binding as B

CONF_RTOL = 1e-6  # confidence tolerance (relative, binary32)


def dev():
    return torch.device("cuda:0")


def to_dev(arr: np.ndarray, dtype: str) -> torch.Tensor:
    """Rows on the device with a 16-byte row stride; the padding past V holds
    NaN, so a read past the end of a row would show up as a NaN status."""
    arr = np.asarray(arr)
    n, V = arr.shape
    es = 2 if dtype == "bf16" else 4
    vpad = -(-V * es // 16) * 16 // es
    if dtype == "bf16":
        buf = np.full((n, vpad), 0x7FC0, np.uint16)
        buf[:, :V] = arr
        t = torch.from_numpy(buf.view(np.int16)).view(torch.bfloat16).to(dev())
    else:
        buf = np.full((n, vpad), np.nan, np.float32)
        buf[:, :V] = arr
        t = torch.from_numpy(buf).to(dev())
    return t[:, :V]


def u32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to(dev())


def run_fused(w, rows=None):
    """Fused step on workload w; returns host numpy outputs."""
    d, t = to_dev(w.draft, w.dtype), to_dev(w.target, w.dtype)
    mode = B.SAMPLED if w.mode == "sampled" else B.GREEDY
    draws = None if w.draws is None else u32_dev(w.draws)
    with_q = w.topk is not None
    out = B.fused(d, t, mode, topk=w.topk, k_max=1024 if with_q else 0, draws=draws, with_q=with_q)
    torch.cuda.synchronize()
    return host(out)


def host(out):
    h = {}
    for k, v in out.items():
        if isinstance(v, torch.Tensor):
            h[k] = v.cpu().numpy()
        elif isinstance(v, dict):
            h[k] = {kk: (vv.cpu().numpy() if isinstance(vv, torch.Tensor) else vv) for kk, vv in v.items()}
        else:
            h[k] = v
    return h


def check_draft_row(h, j, ref, k, label=""):
    """Compare the GPU outputs of draft row j with the oracle's dict."""
    st = int(h["status"][j])
    assert st == ref["status"], f"{label} row {j}: status {st} != {ref['status']}"
    assert int(h["argmax"][j]) == ref["argmax"], f"{label} row {j}: argmax"
    c_gpu, c_ref = float(h["conf"][j]), float(ref["conf"])
    assert abs(c_gpu - c_ref) <= CONF_RTOL * abs(c_ref), f"{label} row {j}: conf {c_gpu} vs {c_ref}"
    if h.get("sample") is not None:
        assert int(h["sample"][j]) == ref["sample"], f"{label} row {j}: sample"
    q = h.get("q")
    if q is None or k is None:
        return
    if k == 0:
        got = q["dense"][j].astype(np.int64)
        if st == O.ST_OK:
            assert (got == ref["counts"]).all(), f"{label} row {j}: dense counts differ at " \
                f"{np.flatnonzero(got != ref['counts'])[:8]}"
        else:
            assert not got.any(), f"{label} row {j}: failed dense row not zero"
    else:
        n = int(q["sp_len"][j])
        assert n == len(ref["ids"]), f"{label} row {j}: sparse len {n} vs {len(ref['ids'])}"
        assert (q["sp_ids"][j, :n] == ref["ids"]).all(), f"{label} row {j}: sparse ids"
        assert (q["sp_cnt"][j, :n].astype(np.int64) == ref["counts"]).all(), f"{label} row {j}: sparse counts"


def check_workload(w, h, requests=None, label=""):
    """Oracle comparison of whole requests (all 11 rows each)."""
    reqs = range(w.R) if requests is None else requests
    for r in reqs:
        tk = None if w.topk is None else w.topk[r * 5:(r + 1) * 5].tolist()
        dr = None if w.draws is None else w.draws[r * 5:(r + 1) * 5].tolist()
        ref = O.request(w.draft[r * 5:(r + 1) * 5], w.target[r * 6:(r + 1) * 6], w.dtype, w.mode,
                        topk=tk, draws=dr)
        for i in range(5):
            check_draft_row(h, r * 5 + i, ref["draft"][i], None if tk is None else tk[i], label)
        assert h["target_status"][r * 6:(r + 1) * 6].tolist() == ref["target_status"], f"{label} req {r}"
        assert h["target_argmax"][r * 6:(r + 1) * 6].tolist() == ref["target_argmax"], f"{label} req {r}"
        assert int(h["req_status"][r]) == ref["req_status"], f"{label} req {r}"
        assert int(h["accept_len"][r]) == ref["accept_len"], f"{label} req {r}"
        assert int(h["bonus"][r]) == ref["bonus"], f"{label} req {r}"
