"""The five configurations at full size (V = 129280), in the launch
configuration the benchmark times.  Every row and request is compared with
the oracle: statuses, argmaxes, samples, sparse lengths, target argmaxes,
accept lengths and bonuses bit for bit, confidences within 1e-6 relative,
and each row's q through a 64-bit digest of its counts (and ids), all
against tests/golden/full_c<n>.npz, which tests/golden/make_full_parity.py
writes from the oracle alone.  A few whole requests are also recomputed by
the oracle here and compared element by element, and invariants are checked
on every row."""
import os
import sys

import numpy as np
import pytest

from oracle import dyadic24 as O
from vocab_wide_draft_amd import workloads as W

from gpu_helpers import CONF_RTOL, check_workload, run_fused

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
sys.path.insert(0, GOLDEN)
import make_full_parity as G  # noqa: E402

pytestmark = pytest.mark.gpu


def _invariants(w, h):
    st = h["status"]
    assert ((h["argmax"] >= 0) & (h["argmax"] < w.V)).all()
    ok = st == 0
    assert ((h["conf"][ok] > 0) & (h["conf"][ok] <= 1)).all()
    assert (h["argmax"][~ok] == 0).all() and (h["conf"][~ok] == 0).all()
    assert ((h["accept_len"] >= 0) & (h["accept_len"] <= 5)).all()
    if w.topk is not None:
        q = h["q"]
        dense = np.flatnonzero(w.topk == 0)
        if dense.size:
            sums = q["dense"][dense].view(np.uint32).astype(np.int64).sum(axis=1)
            assert (sums[ok[dense]] == O.M).all() and (sums[~ok[dense]] == 0).all()


def _gpu_digests(w, h):
    q = h["q"]
    n = w.R * 5
    dig = np.zeros(n, np.uint64)
    ln = np.zeros(n, np.int32)
    for j in range(n):
        k = int(w.topk[j])
        if k == 0:
            ln[j] = -1
            dig[j] = G.q_digest(None, q["dense"][j].view(np.uint32), True, w.V)
        else:
            m = int(q["sp_len"][j])
            ln[j] = m
            dig[j] = G.q_digest(q["sp_ids"][j, :m], q["sp_cnt"][j, :m].view(np.uint32), False, w.V)
    return ln, dig


@pytest.mark.parametrize("cfg,reqs", [(1, [0]), (2, [0, 3]), (3, [0, 37]), (4, [0, 200]), (5, None)])
def test_full_config_every_row(cfg, reqs):
    g = np.load(os.path.join(GOLDEN, f"full_c{cfg}.npz"))
    assert str(g["meta_sources_sha256"]) == G.sources_hash(), \
        f"tests/golden/full_c{cfg}.npz predates the oracle or generator sources: rerun make_full_parity.py"
    w = W.make(cfg)
    assert int(g["meta_seed"]) == W.SEED_BASE + cfg and int(g["meta_V"]) == w.V
    h = run_fused(w)
    _invariants(w, h)
    for key, name in (("status", "d_status"), ("argmax", "d_argmax")):
        bad = np.flatnonzero(h[key] != g[name])
        assert bad.size == 0, f"cfg {cfg}: {key} differs on rows {bad[:10]}"
    if h.get("sample") is not None:
        bad = np.flatnonzero(h["sample"] != g["d_sample"])
        assert bad.size == 0, f"cfg {cfg}: sample differs on rows {bad[:10]}"
    ref = g["d_conf"].astype(np.float64)
    err = np.abs(h["conf"].astype(np.float64) - ref)
    assert (err <= CONF_RTOL * np.abs(ref)).all(), f"cfg {cfg}: confidence off on rows {np.flatnonzero(err > CONF_RTOL * np.abs(ref))[:10]}"
    if w.topk is not None:
        ln, dig = _gpu_digests(w, h)
        bad = np.flatnonzero((ln != g["d_len"]) | (dig != g["d_digest"]))
        assert bad.size == 0, f"cfg {cfg}: q differs on rows {bad[:10]}"
    for key, name in (("target_status", "t_status"), ("target_argmax", "t_argmax"), ("req_status", "r_status"),
                      ("accept_len", "r_accept"), ("bonus", "r_bonus")):
        bad = np.flatnonzero(h[key] != g[name])
        assert bad.size == 0, f"cfg {cfg}: {key} differs at {bad[:10]}"
    if reqs is None:  # the mixed config: requests holding one-hot and duplicate rows, plus each row kind
        special = sorted(set((w.meta["onehot_rows"][:2] // 5).tolist() + (w.meta["dup_rows"][:2] // 5).tolist()))
        reqs = sorted(set(special + [0, 1, 3]))
    check_workload(w, h, requests=reqs, label=f"full cfg{cfg}")
