"""The five configurations at full size (V = 129280), in the launch
configuration the benchmark times: the oracle checks whole sampled requests
(all 11 rows each) and invariants are checked on every row."""
import numpy as np
import pytest
import torch

from oracle import dyadic24 as O
from vocab_wide_draft_amd import workloads as W

from gpu_helpers import check_workload, run_fused

pytestmark = pytest.mark.gpu


def _invariants(w, h):
    n = w.R * 5
    st = h["status"]
    assert ((h["argmax"] >= 0) & (h["argmax"] < w.V)).all()
    ok = st == 0
    assert ((h["conf"][ok] > 0) & (h["conf"][ok] <= 1)).all()
    assert (h["argmax"][~ok] == 0).all() and (h["conf"][~ok] == 0).all()
    assert ((h["accept_len"] >= 0) & (h["accept_len"] <= 5)).all()
    if w.topk is not None:
        q = h["q"]
        for j in range(n):
            k = int(w.topk[j])
            if k == 0:
                if ok[j]:
                    assert int(q["dense"][j].astype(np.int64).sum()) == O.M, j
                    assert q["dense"][j][h["sample"][j]] > 0 if h.get("sample") is not None else True
            else:
                m = int(q["sp_len"][j])
                assert 0 <= m <= k
                if ok[j]:
                    ids = q["sp_ids"][j, :m]
                    assert (np.diff(ids) > 0).all() and int(q["sp_cnt"][j, :m].astype(np.int64).sum()) == O.M
                    assert (q["sp_cnt"][j, :m] > 0).all()
                    if h.get("sample") is not None:
                        assert h["sample"][j] in set(ids.tolist())


@pytest.mark.parametrize("cfg,reqs", [(1, [0]), (2, [0, 1, 2, 3]), (3, [0, 37]), (4, [0, 200]), (5, None)])
def test_full_config(cfg, reqs):
    w = W.make(cfg)
    h = run_fused(w)
    _invariants(w, h)
    if reqs is None:  # the mixed config: requests holding one-hot and duplicate rows, plus each row kind
        special = sorted(set((w.meta["onehot_rows"][:2] // 5).tolist() + (w.meta["dup_rows"][:3] // 5).tolist()))
        reqs = sorted(set(special + [0, 1, 3]))
    check_workload(w, h, requests=reqs, label=f"full cfg{cfg}")
