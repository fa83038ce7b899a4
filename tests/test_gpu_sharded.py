"""GPU parity of the vocabulary-sharded propose emulated on one GPU ("PP1 q
transport and scheduling design", "Sparse support and vocabulary-sharded TP2
follow-up") through the C ABI: status, argmax and the exact-sum S64 equal the
oracle's unsharded values bit for bit, for every shard count."""
import numpy as np
import pytest
import torch

from oracle import dyadic24 as O
from vocab_wide_draft_amd import binding as B
from vocab_wide_draft_amd import workloads as W

from gpu_helpers import to_dev

pytestmark = pytest.mark.gpu


def _rows(V, rng):
    base = (rng.standard_normal(V) * 2).astype(np.float32)
    rows = [base.copy()]
    r = base.copy(); r[V - 1] = r.max() + 1; rows.append(r)                 # maximum in the last shard
    r = base.copy(); mx = r.max() + 1; r[V - 2] = mx; r[1 % V] = mx; rows.append(r)   # tie across shards
    r = np.full(V, -np.inf, np.float32); r[V // 2] = 0.5; rows.append(r)    # one-hot
    r = np.full(V, -1.0, np.float32); r[V - 1] = 0.0; r[0] = -0.0; rows.append(r)    # -0 before +0
    rows.append(np.full(V, 1.25, np.float32))                                # constant
    r = base.copy(); r[:V // 2] = -np.inf; rows.append(r)                    # masked first half
    r = (base - 60.0).astype(np.float32); r[3 % V] = 10.0; rows.append(r)    # tiny weights
    r = base.copy(); r[V // 3] = np.nan; rows.append(r)
    r = base.copy(); r[V - 1] = np.inf; rows.append(r)
    rows.append(np.full(V, -np.inf, np.float32))
    return np.stack(rows)


@pytest.mark.parametrize("dtype,V", [("f32", 3001), ("bf16", 3001), ("bf16", 7), ("bf16", 129280), ("f32", 129280)])
def test_sharded_propose(dtype, V):
    rng = np.random.default_rng(V + 5)
    x = _rows(V, rng)
    raw = W.f32_to_bf16_bits(x) if dtype == "bf16" else x
    want = [O.propose_sum(raw[j], dtype) for j in range(x.shape[0])]
    d = to_dev(raw, dtype)
    for G in sorted({1, 2, 3, 8, min(64, V)}):
        if G > V:
            continue
        out = B.sharded_propose(d, G)
        st, am = out["status"].cpu().numpy(), out["argmax"].cpu().numpy()
        s64, cf = out["s64"].cpu().numpy(), out["conf"].cpu().numpy()
        for j, (ws, wa, wsum) in enumerate(want):
            assert (int(st[j]), int(am[j])) == (ws, wa), (dtype, V, G, j)
            assert s64[j] == wsum, (dtype, V, G, j, s64[j], wsum)
            assert cf[j] == (np.float32(1.0 / wsum) if ws == O.ST_OK else 0.0), (dtype, V, G, j)
