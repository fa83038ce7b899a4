"""Pins for the vocabulary-sharded q oracle (oracle/sharded.py): the merged
shard-local top-k, the counts with globally coordinated tickets and the
shard-then-token sampler must equal the unsharded definitions (pinned
themselves in test_oracle_pins.py) for every shard count, including rows
whose ties straddle shard boundaries."""
import numpy as np
import pytest

from oracle import dyadic24 as O
from oracle import sharded as S

M = 1 << 24
GS = [1, 2, 3, 8, 64]


def _rows(V, rng):
    rows = [(rng.standard_normal(V) * 2).astype(np.float32)]
    vals = rng.standard_normal(3).astype(np.float32)
    rows.append(vals[rng.integers(0, 3, V)])                       # few distinct values: ties everywhere
    r = np.full(V, -np.inf, np.float32); r[rng.integers(0, V, 5)] = 1.0; rows.append(r)   # few finite
    r = np.full(V, 0.5, np.float32); rows.append(r)                  # constant: one tie across all shards
    r = (rng.standard_normal(V) * 2).astype(np.float32); r[rng.random(V) < 0.3] = -np.inf; rows.append(r)
    r = (rng.standard_normal(V) * 2).astype(np.float32); r[[0, V - 1]] = r.max() + 1; rows.append(r)
    return rows


def test_shard_ranges_cover_the_vocabulary():
    for V in (1, 7, 64, 1000, 129280):
        for G in GS:
            if G > V:
                continue
            rg = S.shard_ranges(V, G)
            assert rg[0][0] == 0 and rg[-1][1] == V and all(a[1] == b[0] for a, b in zip(rg, rg[1:]))
    assert S.shard_ranges(129280, 2) == [(0, 64640), (64640, 129280)]


@pytest.mark.parametrize("V", [64, 301])
def test_sharded_topk_equals_global_topk(V):
    rng = np.random.default_rng(V)
    for x in _rows(V, rng):
        for G in GS:
            for k in (1, 7, 32, V, V + 3):
                assert S.sharded_topk(x, k, G).tolist() == O.topk_support(x, k).tolist(), (G, k)


@pytest.mark.parametrize("V", [64, 301, 2000])
def test_sharded_counts_equal_unsharded(V):
    rng = np.random.default_rng(V + 1)
    for x in _rows(V, rng):
        m, _ = O.argmax_first(x)
        st0, c0 = O.dyadic24_counts(O.weights(x, m))
        for G in GS:
            st, c = S.sharded_dense_counts(x, G)
            assert st == st0 and np.array_equal(c, c0), G


def test_sharded_sampler_equals_global_sampler():
    rng = np.random.default_rng(5)
    V = 500
    for x in _rows(V, rng):
        for k in (0, 40):
            st, ids, c = O.q_row(x, k)
            cum = np.cumsum(c)
            us = np.concatenate([rng.integers(0, M, 300), cum[::7], cum[::7] - 1, [0, M - 1]])
            for G in GS:
                for u in us.tolist():
                    assert S.sharded_sample(ids, c, V, G, u) == O.sample(ids, c, u), (G, u)
                assert S.sharded_sample(ids, c, V, G, M)[0] == O.ST_DRAW_RANGE


def test_sharded_q_row_equals_draft_row():
    rng = np.random.default_rng(9)
    V = 777
    for x in _rows(V, rng):
        for k in (0, 1, 50):
            u = int(rng.integers(0, M))
            ref = O.draft_row(x, "f32", k, u)
            for G in GS:
                st, am, ids, c, tok = S.sharded_q_row(x, "f32", k, G, u)
                assert st == ref["status"] and am == ref["argmax"] and tok == ref["sample"]
                assert ids.tolist() == ref["ids"].tolist() and c.tolist() == ref["counts"].tolist()
