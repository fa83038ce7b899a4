"""Plain CPU oracle of the vocabulary-sharded q: what G ranks, each holding a
contiguous shard of the vocabulary, compute and exchange.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library.

Source: "PP1 q transport and scheduling design", section "Sparse support and
vocabulary-sharded TP2 follow-up": local top-k on each shard gives at most
G k candidates, merged by global id with deterministic ties into the exact
global top-k (not an independent local normalisation); for dense sharding
each rank computes its shard's max and sum and the all-reduced values give
the global normalisation, and the count allocation coordinates the remaining
tickets globally; a sharded exact sampler picks the shard by its global count
mass with one leader-owned draw, then the token inside it.

Each function follows those steps shard by shard, with the exchanged
quantities written out as plain lists; the pins check that the results
equal the unsharded definitions of oracle/dyadic24.py, which is what the
pages require ("exact global top-k", one global count vector).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from oracle.dyadic24 import (M, ST_ALLOC_INCONSISTENT, ST_DRAW_RANGE, ST_OK, argmax_first, dyadic24_counts,
                             row_status, to_f32, weights)


def shard_ranges(V: int, G: int):
    """Shard g holds ids [g V / G, (g + 1) V / G) (integer division)."""
    return [(g * V // G, (g + 1) * V // G) for g in range(G)]


def _by_logit(x, ids):
    """ids ordered by logit descending, then id ascending."""
    return sorted(ids, key=lambda v: (-float(x[v]), v))


def sharded_topk(x: np.ndarray, k: int, G: int) -> np.ndarray:
    """Global top-k support from shard-local top-k candidates: each shard
    sends its first min(k, shard size) ids by (logit desc, id asc); the
    leader orders the (at most G k) candidates the same way and keeps k.
    Returns the support ids in ascending order."""
    cands = []
    for lo, hi in shard_ranges(x.size, G):
        cands += _by_logit(x, range(lo, hi))[:k]
    return np.array(sorted(_by_logit(x, cands)[:k]), dtype=np.int64)


def sharded_dense_counts(x: np.ndarray, G: int):
    """Dense dyadic24 counts with the remaining tickets coordinated across
    shards.  Returns (status, counts).

    1. each shard sends its (max, lowest id); the all-reduce gives m;
    2. each shard sends the exact integer sum of its weights
       RN32(exp(RN32(x - m))) scaled by 2**149; the all-reduced sum gives
       S64 = RN64(S) on every rank;
    3. each shard computes p = RN64(w / S64), floors c = floor(p 2**24) and
       exact remainders r, and sends its floor sum;
       remaining = M - sum of the floor sums, with 0 <= remaining <= #{r > 0};
    4. the threshold: ranks exchange their remainders' counts and the
       `remaining` largest remainders over all shards get +1, ties to the
       lowest global id (shards are in id order, so the tie cut goes shard by
       shard)."""
    st = row_status(x)
    if st != ST_OK:
        return st, np.zeros(x.size, np.int64)
    ranges = shard_ranges(x.size, G)
    heads = []
    for lo, hi in ranges:
        seg = x[lo:hi]
        if seg.size and np.isfinite(seg.max()):
            mv = float(seg.max())
            heads.append((mv, lo + int(np.flatnonzero(seg == np.float32(mv))[0])))
    m = max(heads, key=lambda h: (h[0], -h[1]))[0]
    w = weights(x, m)
    shard_sums = [sum(int(v * 2.0**149) for v in w[lo:hi].astype(np.float64).tolist()) for lo, hi in ranges]
    A = sum(shard_sums)
    if A == 0:
        return 3, np.zeros(x.size, np.int64)
    s64 = float(Fraction(A, 1 << 149))
    floors, rems = [], []
    for lo, hi in ranges:
        c, r = [], []
        for v in w[lo:hi].astype(np.float64).tolist():
            y = Fraction(v / s64) * M
            fl = y.numerator // y.denominator
            c.append(fl)
            r.append(y - fl)
        floors.append(c)
        rems.append(r)
    remaining = M - sum(sum(c) for c in floors)
    npos = sum(sum(1 for t in r if t > 0) for r in rems)
    if remaining < 0 or remaining >= M or remaining > npos:
        return ST_ALLOC_INCONSISTENT, np.zeros(x.size, np.int64)
    # every shard's positive remainders, exchanged; the global order is
    # remainder descending, then global id ascending
    pool = [(-r, lo + i) for (lo, _), rs in zip(ranges, rems) for i, r in enumerate(rs) if r > 0]
    winners = {v for _, v in sorted(pool)[:remaining]}
    counts = np.array([c for cs in floors for c in cs], dtype=np.int64)
    for v in winners:
        counts[v] += 1
    assert int(counts.sum()) == M
    return ST_OK, counts


def sharded_sample(ids, counts, V: int, G: int, u):
    """The leader's draw u (24-bit) picks the shard whose cumulative global
    count mass first exceeds u, then the token inside that shard whose
    cumulative count (from the shard's start) exceeds u minus the mass of
    the shards before.  Returns (status, token)."""
    u = int(u)
    if not 0 <= u < M:
        return ST_DRAW_RANGE, 0
    ids = np.asarray(ids).tolist()
    counts = np.asarray(counts).tolist()
    ranges = shard_ranges(V, G)
    mass = [sum(int(c) for v, c in zip(ids, counts) if lo <= v < hi) for lo, hi in ranges]
    before = 0
    for (lo, hi), mg in zip(ranges, mass):
        if u < before + mg:
            run = before
            for v, c in zip(ids, counts):
                if lo <= v < hi:
                    run += int(c)
                    if run > u:
                        return ST_OK, int(v)
        before += mg
    return ST_ALLOC_INCONSISTENT, 0


def sharded_q_row(raw, dtype, k: int, G: int, draw=None):
    """The sharded q of one row and (with a draw) its sample: dense (k == 0)
    with global tickets, or sparse with the merged global top-k support,
    normalised within it (the support's allocation is the unsharded one:
    the leader holds the whole support).  Returns (status, argmax, ids,
    counts, sample) with positive counts only for sparse rows."""
    x = to_f32(raw, dtype)
    st = row_status(x)
    if st != ST_OK:
        return st, 0, np.zeros(0, np.int64), np.zeros(0, np.int64), 0
    m, am = argmax_first(x)
    if k == 0:
        st, c = sharded_dense_counts(x, G)
        ids = np.arange(x.size)
    else:
        ids = sharded_topk(x, k, G)
        st, c = dyadic24_counts(weights(x[ids], m))
        keep = c > 0
        ids, c = ids[keep], c[keep]
    if st != ST_OK:
        return st, 0, np.zeros(0, np.int64), np.zeros(0, np.int64), 0
    tok = 0
    if draw is not None:
        st, tok = sharded_sample(ids, c, x.size, G, draw)
        if st != ST_OK:
            return st, 0, np.zeros(0, np.int64), np.zeros(0, np.int64), 0
    return ST_OK, am, ids, c, tok
