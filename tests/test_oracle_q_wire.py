"""Pins of the wire-form oracle (``oracle.q_wire``) against facts fixed
outside it: IEEE binary32 division in numpy, the exact ratio of a Python
float, round trips through the independently pinned allocation oracle, and
one constructed row per refusal rule of "PP1 q transport and scheduling
design" (sections "Distribution contract and precision" and "Versioned v2
message design")."""
import numpy as np
import pytest

from oracle import dyadic24 as O
from oracle import q_wire as Q

M = 1 << 24


def test_wire_value_matches_ieee_division():
    """c / 2**24 in numpy binary32 (correctly rounded division of the
    correctly rounded c) equals the oracle's rational rounding; for c <= M
    the value is exact (the page states every such value is representable)."""
    rng = np.random.default_rng(7)
    cs = np.concatenate([np.arange(0, 64), M - np.arange(0, 64), [M // 2, M // 3, 5592405, 2796203],
                         rng.integers(0, M + 1, 20000)]).astype(np.uint32)
    got = Q.wire_f32(cs)
    want = np.float32(cs.astype(np.float32)) / np.float32(M)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    for c, v in zip(cs.tolist(), got.tolist()):
        n, d = float(v).as_integer_ratio()
        assert n * M == c * d                         # exact: v * 2**24 == c
    # above M the binary32 conversion rounds to even before the exact scaling
    assert Q.wire_value(M + 1) == np.float32(1.0)
    assert Q.wire_value(M + 3) == np.float32(1.0 + 2.0 ** -22)
    assert Q.wire_value(0).view(np.uint32) == 0       # +0.0, never -0.0


def _dyadic_by_ratio(v: np.float32) -> bool:
    n, d = float(v).as_integer_ratio()
    return d <= M


def test_entry_rules_over_bit_patterns():
    """Every 65,521st binary32 bit pattern (both signs, all exponents,
    subnormals, NaN and infinities): the per-entry verdict agrees with
    classification by the exact ratio of the value."""
    for bits in list(range(0, 1 << 32, 65521)) + [0x7f800000, 0xff800000, 0x7fc00000, 0x80000000,
                                                  0x33800000, 0x33800001, 0x3f800000, 0x3f800001, 1]:
        v = np.array([bits], np.uint32).view(np.float32)[0]
        st, c = Q._entry(v)
        f = float(v)
        if not np.isfinite(f):
            assert st == Q.ST_Q_NONFINITE
        elif bits >> 31:
            assert st == Q.ST_Q_NEGATIVE
        elif not _dyadic_by_ratio(v):
            assert st == Q.ST_Q_NOT_DYADIC
        elif f > 1.0:
            assert st == Q.ST_Q_MASS
        else:
            n, d = f.as_integer_ratio()
            assert st is None and c == n * (M // d)


def _dense_valid(V, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(V) * 2).astype(np.float32)
    st, ids, c = O.q_row(x, 0)
    assert st == O.ST_OK
    return c.astype(np.uint32)


def _sparse_valid(V, k, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(V) * 2).astype(np.float32)
    st, ids, c = O.q_row(x, k)
    assert st == O.ST_OK
    return ids.astype(np.int32), c.astype(np.uint32)


@pytest.mark.parametrize("V,pad", [(1, 3), (7, 1), (300, 4), (1000, 0)])
def test_dense_round_trip(V, pad):
    c = _dense_valid(V, V)
    vals = np.concatenate([Q.wire_f32(c), np.zeros(pad, np.float32)])
    tok = int(np.flatnonzero(c)[-1])
    st, got = Q.check_dense(vals, V, token=tok)
    assert st == O.ST_OK and np.array_equal(got, c)
    st, got = Q.check_dense(vals, V)
    assert st == O.ST_OK and np.array_equal(got, c)


@pytest.mark.parametrize("V,k", [(50, 8), (400, 32), (300, 300)])
def test_sparse_round_trip(V, k):
    ids, c = _sparse_valid(V, k, V + k)
    vals = Q.wire_f32(c)
    st, got = Q.check_sparse(ids, vals, len(ids), k, 64 if k < 64 else k, V, token=int(ids[0]))
    assert st == O.ST_OK
    assert np.array_equal(got[: len(ids)], c) and not got[len(ids):].any()


def test_dense_refusals():
    """One constructed dense row per rule, each breaking that rule alone."""
    V = 64
    c = _dense_valid(V, 3)
    base = Q.wire_f32(c)
    t = int(np.argmax(c))

    def run(vals, token=t, vocab=V):
        return Q.check_dense(vals, vocab, token=token)[0]

    assert run(base) == O.ST_OK
    for bad, code in [(np.nan, Q.ST_Q_NONFINITE), (np.inf, Q.ST_Q_NONFINITE), (-np.inf, Q.ST_Q_NONFINITE)]:
        v = base.copy(); v[5] = bad
        assert run(v) == code
    v = base.copy(); v[5] = -v[5]                                  # negative value
    assert run(v) == Q.ST_Q_NEGATIVE
    v = base.copy(); v[6] = 0; v[t] = Q.wire_value(int(c[t]) + int(c[6]))
    assert run(v) == O.ST_OK
    v[6] = np.float32(-0.0)                                        # -0.0 is refused
    assert run(v) == Q.ST_Q_NEGATIVE
    v = base.copy(); v[7] = np.nextafter(v[7], np.float32(1))      # one ulp off a multiple of 2**-24
    assert v[7] < 2 ** -1 and run(v) == Q.ST_Q_NOT_DYADIC
    v = base.copy(); v[8] = np.float32(2 ** -25)                   # below the grid
    assert run(v) == Q.ST_Q_NOT_DYADIC
    v = base.copy(); v[9] = np.float32(1.5)                        # a count above M
    assert run(v) == Q.ST_Q_MASS
    v = base.copy(); v[10] += np.float32(2 ** -24)                 # total M + 1
    assert run(v) == Q.ST_Q_MASS
    v = base.copy(); v[t] -= np.float32(2 ** -24)                  # total M - 1
    assert run(v) == Q.ST_Q_MASS
    padded = np.concatenate([base, np.zeros(4, np.float32)])
    assert run(padded) == O.ST_OK
    p = padded.copy(); p[V + 2] = np.float32(-0.0)                 # padding must be +0.0
    assert run(p) == Q.ST_Q_PADDING
    p = padded.copy(); p[V + 3] = np.float32(2 ** -24)
    assert run(p) == Q.ST_Q_PADDING
    p = padded.copy(); p[V] = np.nan                               # padding NaN: a padding fault only
    assert run(p) == Q.ST_Q_PADDING
    assert run(base, token=V) == Q.ST_Q_TOKEN
    assert run(base, token=-1) == Q.ST_Q_TOKEN
    # zero q at the proposed token: move that token's mass to another one
    v = base.copy(); s = int(np.argsort(c)[-2])
    v[s] = Q.wire_value(int(c[s]) + int(c[t])); v[t] = 0
    assert run(v, token=t) == Q.ST_Q_TOKEN and run(v, token=s) == O.ST_OK
    # two rules broken: the smaller code wins, and every count is zero
    v = base.copy(); v[1] = np.nan; v[2] = np.float32(1.5)
    st, got = Q.check_dense(v, V, token=V + 5)
    assert st == Q.ST_Q_NONFINITE and not got.any()


def test_sparse_refusals():
    V, k, kmax = 200, 16, 32
    ids, c = _sparse_valid(V, k, 11)
    vals = Q.wire_f32(c)
    n = len(ids)
    t = int(ids[0])

    def run(i=ids, v=vals, length=n, topk=k, token=t):
        return Q.check_sparse(i, v, length, topk, kmax, V, token=token)[0]

    assert run() == O.ST_OK
    assert run(topk=0) == O.ST_BAD_TOPK and run(topk=kmax + 1) == O.ST_BAD_TOPK
    assert run(length=k + 1) == Q.ST_Q_BAD_LEN and run(length=-1) == Q.ST_Q_BAD_LEN
    i = ids.copy(); i[-1] = V
    assert run(i=i) == Q.ST_Q_BAD_ID
    i = ids.copy(); i[0] = -1
    assert run(i=i, token=int(ids[1])) == Q.ST_Q_BAD_ID
    i = ids.copy(); i[1], i[2] = i[2], i[1]                        # unsorted
    assert run(i=i) == Q.ST_Q_UNSORTED
    # a duplicate id with zero values: still refused
    i = np.concatenate([ids, ids[-1:]]); v = np.concatenate([vals, np.zeros(1, np.float32)])
    assert run(i=i, v=v, length=n + 1, topk=kmax) == Q.ST_Q_UNSORTED
    # a single zero-valued entry is legal
    extra = int(np.setdiff1d(np.arange(V), ids)[-1])
    i = np.sort(np.concatenate([ids, [extra]])).astype(np.int32)
    v = np.zeros(n + 1, np.float32); v[np.searchsorted(i, ids)] = vals
    assert run(i=i, v=v, length=n + 1, topk=kmax) == O.ST_OK
    assert run(i=i, v=v, length=n + 1, topk=kmax, token=extra) == Q.ST_Q_TOKEN   # zero q at the token
    v = vals.copy(); v[3] = np.float32(3e-9)
    assert run(v=v) == Q.ST_Q_NOT_DYADIC
    v = vals.copy(); v[2] = -v[2]
    assert run(v=v) == Q.ST_Q_NEGATIVE
    assert run(length=n - 1) == Q.ST_Q_MASS                         # a dropped entry
    assert run(length=0) == Q.ST_Q_MASS
    assert run(token=extra) == Q.ST_Q_TOKEN                          # token outside the support
    # several rules: the smallest code
    i = ids.copy(); i[1] = i[0]; v = vals.copy(); v[4] = np.inf
    st, got = Q.check_sparse(i, v, n, k, kmax, V, token=t)
    assert st == Q.ST_Q_UNSORTED and not got.any()


def test_margin_closed_forms():
    big = np.finfo(np.float32).max
    assert Q.margin(np.array([1.0, 2.0], np.float32)) == np.float32(1.0)
    assert Q.margin(np.array([3.0, 1.0, 3.0], np.float32)) == 0.0                  # repeated maximum
    assert Q.margin(np.array([-np.inf, 5.0, -np.inf], np.float32)) == big          # one finite logit
    assert Q.margin(np.array([7.0], np.float32)) == big                            # V = 1
    z = Q.margin(np.array([-0.0, 0.0, -1.0], np.float32))
    assert z == 0 and not np.signbit(z)                                             # +0.0
    z = Q.margin(np.array([0.0, -0.0], np.float32))
    assert z == 0 and not np.signbit(z)
    assert Q.margin(np.array([3e38, -3e38], np.float32)) == big                    # overflow
    assert Q.margin(np.array([1.0, np.nan], np.float32)) == 0.0                    # refused rows
    assert Q.margin(np.array([1.0, np.inf], np.float32)) == 0.0
    assert Q.margin(np.full(4, -np.inf, np.float32)) == 0.0
    # binary32 rounding of the difference: 1 - 2**-30 rounds to 1
    assert Q.margin(np.array([1.0, 2.0 ** -30], np.float32)) == np.float32(1.0)


def test_margin_against_partition():
    """Random rows (bf16-like values with repeats, masks): the top two by
    numpy.partition, subtracted in binary32."""
    rng = np.random.default_rng(3)
    for n in (2, 3, 17, 1000):
        for _ in range(40):
            x = np.round(rng.standard_normal(n) * 4, int(rng.integers(0, 3))).astype(np.float32)
            if rng.integers(0, 3) == 0:
                x[rng.random(n) < 0.5] = -np.inf
            if not np.isfinite(x).any():
                x[0] = 1.0
            top = np.partition(x, n - 2)[n - 2:]
            m1, m2 = np.float32(top.max()), np.float32(top.min())
            want = np.finfo(np.float32).max if m2 == -np.inf else np.float32(m1 - m2)
            got = Q.margin(x)
            assert got == want and got >= 0
