"""Pins for the CPU oracle: each check compares it with something other than
itself -- brute force, hand-worked closed forms, an independent
high-precision evaluation, a library routine on a special case, or an
invariant that the pages' definition implies."""
import itertools
import json
import math
import os
from fractions import Fraction

import mpmath
import numpy as np
import pytest

from oracle import dyadic24 as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
M = 1 << 24


# ----------------------------------------------------------------- rounding
def test_round_to_f32_matches_ieee_cast():
    """Special case that reduces to a library routine: for rationals that are
    binary64 values, RN32 equals numpy's IEEE binary64 -> binary32 cast."""
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.random(3000) * 10.0,
        np.exp(rng.uniform(-110, 0, 3000)),  # includes binary32 subnormals
        np.array([2.0**-150, 2.0**-149, 3 * 2.0**-150, 1.0 + 2.0**-24, 1.0 + 3 * 2.0**-24,
                  (1.0 + 2.0**-23) * 2.0**-127, 2.0**-126 * (1 - 2.0**-24)]),
    ])
    for v in vals:
        assert O.round_to_f32(Fraction(float(v))) == np.float32(v), v


# ---------------------------------------------------------------- exp / weights
def _mp_rn32_exp(d: float) -> np.float32:
    """Independent RN32(exp(d)): mpmath at 100 digits, nearest of the three
    binary32 candidates around a first guess (ties cannot occur for d != 0)."""
    with mpmath.workdps(100):
        e = mpmath.exp(mpmath.mpf(float(d)))
        g = np.float32(float(e))
        cands = {g, np.nextafter(g, np.float32(0)), np.nextafter(g, np.float32(np.inf))}
        return min(cands, key=lambda c: abs(mpmath.mpf(float(c)) - e))


def _near_midpoint_inputs(n_scan=2_000_000, keep=300, seed=7):
    """binary32 d whose exp lies closest to a binary32 rounding midpoint
    (found with binary64, then used as hard cases)."""
    rng = np.random.default_rng(seed)
    d = rng.uniform(-103.0, 0.0, n_scan).astype(np.float32)
    y = np.exp(d.astype(np.float64))
    f = y.astype(np.float32).astype(np.float64)
    ulp = np.spacing(y.astype(np.float32)).astype(np.float64)
    frac = np.abs(np.abs(y - f) / ulp - 0.5)
    return d[np.argsort(frac)[:keep]]


def test_cr_exp_special_values():
    d = np.array([0.0, -0.0, -np.inf, -104.0, -103.97, -200.0, -87.336, -1e-30], np.float32)
    w = O.cr_exp_f32(d)
    assert w[0] == 1.0 and w[1] == 1.0 and w[2] == 0.0 and w[3] == 0.0 and w[5] == 0.0
    assert w[4] > 0 and w[4] < np.float32(2.0**-126)  # subnormal weight kept
    assert w[7] == 1.0


def test_cr_exp_against_mpmath_random_and_hard_cases():
    rng = np.random.default_rng(3)
    d = np.concatenate([
        rng.uniform(-104.0, 0.0, 6000).astype(np.float32),
        -np.abs(rng.standard_normal(2000).astype(np.float32)),
        np.arange(-1040, 1).astype(np.float32) / np.float32(10.0),
        _near_midpoint_inputs(),
    ])
    w = O.cr_exp_f32(d)
    for di, wi in zip(d.tolist(), w.tolist()):
        assert np.float32(wi) == _mp_rn32_exp(di), di


def test_decimal_fallback_matches_mpmath():
    for d in _near_midpoint_inputs(keep=40, seed=11):
        assert O._exp_f32_decimal(float(d)) == _mp_rn32_exp(float(d))


def test_cr_exp_monotone():
    d = np.sort(np.random.default_rng(5).uniform(-104, 0, 200000).astype(np.float32))
    w = O.cr_exp_f32(d)
    assert (np.diff(w.astype(np.float64)) >= 0).all()


def test_weights_argmax_is_one_and_masks_are_zero():
    x = np.array([-np.inf, 3.5, 1.25, 3.5, -2.0], np.float32)
    w = O.weights(x, 3.5)
    assert w[1] == 1.0 and w[3] == 1.0 and w[0] == 0.0
    assert 0 < w[4] < w[2] < 1


# ------------------------------------------------------------------ exact sum
def test_exact_sum_matches_fractions():
    rng = np.random.default_rng(9)
    for _ in range(20):
        w = O.cr_exp_f32(-rng.exponential(20.0, 500).astype(np.float32))
        ref = sum((Fraction(float(v)) for v in w), Fraction(0))
        assert Fraction(O.exact_sum_scaled(w), 1 << 149) == ref


# ------------------------------------------------------------ dyadic24 counts
def test_closed_forms():
    data = json.load(open(os.path.join(GOLDEN, "closed_forms.json")))
    for case in data["cases"]:
        st, c = O.dyadic24_counts(np.array(case["w"], np.float32))
        assert st == O.ST_OK
        assert c.tolist() == case["counts"], case


def _fp64_y(w):
    """y_v from the binary64 definition, written with Fractions."""
    a = sum(Fraction(float(v)) for v in w)
    s64 = float(a)
    return [Fraction(float(v) / s64) * M for v in np.asarray(w, np.float32).astype(np.float64)]


def test_largest_remainder_is_the_least_squares_apportionment_bruteforce():
    """Brute force over every apportionment with c_v in {floor y, floor y + 1}
    and sum M: the oracle's counts minimise sum (c - y)^2, and among equal
    minimisers the extra counts sit on the lowest indices."""
    rng = np.random.default_rng(13)
    trials = 0
    for n in range(1, 8):
        for _ in range(25):
            kind = rng.integers(0, 3)
            if kind == 0:
                w = O.cr_exp_f32(-rng.uniform(0, 6, n).astype(np.float32))
            elif kind == 1:  # few distinct values: remainder ties
                vals = O.cr_exp_f32(-rng.uniform(0, 3, 2).astype(np.float32))
                w = vals[rng.integers(0, 2, n)]
            else:  # zeros and dyadic weights
                w = (rng.integers(0, 5, n) / 4.0).astype(np.float32)
                if not w.any():
                    w[0] = 1
            st, c = O.dyadic24_counts(w)
            assert st == O.ST_OK
            y = _fp64_y(w)
            fl = [math.floor(v) for v in y]
            rem = M - sum(fl)
            best = None
            for extra in itertools.combinations(range(n), rem):
                cand = list(fl)
                for i in extra:
                    cand[i] += 1
                if any(cand[i] > 0 and w[i] == 0 for i in range(n)):
                    continue
                cost = sum((Fraction(cand[i]) - y[i]) ** 2 for i in range(n))
                key = (cost, [-(cand[i] - fl[i]) for i in range(n)])
                if best is None or key < best[0]:
                    best = (key, cand)
            assert c.tolist() == best[1], (w, c, best)
            trials += 1
    assert trials == 175


def test_fp64_definition_agrees_with_exact_hamilton_on_random_rows():
    """The pages define q as the exact rational normalisation of the rounded
    weights; the binary64 allocation must reproduce it on ordinary rows."""
    rng = np.random.default_rng(17)
    for n in (3, 50, 1000, 20000):
        for _ in range(3):
            w = O.cr_exp_f32(-rng.exponential(3.0, n).astype(np.float32))
            a = O.dyadic24_counts(w)
            b = O.hamilton_exact(w)
            assert a[0] == b[0] == O.ST_OK
            assert (a[1] == b[1]).all()


def test_count_invariants():
    rng = np.random.default_rng(19)
    for _ in range(30):
        n = int(rng.integers(1, 3000))
        w = O.cr_exp_f32(-rng.exponential(rng.uniform(0.1, 30), n).astype(np.float32))
        w[rng.random(n) < 0.2] = 0
        if not w.any():
            w[0] = 1
        st, c = O.dyadic24_counts(w)
        assert st == O.ST_OK and int(c.sum()) == M
        assert (c[w == 0] == 0).all()
        y = _fp64_y(w)
        for i in range(n):
            assert math.floor(y[i]) <= c[i] <= math.floor(y[i]) + 1
        order = np.lexsort((np.arange(n), -w.astype(np.float64)))
        cs = c[order]
        assert (np.diff(cs) <= 0).all()  # heavier (or equal and lower-index) never gets fewer


def test_rejections():
    assert O.dyadic24_counts(np.zeros(4, np.float32))[0] == O.ST_ROW_ZERO_MASS
    assert O.dyadic24_counts(np.array([1, np.nan], np.float32))[0] == O.ST_ROW_NAN
    assert O.dyadic24_counts(np.array([1, np.inf], np.float32))[0] == O.ST_ROW_POSINF
    assert O.dyadic24_counts(np.array([1, -1], np.float32))[0] == O.ST_BAD_WEIGHT
    assert O.dyadic24_counts(np.array([1, 1.5], np.float32))[0] == O.ST_BAD_WEIGHT
    assert O.dyadic24_counts(np.array([1, -np.inf], np.float32))[0] == O.ST_BAD_WEIGHT
    st, c = O.dyadic24_counts(np.array([1, -0.0], np.float32))
    assert st == O.ST_OK and c.tolist() == [M, 0]


def test_remaining_assertion_cannot_fail():
    """The binary64 quotients sum to within 2^-27 of M (two roundings of
    relative size 2^-53 each: S64 = RN64(S), p_v = RN64(w_v / S64)), so
    remaining = (M - sum y) + sum r lies in (-1, #{r > 0} + 1): the
    "0 <= remaining <= #{r > 0}" refusal is never taken for weights in
    [0, 1] with a positive sum.  Checked exactly with fractions on weight
    vectors built to push the roundings one way: many equal weights,
    powers of two, one large weight beside many tiny or subnormal ones,
    sums that land on binary64 midpoints."""
    rng = np.random.default_rng(67)
    f32 = np.float32
    cases = [
        np.full(3, 1.0, f32), np.full(7, 0.6, f32), np.full(131072, 1.0, f32), np.full(131071, 0.75, f32),
        np.array([1.0] + [2.0**-149] * 5000, f32), np.array([1.0, 2.0**-53, 2.0**-53], f32),
        np.array([1.0] * 3 + [2.0**-60] * 9, f32), (2.0 ** -rng.integers(0, 149, 4000)).astype(f32),
    ]
    for _ in range(12):
        n = int(rng.integers(2, 20000))
        w = O.cr_exp_f32(-rng.exponential(rng.uniform(0.5, 40), n).astype(f32))
        w[rng.random(n) < 0.1] = rng.choice(w, 1)[0]
        cases.append(w)
    for w in cases:
        S = sum(Fraction(float(v)) for v in w)
        s64 = float(S)
        ys = [Fraction(float(v) / s64) * M for v in w.astype(np.float64)]
        total = sum(ys)
        assert abs(total - M) < Fraction(1, 1 << 27), len(w)
        fl = [y.numerator // y.denominator for y in ys]
        remaining = M - sum(fl)
        assert 0 <= remaining <= sum(1 for y, c in zip(ys, fl) if y != c) < M
        st, c = O.dyadic24_counts(w)
        assert st == O.ST_OK and int(c.sum()) == M


def test_sum_midpoint_rounds_to_even():
    """S = 1 + 2**-53 lies exactly between two binary64 values: RN64 keeps 1,
    so the small token gets p = 2**-53 and y = 2**-29 (count 0)."""
    st, c = O.dyadic24_counts(np.array([1.0, 2.0**-53], np.float32))
    assert st == O.ST_OK and c.tolist() == [M, 0]


# ------------------------------------------------------------------- sampling
def test_sampling_exhaustive_histogram_equals_counts():
    """All 2**24 draws: token v is returned for exactly c_v of them."""
    rng = np.random.default_rng(23)
    w = O.cr_exp_f32(-rng.exponential(2.0, 300).astype(np.float32))
    w[::7] = 0
    st, c = O.dyadic24_counts(w)
    ids = np.arange(300) * 3 + 11
    toks = O.sample_many(ids, c, np.arange(M, dtype=np.int64))
    hist = np.bincount((toks - 11) // 3, minlength=300)
    assert (hist == c).all()


def test_sampling_boundaries_scalar_vs_searchsorted():
    ids = np.array([4, 9, 10, 30])
    c = np.array([5, 0, M - 6, 1])
    cum = np.cumsum(c)
    for u in [0, 4, 5, 6, int(cum[2]) - 1, int(cum[2]), M - 1]:
        st, tok = O.sample(ids, c, u)
        assert st == O.ST_OK and tok == int(O.sample_many(ids, c, [u])[0])
    assert O.sample(ids, c, 0)[1] == 4 and O.sample(ids, c, M - 1)[1] == 30
    assert O.sample(ids, c, 5)[1] == 10  # zero-count token never returned
    assert O.sample(ids, c, M)[0] == O.ST_DRAW_RANGE


# ------------------------------------------------------- argmax, confidence
def test_argmax_first_occurrence_like_numpy():
    rng = np.random.default_rng(29)
    for _ in range(200):
        x = rng.integers(-3, 4, int(rng.integers(1, 50))).astype(np.float32)
        assert O.argmax_first(x)[1] == int(np.argmax(x))
    x = np.array([-1.0, -0.0, 0.0, -0.0], np.float32)
    assert O.argmax_first(x)[1] == 1
    x = np.array([-np.inf, -np.inf, -5.0], np.float32)
    assert O.argmax_first(x)[1] == 2


def test_confidence_closed_forms_and_mpmath():
    V = 1000
    x = np.full(V, -np.inf, np.float32)
    x[17] = 2.5
    assert O.confidence(x, 2.5) == 1.0
    x[3] = x[500] = 2.5
    assert O.confidence(x, 2.5) == np.float32(1 / 3)
    assert O.confidence(np.full(V, -7.25, np.float32), -7.25) == np.float32(1 / V)
    rng = np.random.default_rng(31)
    y = (rng.standard_normal(4000) * 3).astype(np.float32)
    m = float(y.max())
    with mpmath.workdps(50):
        ref = 1 / mpmath.fsum(mpmath.exp(mpmath.mpf(float(v)) - m) for v in y)
    assert abs(float(O.confidence(y, m)) - float(ref)) <= 1e-7 * float(ref)


def test_row_status_constructed():
    f = np.float32
    assert O.row_status(np.array([1, np.nan, np.inf], f)) == O.ST_ROW_NAN
    assert O.row_status(np.array([1, np.inf, -np.inf], f)) == O.ST_ROW_POSINF
    assert O.row_status(np.array([-np.inf] * 3, f)) == O.ST_ROW_ZERO_MASS
    assert O.row_status(np.array([-np.inf, -1e30], f)) == O.ST_OK


# ----------------------------------------------------------------- top-k
def test_topk_against_python_sorted():
    rng = np.random.default_rng(37)
    for _ in range(100):
        n = int(rng.integers(1, 400))
        x = rng.integers(-4, 5, n).astype(np.float32)
        x[rng.random(n) < 0.2] = -np.inf
        x[rng.random(n) < 0.1] = -0.0
        k = int(rng.integers(1, n + 5))
        ref = sorted(sorted(range(n), key=lambda i: (-float(x[i]), i))[:k])
        assert O.topk_support(x, k).tolist() == ref


def test_sparse_with_k_covering_all_finite_equals_dense():
    rng = np.random.default_rng(41)
    x = (rng.standard_normal(300) * 2).astype(np.float32)
    x[rng.random(300) < 0.8] = -np.inf
    nfin = int(np.isfinite(x).sum())
    st_d, ids_d, c_d = O.q_row(x, 0)
    st_s, ids_s, c_s = O.q_row(x, nfin + 3)
    keep = c_d > 0
    assert st_d == st_s == O.ST_OK
    assert ids_s.tolist() == ids_d[keep].tolist() and c_s.tolist() == c_d[keep].tolist()


# ------------------------------------------------------------------ verify
def test_verify_bruteforce():
    rng = np.random.default_rng(43)
    for _ in range(2000):
        t = rng.integers(0, 3, 6).tolist()
        d = rng.integers(0, 3, 5).tolist()
        ds = [0 if rng.random() > 0.1 else 1 for _ in range(5)]
        st, acc, bonus = O.verify_greedy(d, ds, t, [0] * 6, 3)
        mism = [i for i in range(5) if not (ds[i] == 0 and d[i] == t[i])]
        L = mism[0] if mism else 5
        assert (st, acc, bonus) == (O.ST_OK, L, t[L])
        assert acc <= 5
    assert O.verify_greedy([0] * 5, [0] * 5, [0] * 6, [0, 0, 1, 0, 0, 0], 3) == (O.ST_TARGET_INVALID, 0, 0)
    assert O.verify_greedy([0, 7, 0, 0, 0], [0] * 5, [0] * 6, [0] * 6, 3) == (O.ST_DRAFT_INVALID, 0, 0)


def _draw_hist_closed_form(a, k):
    """Histogram of inverse-CDF tokens over the 2**k draws u = U * 2**(64 - k):
    token v takes the U with C_(v-1) 2**k / total <= U < C_v 2**k / total,
    i.e. ceil(C_v 2**k / total) - ceil(C_(v-1) 2**k / total) of them."""
    total = sum(a)
    out, prev, run = [], 0, 0
    for av in a:
        run += av
        cur = -((-run << k) // total)  # ceil(run * 2**k / total)
        out.append(cur - prev)
        prev = cur
    return out


def test_inverse_cdf_exhaustive_small_draws():
    """Every 2**k draw of a k-bit grid: the histogram of the exact inverse-CDF
    draw equals the closed-form floor shares, on weights with zeros, ties and
    a wide dynamic range; a one-hot row always gives its token."""
    rng = np.random.default_rng(59)
    for k in (1, 4, 10, 13):
        for trial in range(6):
            n = int(rng.integers(1, 9))
            bits = int(rng.integers(1, 150))
            a = [int.from_bytes(rng.bytes(19), "little") >> (152 - bits) for _ in range(n)]
            a = [v if rng.random() > 0.3 else 0 for v in a]
            if sum(a) == 0:
                a[-1] = 1
            got = np.bincount([O.inverse_cdf(a, U << (64 - k)) for U in range(1 << k)], minlength=n)
            assert got.tolist() == _draw_hist_closed_form(a, k), (a, k)
    a = [0, 0, 5, 0]
    assert {O.inverse_cdf(a, int(u)) for u in [0, 1, 2**63, 2**64 - 1]} == {2}
    a = [3, 1]  # boundaries: u * 4 / 2**64 crosses 3 at u = 3 * 2**62
    assert O.inverse_cdf(a, 3 * 2**62 - 1) == 0 and O.inverse_cdf(a, 3 * 2**62) == 1
    assert O.inverse_cdf(a, 2**64 - 1) == 1
    with pytest.raises(ValueError):
        O.inverse_cdf(a, 2**64)


def test_weight_ints_pins():
    """p's integer weights are the binary32 weights times 2**149 (exact), the
    argmax token gets 2**149, masked tokens 0, and the constant row gives the
    uniform distribution."""
    x = np.array([-np.inf, 0.5, 2.0, 2.0, -3.0], np.float32)
    st, a, A = O.weight_ints(x, "f32")
    assert st == O.ST_OK and a[0] == 0 and a[2] == a[3] == 1 << 149 and A == sum(a)
    assert Fraction(a[1], 1 << 149) == Fraction(float(O.cr_exp_f32(np.array([-1.5], np.float32))[0]))
    st, a, A = O.weight_ints(np.full(7, -1.25, np.float32), "f32")
    assert a == [1 << 149] * 7 and A == 7 << 149
    assert O.weight_ints(np.array([0.0, np.nan], np.float32), "f32")[0] == O.ST_ROW_NAN


def test_verify_stochastic_pins():
    """Stochastic verification draws each target token exactly from p at
    T = 1: with one-hot target rows every draw gives the argmax, so it equals
    greedy verification; the emitted tokens are the target's own draws
    t_0 .. t_L; the first emitted token over a k-bit grid of draws has the
    closed-form histogram of p's integer weights, including tokens whose
    dyadic24 count would be 0; a refused target row refuses the request."""
    rng = np.random.default_rng(41)
    V = 9
    for _ in range(50):
        tg = np.full((6, V), -np.inf, np.float32)
        am = rng.integers(0, V, 6)
        tg[np.arange(6), am] = 1.0
        d = [int(am[i]) if rng.random() < 0.7 else int((am[i] + 1) % V) for i in range(5)]
        ds = [O.ST_OK] * 5
        draws = [int(v) for v in rng.integers(0, 2**63, 6, dtype=np.uint64) * 2 + 1]
        st, acc, bonus, toks, sts = O.verify_stochastic(d, ds, tg, "f32", draws)
        g = O.verify_greedy(d, ds, list(am), [O.ST_OK] * 6, V)
        assert (st, acc, bonus) == g and toks == list(am)
    for _ in range(50):
        tg = (rng.standard_normal((6, V)) * 1.5).astype(np.float32)
        draws = [int(v) for v in rng.integers(0, 2**63, 6, dtype=np.uint64) * 2]
        toks = [O.target_draw_row(tg[i], "f32", draws[i])[1] for i in range(6)]
        d = [toks[i] if rng.random() < 0.6 else int(rng.integers(0, V)) for i in range(5)]
        st, acc, bonus, t2, _ = O.verify_stochastic(d, [O.ST_OK] * 5, tg, "f32", draws)
        assert st == O.ST_OK and t2 == toks
        assert d[:acc] == toks[:acc] and bonus == toks[acc] and (acc == 5 or d[acc] != toks[acc])
    # a token far in the tail (dyadic24 count 0) is still drawn with its share of p
    x = np.array([0.0, -20.0, -30.0, -2.0], np.float32)
    assert O.q_row(x, 0)[2][2] == 0
    w = O.weights(x, 0.0)
    a = [int(Fraction(float(v)) * (1 << 149)) for v in w]
    k = 16
    hist = np.bincount([O.target_draw_row(x, "f32", U << (64 - k))[1] for U in range(1 << k)], minlength=4)
    assert hist.tolist() == _draw_hist_closed_form(a, k)
    u_tail = -((-(a[0] + a[1]) << 64) // sum(a))  # first draw that reaches token 2
    assert O.target_draw_row(x, "f32", u_tail)[1] == 2 and O.target_draw_row(x, "f32", u_tail - 1)[1] == 1
    tg = np.stack([x] * 6)
    tg2 = tg.copy(); tg2[3, 1] = np.nan
    st, _, _, _, sts = O.verify_stochastic([0] * 5, [O.ST_OK] * 5, tg2, "f32", [0] * 6)
    assert st == O.ST_TARGET_INVALID and sts[3] == O.ST_ROW_NAN


def test_weights_rounds_the_difference_to_binary32():
    """d = RN32(x - m) is a binary32 subtraction: on pairs whose difference is
    not a binary32 value, the weight equals an independent RN32(exp(d)) of
    the difference rounded with fractions, and on many of them it differs
    from the weight of the unrounded binary64 difference (so a subtraction
    in binary64 would fail this pin)."""
    rng = np.random.default_rng(61)
    n_inexact = n_teeth = 0
    for _ in range(600):
        m = np.float32(rng.uniform(1.0, 64.0))
        x = np.float32(m - np.float32(rng.uniform(0.5, 40.0)) + np.float32(rng.uniform(-1e-3, 1e-3)))
        if rng.random() < 0.3:
            x = np.float32(rng.uniform(-1e-4, 1e-4))  # far smaller magnitude than m
        exact = Fraction(float(x)) - Fraction(float(m))
        if exact > 0:
            continue
        d = -O.round_to_f32(-exact)  # RN32 is symmetric
        if Fraction(float(d)) == exact:
            continue
        n_inexact += 1
        w = O.weights(np.array([x], np.float32), float(m))[0]
        assert w == _mp_rn32_exp(float(d)), (x, m)
        if w != _mp_rn32_exp(float(exact)):
            n_teeth += 1
    assert n_inexact > 300 and n_teeth > 20, (n_inexact, n_teeth)


def test_propose_sum_closed_forms():
    """S64 of constant, one-hot and n-equal-maxima rows, and a row whose
    exact sum needs rounding to binary64."""
    V = 1000
    st, a, s = O.propose_sum(np.full(V, 2.5, np.float32), "f32")
    assert (st, a, s) == (O.ST_OK, 0, float(V))
    x = np.full(V, -np.inf, np.float32); x[17] = 3.0
    assert O.propose_sum(x, "f32") == (O.ST_OK, 17, 1.0)
    x[[5, 900]] = 3.0
    assert O.propose_sum(x, "f32") == (O.ST_OK, 5, 3.0)
    # 1 + 2^-60 (twice) + 2^-149 ... : the exact sum rounds once
    x = np.array([0.0] + [-np.inf] * 3, np.float32)
    x[1] = np.float32(-41.58883083359672)          # exp gives a weight far below 2^-53
    st, a, s = O.propose_sum(x, "f32")
    w = O.weights(x, 0.0)
    assert s == 1.0 + float(w[1]) and w[1] > 0      # binary64 sum of two terms, rounded once
    assert O.propose_sum(np.array([1.0, np.nan], np.float32), "f32") == (O.ST_ROW_NAN, 0, 0.0)
