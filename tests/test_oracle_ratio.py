"""Pins for the probability-ratio verification oracle (oracle/ratio.py):
the speculative-sampling identity that the output of one verified position
is distributed as p, checked exactly on draw grids; the cross-multiplied
ratio test against a direct comparison of rationals; the residual weights
against max(p - q, 0) with fractions; closed forms; the toy selection-bias
regression of "PP1 q transport and scheduling design", "Depth admission must
not inspect its own future draws"."""
from fractions import Fraction

import numpy as np

from oracle import dyadic24 as O
from oracle import ratio as RT

M = 1 << 24


def _rand_u64(rng, n):
    return [int.from_bytes(rng.bytes(8), "little") for _ in range(n)]


def test_accepts_matches_rational_comparison():
    """u c_x A < A_x 2**88 is U < p(x) / q(x) with U = u / 2**64."""
    rng = np.random.default_rng(71)
    for _ in range(4000):
        A = int.from_bytes(rng.bytes(21), "little") + 1
        ax = int(rng.integers(0, 1 << 62)) << int(rng.integers(0, 88))
        ax = min(ax, A)
        cx = int(rng.integers(1, M + 1))
        u = _rand_u64(rng, 1)[0]
        want = Fraction(u, 1 << 64) < (Fraction(ax, A) / Fraction(cx, M))
        assert RT.accepts(u, cx, ax, A) == want
    # boundaries: p(x) / q(x) = 1/2 accepts exactly the draws below 2**63
    A, ax, cx = 4 << 149, 1 << 149, 1 << 23
    assert RT.accepts(2**63 - 1, cx, ax, A) and not RT.accepts(2**63, cx, ax, A)
    # p(x) >= q(x) accepts every draw
    assert RT.accepts(2**64 - 1, 1 << 22, 1 << 149, 4 << 149)


def test_residual_weights_are_max_p_minus_q():
    rng = np.random.default_rng(73)
    for _ in range(200):
        n = int(rng.integers(1, 12))
        a = [int(v) << 120 for v in rng.integers(0, 1 << 29, n)]
        if sum(a) == 0:
            a[0] = 1 << 149
        A = sum(a)
        ids = np.sort(rng.choice(n, int(rng.integers(1, n + 1)), replace=False))
        cnt = rng.multinomial(M, np.ones(len(ids)) / len(ids))
        r = RT.residual_weights(a, A, ids, cnt)
        q = [Fraction(0)] * n
        for v, c in zip(ids.tolist(), cnt.tolist()):
            q[v] = Fraction(int(c), M)
        for v in range(n):
            assert Fraction(r[v], M * A) == max(Fraction(a[v], A) - q[v], Fraction(0))


def _first_token_distribution(tg_row, ids, cnt, k_acc, k_fin):
    """Distribution of the token emitted at one position, with x drawn from q
    (weight c_x / M) and the acceptance and final draws running over k-bit
    grids, computed with the oracle's own decisions."""
    st, a, A = O.weight_ints(tg_row, "f32")
    assert st == O.ST_OK
    n = len(a)
    r = RT.residual_weights(a, A, ids, cnt)
    res_hist = np.bincount([O.inverse_cdf(r, U << (64 - k_fin)) for U in range(1 << k_fin)], minlength=n) \
        if sum(r) else np.zeros(n, np.int64)
    out = [Fraction(0)] * n
    for x, cx in zip(ids.tolist(), cnt.tolist()):
        if cx == 0:
            continue
        n_acc = sum(RT.accepts(U << (64 - k_acc), int(cx), a[x], A) for U in range(1 << k_acc))
        pacc = Fraction(n_acc, 1 << k_acc)
        out[x] += Fraction(int(cx), M) * pacc
        if pacc < 1:
            for v in range(n):
                out[v] += Fraction(int(cx), M) * (1 - pacc) * Fraction(int(res_hist[v]), 1 << k_fin)
    return out, [Fraction(v, A) for v in a]


def test_one_position_preserves_p_on_draw_grids():
    """q can be far from p and the verified token still follows p: on k-bit
    grids of both draws, the emitted distribution is within 3 * 2**-k of p
    for every token (each grid rounds a probability by at most 2**-k, and
    a token collects at most three such roundings)."""
    rng = np.random.default_rng(79)
    k = 10
    for trial in range(8):
        n = int(rng.integers(2, 7))
        tg = (rng.standard_normal(n) * 2).astype(np.float32)
        if trial % 3 == 0:
            tg[rng.integers(0, n)] = -np.inf
        kq = int(rng.integers(1, n + 1))
        ids = np.sort(rng.choice(n, kq, replace=False))
        cnt = rng.multinomial(M, rng.dirichlet(np.ones(kq)))
        keep = cnt > 0
        ids, cnt = ids[keep], cnt[keep]
        got, p = _first_token_distribution(tg, ids, cnt, k, k)
        assert sum(got) == 1 or abs(sum(got) - 1) <= Fraction(2 * n, 1 << k)
        for v in range(n):
            assert abs(got[v] - p[v]) <= Fraction(3, 1 << k), (trial, v, float(got[v]), float(p[v]))


def test_rational_identity_and_toy_selection_bias():
    """The exact identity behind the pin above, with rational p and q: the
    fixed-depth rule (admit every position before its draw) returns p; the
    selective rule of the pages' toy regression -- q = p uniform on two
    tokens, admit the first draw only when it is token 0, otherwise resample
    target-only -- puts mass 3/4 on token 0 instead of 1/2."""
    rng = np.random.default_rng(83)
    for _ in range(30):
        n = int(rng.integers(1, 6))
        p = [Fraction(int(v)) for v in rng.integers(0, 9, n)]
        if sum(p) == 0:
            p[0] = Fraction(1)
        p = [v / sum(p) for v in p]
        q = [Fraction(int(v)) for v in rng.integers(0, 9, n)]
        if sum(q) == 0:
            q[-1] = Fraction(1)
        q = [v / sum(q) for v in q]
        assert RT.selective_first_draw_mass(p, q, lambda x: True) == p
    half = [Fraction(1, 2), Fraction(1, 2)]
    assert RT.selective_first_draw_mass(half, half, lambda x: True)[0] == Fraction(1, 2)
    assert RT.selective_first_draw_mass(half, half, lambda x: x == 0)[0] == Fraction(3, 4)
    # the same toy case through the integer oracle: target row (0, 0) gives
    # p = (1/2, 1/2), q = (2**23, 2**23); the fixed-depth rule always
    # accepts, so token 0 comes out with mass exactly 1/2
    tg = np.zeros(2, np.float32)
    got, p = _first_token_distribution(tg, np.array([0, 1]), np.array([M // 2, M // 2]), 8, 8)
    assert got == [Fraction(1, 2), Fraction(1, 2)] == p


def _dense_q(x):
    st, ids, c = O.q_row(x, 0)
    assert st == O.ST_OK
    return ids, c


def test_verify_ratio_closed_cases():
    rng = np.random.default_rng(89)
    V = 6
    # q equal to a dyadic p (four equal logits): every proposal is accepted
    base = np.full(V, -np.inf, np.float32)
    base[[0, 2, 3, 5]] = 1.5
    tg = np.stack([base] * 6)
    q = [_dense_q(base)] * 5
    for _ in range(20):
        toks = [int(rng.choice([0, 2, 3, 5])) for _ in range(5)]
        fin = _rand_u64(rng, 1)[0]
        st, acc, tok, nread = RT.verify_ratio(toks, [O.ST_OK] * 5, q, tg, "f32", _rand_u64(rng, 5), fin)
        assert (st, acc, nread) == (O.ST_OK, 5, 6)
        assert tok == O.target_draw_row(base, "f32", fin)[1]
    # a proposal with p(x) = 0 is always rejected; the residual is p itself
    # when q's support holds only tokens with p = 0
    tg = (rng.standard_normal((6, V))).astype(np.float32)
    tg[0, 4] = -np.inf
    q0 = (np.array([4]), np.array([M]))
    qs = [q0] + [_dense_q(tg[i]) for i in range(1, 5)]
    fin = _rand_u64(rng, 1)[0]
    st, acc, tok, nread = RT.verify_ratio([4, 0, 0, 0, 0], [O.ST_OK] * 5, qs, tg, "f32", [0] * 5, fin)
    assert (st, acc, nread) == (O.ST_OK, 0, 1) and tok == O.target_draw_row(tg[0], "f32", fin)[1]
    # a failed draft row ends the chain: target-only draw at that position
    st, acc, tok, nread = RT.verify_ratio([0] * 5, [O.ST_ROW_NAN] + [O.ST_OK] * 4, [None] + qs[1:], tg, "f32",
                                          [0] * 5, fin)
    assert (st, acc, nread) == (O.ST_OK, 0, 1) and tok == O.target_draw_row(tg[0], "f32", fin)[1]
    # refusals: token out of range, zero q at the token, a refused target row that is read
    assert RT.verify_ratio([V, 0, 0, 0, 0], [O.ST_OK] * 5, qs, tg, "f32", [0] * 5, 0)[0] == O.ST_DRAFT_INVALID
    assert RT.verify_ratio([3, 0, 0, 0, 0], [O.ST_OK] * 5, qs, tg, "f32", [0] * 5, 0)[0] == O.ST_DRAFT_INVALID
    bad = tg.copy(); bad[0, 1] = np.inf
    assert RT.verify_ratio([4, 0, 0, 0, 0], [O.ST_OK] * 5, qs, bad, "f32", [0] * 5, 0)[:2] == (O.ST_TARGET_INVALID, 0)
    # a refused row after the one that ends the request is never read
    late = tg.copy(); late[3, 1] = np.nan
    assert RT.verify_ratio([4, 0, 0, 0, 0], [O.ST_OK] * 5, qs, late, "f32", [0] * 5, fin)[0] == O.ST_OK


def test_verify_ratio_matches_step_by_step_brute_force():
    """Random requests against a step-by-step evaluation with fractions."""
    rng = np.random.default_rng(97)
    V = 7
    for _ in range(60):
        tg = (rng.standard_normal((6, V)) * 1.5).astype(np.float32)
        dr = (rng.standard_normal((5, V)) * 1.5).astype(np.float32)
        qs, toks = [], []
        for i in range(5):
            k = int(rng.integers(0, 4))
            st, ids, c = O.q_row(dr[i], k)
            qs.append((ids, c))
            toks.append(int(O.sample(ids, c, int(rng.integers(0, M)))[1]))
        ad, fin = _rand_u64(rng, 5), _rand_u64(rng, 1)[0]
        got = RT.verify_ratio(toks, [O.ST_OK] * 5, qs, tg, "f32", ad, fin)
        for i in range(6):
            st, a, A = O.weight_ints(tg[i], "f32")
            p = [Fraction(v, A) for v in a]
            if i == 5:
                want = (O.ST_OK, 5, O.inverse_cdf(a, fin), 6)
                break
            qi = [Fraction(0)] * V
            for v, c in zip(qs[i][0].tolist(), qs[i][1].tolist()):
                qi[v] = Fraction(int(c), M)
            x = toks[i]
            if Fraction(ad[i], 1 << 64) < p[x] / qi[x]:
                continue
            res = [max(p[v] - qi[v], Fraction(0)) for v in range(V)]
            tot = sum(res)
            # first v whose cumulative residual share exceeds U
            run, tok = Fraction(0), None
            for v in range(V):
                run += res[v] / tot
                if run > Fraction(fin, 1 << 64):
                    tok = v
                    break
            want = (O.ST_OK, i, tok, i + 1)
            break
        assert got == want
