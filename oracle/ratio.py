"""Plain CPU oracle for probability-ratio verification with the dyadic q and
full-vocabulary residual sampling.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library.

Sources, cited by page title and section:

* "PP1 q transport and scheduling design", section "Distribution contract and
  precision", last paragraph: the full target p is the distribution at T = 1;
  ratio tests and full-vocabulary residual sampling use this p and the
  defined (dyadic) q; GPU finite-precision work must be qualified against
  the rational oracle.  Same page, section "Sparse support and
  vocabulary-sharded TP2 follow-up": max(p - q, 0) is formed for every token,
  including tokens outside a sparse q's support.  Same page, section
  "Versioned v2 message design": zero q at the proposed token is refused;
  acceptance and correction draws belong to separate RNG domains.
* "DeepSeek-V4.1 DSpark", section "State and sampling contracts": anchor plus
  five proposals; the accepted prefix is committed.

Everything here is exact: p_v = A_v / A with the integer weights of
``dyadic24.weight_ints``, q_v = c_v / 2**24, draws are uniform 64-bit
integers u standing for U = u / 2**64.

Steps of one request (fixed depth five; no position is admitted or dropped
after looking at its own draw):

* every valid draft row must carry a token in [0, V) with q(token) > 0,
  else DRAFT_INVALID;
* for positions i = 0 .. 4, in order: target row i is read (refused ->
  TARGET_INVALID); a draft row that failed ends the chain and the token at i
  is drawn from p_i (target-only sampling); otherwise the proposal x is
  accepted when U < p_i(x) / q_i(x), i.e. u * c_x * A < A_x * 2**88; on
  rejection the token at i is drawn from the residual max(p_i - q_i, 0),
  whose integer weights are max(2**24 A_v - c_v A, 0), and the request ends;
* after five acceptances the bonus token is drawn from p_5.
The token that ends the request (correction or bonus) uses the request's
final draw.  Rows after the one that ends the request are never read.
"""
from __future__ import annotations

import numpy as np

from oracle.dyadic24 import (N_DRAFT, ST_ALLOC_INCONSISTENT, ST_DRAFT_INVALID, ST_OK, ST_TARGET_INVALID,
                             inverse_cdf, weight_ints)

ACCEPT_SHIFT = 64 + 24  # u / 2**64 < (A_x / A) / (c_x / 2**24)


def q_count(ids, counts, x) -> int:
    """q's count of token x: its entry in the (ascending) support, else 0."""
    for v, c in zip(np.asarray(ids).tolist(), np.asarray(counts).tolist()):
        if int(v) == int(x):
            return int(c)
    return 0


def accepts(u, c_x: int, a_x: int, a_total: int) -> bool:
    """The ratio test for a proposal x drawn from q: accept when
    U = u / 2**64 < p(x) / q(x) with p(x) = a_x / a_total and q(x) = c_x / 2**24
    (c_x > 0), written without division: u c_x A < a_x 2**88."""
    return int(u) * c_x * a_total < a_x << ACCEPT_SHIFT


def residual_weights(a, a_total: int, ids, counts) -> list[int]:
    """Integer weights of max(p - q, 0) over the whole vocabulary, scaled by
    2**24 * A: max(2**24 A_v - c_v A, 0), with c_v = 0 outside q's support."""
    c = [0] * len(a)
    for v, cv in zip(np.asarray(ids).tolist(), np.asarray(counts).tolist()):
        c[int(v)] = int(cv)
    return [max((int(av) << 24) - cv * a_total, 0) for av, cv in zip(a, c)]


def verify_ratio(draft_tokens, draft_status, draft_q, target_rows, dtype, accept_draws, final_draw):
    """Probability-ratio verification of one request.

    draft_tokens[i], draft_status[i]: the proposal at position i and its
    draft row's status; draft_q[i] = (ids, counts) of that row's dyadic q
    (dense: ids = arange(V)); target_rows: the 6 target logit rows; accept_draws:
    5 uniform 64-bit draws (acceptance domain); final_draw: one uniform 64-bit
    draw (correction / bonus domain).

    Returns (req_status, accept_len, token, rows_read): accept_len proposals
    are committed, then `token` (the correction or the bonus).  A refused
    request has accept_len = token = 0.
    """
    vocab = len(target_rows[0])
    cx = [0] * N_DRAFT
    for i in range(N_DRAFT):
        if draft_status[i] != ST_OK:
            continue
        x = int(draft_tokens[i])
        if not 0 <= x < vocab:
            return ST_DRAFT_INVALID, 0, 0, 0
        cx[i] = q_count(*draft_q[i], x)
        if cx[i] == 0:
            return ST_DRAFT_INVALID, 0, 0, 0
    for i in range(N_DRAFT + 1):
        st, a, a_total = weight_ints(target_rows[i], dtype)
        if st != ST_OK:
            return ST_TARGET_INVALID, 0, 0, i + 1
        if i == N_DRAFT or draft_status[i] != ST_OK:
            return ST_OK, i, inverse_cdf(a, final_draw), i + 1
        x = int(draft_tokens[i])
        if accepts(accept_draws[i], cx[i], a[x], a_total):
            continue
        r = residual_weights(a, a_total, *draft_q[i])
        if sum(r) == 0:  # impossible for a q whose counts sum to 2**24
            return ST_ALLOC_INCONSISTENT, 0, 0, i + 1
        return ST_OK, i, inverse_cdf(r, final_draw), i + 1
    raise AssertionError("unreachable")


def selective_first_draw_mass(p, q, admit):
    """Output distribution of the first token under a policy that looks at
    its own draw: x is drawn from q; if admit(x) the position is verified
    (accepted with probability min(1, p/q), else the residual is drawn),
    otherwise the draw is discarded and the token is drawn from p
    (target-only).  p and q are exact rational vectors (fractions).  This is
    the selection that "Depth admission must not inspect its own future
    draws" forbids; the fixed-depth rule is admit = always."""
    from fractions import Fraction

    n = len(p)
    res = [max(p[v] - q[v], Fraction(0)) for v in range(n)]
    rs = sum(res)
    out = [Fraction(0)] * n
    for x in range(n):
        if q[x] == 0:
            continue
        if not admit(x):
            for v in range(n):
                out[v] += q[x] * p[v]
            continue
        acc = min(Fraction(1), p[x] / q[x])
        out[x] += q[x] * acc
        if acc < 1:
            for v in range(n):
                out[v] += q[x] * (1 - acc) * res[v] / rs
    return out

