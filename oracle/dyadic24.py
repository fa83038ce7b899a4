"""Plain CPU oracle for the DSpark vocabulary-wide propose / dyadic24 / verify step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library and imports
nothing from the ``vocab_wide_draft_amd`` package.

It is deliberately slow and literal: numpy is used for array handling, IEEE
binary64 division and a sort; every count, sum and comparison that decides an
integer result is done with exact Python integers.  Sources, cited by page
title and section:

* "PP1 q transport and scheduling design", section "Distribution contract and
  precision" -- the ``dyadic24-standard-v1`` categorical q: FP32-rounded
  weights, exact normalisation, integer counts that sum to M = 2**24,
  floor plus largest remainders with ties to the lowest global token ID,
  FP64 allocation arithmetic with the ``0 <= remaining < M`` and exact-sum
  assertions, rejection of NaN / +inf / zero mass with -inf masks allowed,
  sparse top-k support normalised within the support, and sampling by the
  first exact cumulative count strictly greater than a 24-bit draw.
* "Remote DSpark drafter -- wire and state contract (DSV41-OFFLOAD)",
  section 2 (greedy argmax, lowest index on ties; N = 5 block positions,
  anchor-as-first) and section 6.3 (failed entries report id 0 and
  confidence 0.0; confidences must lie in [0, 1]).
* "DeepSeek-V4.1 DSpark", section "State and sampling contracts" (greedy
  verification matches the target argmax over the anchor plus up to five
  proposals and commits the accepted prefix).

Readings where the pages leave a step open:
confidence is the softmax max-probability 1 / sum(exp(x - m)); the weight of
a token is RN32(exp(RN32(x - m))) correctly rounded; S is summed exactly and
rounded once to binary64; the remaining assertion also requires
remaining <= #{r > 0}; any nonzero row status zeroes every output of the row.

Parity pins: every function here is checked in ``tests/test_oracle_*.py``
against brute force, closed forms, invariants or an independent
high-precision evaluation.  No function is "parity unpinned".
"""
from __future__ import annotations

import math
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np

M = 1 << 24  # total dyadic mass, "PP1 q transport ...", "Distribution contract"
N_DRAFT = 5  # block positions, "Remote DSpark drafter -- wire and state contract", section 2
N_TARGET = N_DRAFT + 1  # anchor + five proposals, "DeepSeek-V4.1 DSpark"

ST_OK = 0
ST_ROW_NAN = 1
ST_ROW_POSINF = 2
ST_ROW_ZERO_MASS = 3
ST_DRAW_RANGE = 4
ST_ALLOC_INCONSISTENT = 5
ST_TARGET_INVALID = 6
ST_DRAFT_INVALID = 7
ST_BAD_WEIGHT = 8  # weights-only allocation: a weight below 0 or above 1
ST_BAD_TOPK = 9

SEMANTIC_ID = "dyadic24-standard-v1"

DT_F32 = "f32"
DT_BF16 = "bf16"


# --------------------------------------------------------------------------
# input decoding
# --------------------------------------------------------------------------
def to_f32(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact conversion of one logit row to binary32.

    bf16 logits are the top 16 bits of a binary32 value, so widening is a
    shift of the bit pattern; binary32 rows are returned as they are.
    """
    if dtype == DT_BF16:
        bits = np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32)
    if dtype == DT_F32:
        return np.asarray(raw, dtype=np.float32)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# row validity, argmax, confidence
# --------------------------------------------------------------------------
def row_status(x: np.ndarray) -> int:
    """Validity of a logit row ("Distribution contract and precision").

    NaN anywhere -> ROW_NAN; otherwise any +inf -> ROW_POSINF; otherwise a row
    whose entries are all -inf has zero effective mass -> ROW_ZERO_MASS.
    -inf entries are allowed masks.  An empty row has zero mass.
    """
    if x.size == 0:
        return ST_ROW_ZERO_MASS
    if np.isnan(x).any():
        return ST_ROW_NAN
    if np.isposinf(x).any():
        return ST_ROW_POSINF
    if np.isneginf(x).all():
        return ST_ROW_ZERO_MASS
    return ST_OK


def argmax_first(x: np.ndarray) -> tuple[float, int]:
    """Row maximum and the lowest index attaining it ("Remote DSpark drafter -- wire and state
    contract", section 2:
    greedy argmax resolves ties to the lower vocabulary index).  IEEE
    comparison, so -0.0 and +0.0 are equal."""
    m = float(x.max())
    hits = [i for i in np.flatnonzero(x == np.float32(m))]
    return m, int(hits[0])


def confidence(x: np.ndarray, m: float) -> np.float32:
    """Softmax probability of the argmax token: 1 / sum_v exp(x_v - m).

    x_v - m is formed in binary64 (exact for binary32 operands of the ranges
    used here), the exponentials in binary64 and the sum with math.fsum, then
    the reciprocal is rounded to binary32.
    """
    t = np.exp(x.astype(np.float64) - m)
    s = math.fsum(t.tolist())
    return np.float32(1.0 / s)


# --------------------------------------------------------------------------
# correctly rounded binary32 exponential
# --------------------------------------------------------------------------
def round_to_f32(q: Fraction) -> np.float32:
    """Round a non-negative rational to the nearest binary32, ties to even,
    with gradual underflow.  Pure integer arithmetic."""
    if q < 0:
        raise ValueError("negative")
    if q == 0:
        return np.float32(0.0)
    num, den = q.numerator, q.denominator
    e = num.bit_length() - den.bit_length()  # 2**e <= q < 2**(e+2)
    if Fraction(2) ** e > q:
        e -= 1
    if Fraction(2) ** (e + 1) <= q:
        e += 1
    # now 2**e <= q < 2**(e+1)
    qe = max(e, -126) - 23  # quantum of the binade (fixed 2**-149 below 2**-126)
    scaled = q / (Fraction(2) ** qe)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    if n * 2.0**qe > float(np.finfo(np.float32).max):
        return np.float32(np.inf)
    return np.float32(float(n) * 2.0**qe)


def _exp_f32_decimal(d: float) -> np.float32:
    """RN32(exp(d)) from a 60-digit decimal exponential (the decimal module
    rounds exp correctly to the context precision); the result is accepted
    only if the rounding is the same at both ends of the decimal's error
    interval."""
    with localcontext() as ctx:
        ctx.prec = 60
        val = Decimal(d).exp()
    f = Fraction(val)
    eps = Fraction(1, 10**57)
    lo, hi = round_to_f32(f * (1 - eps)), round_to_f32(f * (1 + eps))
    if lo != hi:
        raise ArithmeticError(f"exp({d!r}) too close to a binary32 midpoint")
    return lo


def cr_exp_f32(d: np.ndarray) -> np.ndarray:
    """w = RN32(exp(d)) for binary32 d <= 0, correctly rounded.

    exp(-inf) = 0.  A binary64 exponential (error far below 2**-40 relative)
    decides the binary32 rounding whenever the whole interval
    y * (1 -+ 2**-40) rounds to the same binary32; the few remaining inputs
    are decided by the decimal evaluation above.
    """
    d = np.asarray(d, dtype=np.float32)
    if (d > 0).any() or np.isnan(d).any():
        raise ValueError("weights are only defined for d <= 0")
    y = np.exp(d.astype(np.float64))
    lo = (y * (1.0 - 2.0**-40)).astype(np.float32)
    hi = (y * (1.0 + 2.0**-40)).astype(np.float32)
    out = y.astype(np.float32)
    for i in np.flatnonzero(lo != hi):
        out.flat[i] = _exp_f32_decimal(float(d.flat[i]))
    return out


def weights(x_support: np.ndarray, m: float) -> np.ndarray:
    """FP32-rounded weights ("Distribution contract": the FP32 helper first
    rounds weights): d = RN32(x - m) as a binary32 subtraction, then
    w = RN32(exp(d)); -inf logits give weight 0."""
    d = (np.asarray(x_support, dtype=np.float32) - np.float32(m)).astype(np.float32)
    return cr_exp_f32(d)


# --------------------------------------------------------------------------
# dyadic24 counts
# --------------------------------------------------------------------------
def exact_sum_scaled(w: np.ndarray) -> int:
    """A = sum_v w_v * 2**149 as an exact integer (every binary32 is an
    integer multiple of 2**-149)."""
    total = 0
    for v in np.asarray(w, dtype=np.float32).astype(np.float64).tolist():
        total += int(v * 2.0**149)
    return total


def dyadic24_counts(w: np.ndarray) -> tuple[int, np.ndarray]:
    """Integer counts c_v >= 0 with sum M from non-negative binary32 weights.

    "Distribution contract and precision": floor plus largest remainders,
    ties by lowest token index, FP64 allocation arithmetic, assert
    0 <= remaining < M and the exact final sum; refuse an inconsistent
    allocation.  Steps:
      S   = sum w exactly;  S64 = RN64(S)
      p_v = RN64(w_v / S64) (IEEE division);  y_v = p_v * 2**24 (exact)
      c_v = floor(y_v);  r_v = y_v - c_v (exact)
      remaining = M - sum c_v; require 0 <= remaining <= #{v: r_v > 0}
      the `remaining` largest r_v, ties to the lowest index, get +1.
    Returns (status, counts int64[n]); an inconsistent or zero-mass input
    returns a zero vector with its status.
    """
    w = np.asarray(w, dtype=np.float32)
    n = w.size
    zero = np.zeros(n, dtype=np.int64)
    if np.isnan(w).any():
        return ST_ROW_NAN, zero
    if np.isposinf(w).any():
        return ST_ROW_POSINF, zero
    if (w < 0).any() or (w > 1).any():  # normalised weights lie in [0, 1]
        return ST_BAD_WEIGHT, zero
    a = exact_sum_scaled(w)
    if a == 0:
        return ST_ROW_ZERO_MASS, zero
    s64 = float(Fraction(a, 1 << 149))  # correctly rounded int/int division
    p = w.astype(np.float64) / s64
    y = p * float(M)
    c = np.floor(y)
    r = y - c
    counts = c.astype(np.int64)
    remaining = M - int(sum(int(v) for v in counts.tolist()))
    positive = int(np.count_nonzero(r > 0))
    if remaining < 0 or remaining >= M or remaining > positive:
        return ST_ALLOC_INCONSISTENT, zero
    idx = np.arange(n)
    order = np.lexsort((idx, -r))  # r descending, then index ascending
    counts[order[:remaining]] += 1
    if int(sum(int(v) for v in counts.tolist())) != M:
        return ST_ALLOC_INCONSISTENT, zero
    return ST_OK, counts


def hamilton_exact(w: np.ndarray) -> tuple[int, np.ndarray]:
    """Qualification only (not the contract): largest remainders on the exact
    rationals p_v = w_v / S, with no binary64 rounding at all."""
    w = np.asarray(w, dtype=np.float32)
    ints = [int(v * 2.0**149) for v in w.astype(np.float64).tolist()]
    a = sum(ints)
    if a == 0:
        return ST_ROW_ZERO_MASS, np.zeros(w.size, dtype=np.int64)
    ys = [Fraction(v * M, a) for v in ints]
    c = [y.numerator // y.denominator for y in ys]
    rem = M - sum(c)
    order = sorted(range(w.size), key=lambda i: (-(ys[i] - c[i]), i))
    for i in order[:rem]:
        c[i] += 1
    return ST_OK, np.array(c, dtype=np.int64)


def topk_support(x: np.ndarray, k: int) -> np.ndarray:
    """Global top-k support ("Sparse support and vocabulary-sharded TP2
    follow-up": deterministic ties).  Order by logit descending, then token
    index ascending; return the first min(k, V) indices in ascending order."""
    idx = np.arange(x.size)
    order = np.lexsort((idx, -x.astype(np.float64)))
    return np.sort(order[: min(k, x.size)])


def q_row(x: np.ndarray, k: int, m: float | None = None) -> tuple[int, np.ndarray, np.ndarray]:
    """dyadic24 q of one valid logit row.  k == 0 means dense (support = all
    tokens); otherwise the top-k support is chosen first, weights are
    normalised within it, and zero-count entries are dropped.

    Returns (status, ids ascending, counts) with counts > 0 only for sparse,
    and the full count vector (ids = arange(V)) for dense.
    """
    if m is None:
        m, _ = argmax_first(x)
    ids = np.arange(x.size) if k == 0 else topk_support(x, k)
    st, c = dyadic24_counts(weights(x[ids], m))
    if st != ST_OK:
        return st, ids[:0], c[:0]
    if k == 0:
        return ST_OK, ids, c
    keep = c > 0
    return ST_OK, ids[keep], c[keep]


# --------------------------------------------------------------------------
# sampling and verification
# --------------------------------------------------------------------------
def sample(ids: np.ndarray, counts: np.ndarray, u) -> tuple[int, int]:
    """Token for a 24-bit draw u: the first id (ascending) whose inclusive
    cumulative count is strictly greater than u.  u >= 2**24 -> DRAW_RANGE."""
    u = int(u)
    if u < 0 or u >= M:
        return ST_DRAW_RANGE, 0
    run = 0
    for tok, c in zip(np.asarray(ids).tolist(), np.asarray(counts).tolist()):
        run += int(c)
        if run > u:
            return ST_OK, int(tok)
    return ST_ALLOC_INCONSISTENT, 0


def sample_many(ids: np.ndarray, counts: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Vectorised form of `sample` for draws already known to be < 2**24."""
    cum = np.cumsum(np.asarray(counts, dtype=np.int64))
    pos = np.searchsorted(cum, np.asarray(u, dtype=np.int64), side="right")
    return np.asarray(ids)[pos]


def verify_greedy(draft_tokens, draft_status, target_argmax, target_status, vocab):
    """Greedy verification of one request ("DeepSeek-V4.1 DSpark", "State and
    sampling contracts"; "Remote DSpark drafter -- wire and state contract",
    section 2, anchor-as-first).

    Target row i (i = 0 is the anchor row) predicts the token at draft
    position i; row 5 only supplies the bonus.  accept_len is the number of
    leading positions whose draft row is valid and whose token equals the
    target argmax; bonus is the target argmax at position accept_len.
    Any invalid target row -> TARGET_INVALID; a valid draft row carrying a
    token outside [0, V) -> DRAFT_INVALID; both give accept_len = bonus = 0.
    """
    if any(s != ST_OK for s in target_status):
        return ST_TARGET_INVALID, 0, 0
    for d, s in zip(draft_tokens, draft_status):
        if s == ST_OK and not (0 <= int(d) < vocab):
            return ST_DRAFT_INVALID, 0, 0
    n = 0
    while n < len(draft_tokens) and draft_status[n] == ST_OK and int(draft_tokens[n]) == int(target_argmax[n]):
        n += 1
    return ST_OK, n, int(target_argmax[n])


# --------------------------------------------------------------------------
# whole rows and requests
# --------------------------------------------------------------------------
def draft_row(raw, dtype, k=None, draw=None):
    """Every output of one draft row.

    k is None -> no q; 0 -> dense q; > 0 -> sparse top-k q.  draw is None ->
    no sample.  Any nonzero status zeroes every output of the row.
    """
    x = to_f32(raw, dtype)
    out = {"status": row_status(x), "argmax": 0, "conf": np.float32(0.0),
           "ids": np.zeros(0, np.int64), "counts": np.zeros(0, np.int64), "sample": 0}
    if out["status"] != ST_OK:
        return out
    m, a = argmax_first(x)
    out["argmax"], out["conf"] = a, confidence(x, m)
    if k is not None:
        st, ids, c = q_row(x, int(k), m)
        if st != ST_OK:
            return {**out, "status": st, "argmax": 0, "conf": np.float32(0.0)}
        out["ids"], out["counts"] = ids, c
        if draw is not None:
            st, tok = sample(ids, c, draw)
            if st != ST_OK:
                return {**out, "status": st, "argmax": 0, "conf": np.float32(0.0),
                        "ids": np.zeros(0, np.int64), "counts": np.zeros(0, np.int64)}
            out["sample"] = tok
    return out


def target_row(raw, dtype):
    x = to_f32(raw, dtype)
    st = row_status(x)
    if st != ST_OK:
        return st, 0
    return ST_OK, argmax_first(x)[1]


def request(draft_rows, target_rows, dtype, mode, topk=None, draws=None):
    """One request: 5 draft rows and 6 target rows (binary32 or bf16 bits).

    mode "greedy": the verified tokens are the draft argmaxes; "sampled": the
    verified tokens are the samples.  topk: None (no q) or per-row k (0 =
    dense).  draws: None or 5 draws.
    """
    vocab = len(target_rows[0])
    drafts = []
    for i in range(N_DRAFT):
        k = None if topk is None else topk[i]
        u = None if draws is None else draws[i]
        drafts.append(draft_row(draft_rows[i], dtype, k, u))
    tg = [target_row(target_rows[i], dtype) for i in range(N_TARGET)]
    toks = [d["argmax"] if mode == "greedy" else d["sample"] for d in drafts]
    rst, acc, bonus = verify_greedy(toks, [d["status"] for d in drafts],
                                    [t[1] for t in tg], [t[0] for t in tg], vocab)
    return {"draft": drafts, "target_status": [t[0] for t in tg],
            "target_argmax": [t[1] for t in tg], "req_status": rst,
            "accept_len": acc, "bonus": bonus}


# --------------------------------------------------------------------------
# the target distribution p and exact draws from it
# --------------------------------------------------------------------------
def weight_ints(raw, dtype):
    """The target distribution of one row at T = 1 as exact integers.

    "PP1 q transport and scheduling design", "Distribution contract and
    precision": the full target p is the distribution after the unchanged
    target processors at T = 1, and the CPU oracle's FP32 helper first rounds
    weights, then normalises them as exact rationals.  Reading: p_v = A_v / A
    with A_v = w_v * 2**149 (w_v = RN32(exp(RN32(x_v - m))), the same weights
    as the draft's q) and A = sum A_v.  Returns (status, [A_v], A); a refused
    row gives (status, None, 0)."""
    x = to_f32(raw, dtype)
    st = row_status(x)
    if st != ST_OK:
        return st, None, 0
    m, _ = argmax_first(x)
    w = weights(x, m)
    a = [int(v * 2.0**149) for v in w.astype(np.float64).tolist()]
    return ST_OK, a, sum(a)


def inverse_cdf(a, u) -> int:
    """Exact inverse-CDF draw from non-negative integer weights a (total > 0)
    with a uniform 64-bit draw u: the first index v (ascending) whose
    inclusive cumulative weight C_v satisfies C_v * 2**64 > u * total, i.e.
    C_v > floor(u * total / 2**64).  Index v is returned for
    ceil(C_v 2**64 / total) - ceil(C_(v-1) 2**64 / total) of the 2**64 draws,
    within one draw of the exact share a_v / total."""
    u = int(u)
    if not 0 <= u < 1 << 64:
        raise ValueError("draw out of range")
    total = sum(int(t) for t in a)
    if total <= 0:
        raise ValueError("zero total")
    t = (u * total) >> 64
    run = 0
    for v, av in enumerate(a):
        run += int(av)
        if run > t:
            return v
    raise AssertionError("unreachable: t < total")


def target_draw_row(raw, dtype, draw):
    """The target's own token for one row: an exact inverse-CDF draw from p
    (weight_ints) with a 64-bit draw.  Returns (status, token); a refused row
    gives token 0."""
    st, a, _ = weight_ints(raw, dtype)
    if st != ST_OK:
        return st, 0
    return ST_OK, inverse_cdf(a, draw)


# --------------------------------------------------------------------------
# stochastic verification
# --------------------------------------------------------------------------
def verify_stochastic(draft_tokens, draft_status, target_rows, dtype, target_draws):
    """Stochastic verification of one request ("DeepSeek-V4.1 DSpark",
    "State and sampling contracts"): each of the 6 target rows draws its own
    token from the target distribution with its own noise; the proposals are
    accepted while they equal those draws, up to the first mismatch, and the
    bonus is the target's draw at that position.  The target distribution is
    the full p of weight_ints (the rounding to dyadic counts belongs to the
    proposal only, "Distribution contract and precision"), drawn exactly
    with one 64-bit draw per row.  The acceptance rule is the greedy one
    applied to the drawn target tokens.  Returns (req_status, accept_len,
    bonus, target tokens, target statuses)."""
    vocab = len(target_rows[0])
    tg = [target_draw_row(target_rows[i], dtype, target_draws[i]) for i in range(N_TARGET)]
    toks, sts = [t[1] for t in tg], [t[0] for t in tg]
    rst, acc, bonus = verify_greedy(draft_tokens, draft_status, toks, sts, vocab)
    return rst, acc, bonus, toks, sts


# --------------------------------------------------------------------------
# vocabulary-sharded propose
# --------------------------------------------------------------------------
def propose_sum(raw, dtype):
    """What a vocabulary-sharded propose must reproduce for one row, whatever
    the shards ("PP1 q transport and scheduling design", "Sparse support and
    vocabulary-sharded TP2 follow-up": shard maxima merged, exact shard sums
    merged as integers): (status, argmax, S64) with S64 = RN64 of the exact
    sum of the weights RN32(exp(RN32(x - m))); a refused row gives (st, 0, 0.0)."""
    x = to_f32(raw, dtype)
    st = row_status(x)
    if st != ST_OK:
        return st, 0, 0.0
    m, a = argmax_first(x)
    A = exact_sum_scaled(weights(x, m))
    return ST_OK, a, math.ldexp(float(A), -149)
