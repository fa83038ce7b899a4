"""Plain CPU oracle for q on the wire: the FP32 form of a dyadic24 q row, the
receiver's check of it, and the margin a reply entry may carry.

TEST INFRASTRUCTURE ONLY, like ``oracle.dyadic24`` (which it uses for the
constants and for binary32 rounding): only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use it,
and it shares no code with the HIP library.

Sources, cited by page title and section:

* "PP1 q transport and scheduling design", section "Distribution contract and
  precision": q(v) = c_v / M with M = 2**24 is sent as a little-endian binary32
  value; every such value is exact; the receiver multiplies by M, requires an
  integer, and checks the total with 64-bit integers; there is no
  renormalisation on the receiving side.
* "Remote DSpark drafter -- wire and state contract (DSV41-OFFLOAD)",
  section 6.3: the optional margin, top1 - top2 of the logits, finite and
  >= 0 in a reply (readings in ``margin``).
* "PP1 q transport and scheduling design", section "Versioned v2 message
  design": the receiver refuses
  duplicate sparse ids (zeros included), an unsorted or non-canonical
  support, ids outside the vocabulary, non-finite, negative or non-dyadic
  values, a total other than M and a zero q at the proposed token; dense
  padding past the vocabulary must be zero.

Readings where the pages leave a step open (each one is listed with the
design notes):

* the status of a refused row is the smallest code among the rules it breaks,
  so that one row gets one status whatever the order of the checks;
* "negative" is the sign bit, so -0.0 is refused: the wire value of a zero
  count is +0.0;
* a value above 1 is a count above M and is reported as a wrong total;
* a sparse row may hold zero-valued entries (the pages refuse duplicate
  zeros, so single ones are legal); canonical order is strictly ascending id;
* a sparse row declares at most ``topk`` entries, ``0 <= len <= topk``;
* dense padding is the entries in [V, padded) of a row; each must be the bit
  pattern of +0.0, and no other check applies to it;
* the counts recovered by the check are written for a row that passes, and a
  refused row's counts are all zero (failed entries report zeros, as
  everywhere on the path).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from oracle.dyadic24 import M, ST_BAD_TOPK, ST_OK, round_to_f32, row_status

ST_Q_BAD_LEN = 10     # sparse length outside [0, topk]
ST_Q_BAD_ID = 11      # sparse id outside [0, V)
ST_Q_UNSORTED = 12    # sparse ids not strictly ascending (duplicates included)
ST_Q_NONFINITE = 13   # NaN or an infinity
ST_Q_NEGATIVE = 14    # sign bit set (-0.0 included)
ST_Q_NOT_DYADIC = 15  # value * 2**24 not an integer
ST_Q_PADDING = 16     # dense padding entry that is not +0.0
ST_Q_MASS = 17        # a value above 1, or total count != M
ST_Q_TOKEN = 18       # proposed token outside [0, V) or with q = 0


def wire_value(c: int) -> np.float32:
    """Wire value of one count: c / M rounded to binary32 ("Distribution
    contract and precision").  For c <= M the quotient is a multiple of 2**-24
    with at most 25 significant bits and is represented exactly."""
    return round_to_f32(Fraction(int(c), M))


def wire_f32(counts) -> np.ndarray:
    """Wire values of a vector of counts."""
    return np.array([wire_value(c) for c in np.asarray(counts).tolist()], dtype=np.float32)


def _entry(v: np.float32):
    """Checks of one transmitted value.  Returns (failed status or None,
    recovered count or None).  The count is the exact rational v * M."""
    bits = int(np.asarray(v, dtype=np.float32).view(np.uint32))
    f = float(v)
    if f != f or f in (float("inf"), float("-inf")):
        return ST_Q_NONFINITE, None
    if bits >> 31:
        return ST_Q_NEGATIVE, None
    scaled = Fraction(f) * M
    if scaled.denominator != 1:
        return ST_Q_NOT_DYADIC, None
    if scaled > M:
        return ST_Q_MASS, None
    return None, int(scaled)


def check_dense(vals, vocab: int, token=None) -> tuple[int, np.ndarray]:
    """Receiver check of one dense wire row.  ``vals`` holds the transmitted
    entries, the vocabulary first and then any padding (len(vals) >= vocab).
    Returns (status, counts[vocab]); counts are zero unless the status is OK."""
    vals = np.asarray(vals, dtype=np.float32)
    fails = set()
    counts = [0] * vocab
    for v in range(vocab):
        st, c = _entry(vals[v])
        if st is not None:
            fails.add(st)
        else:
            counts[v] = c
    for v in range(vocab, vals.size):
        if int(vals[v:v + 1].view(np.uint32)[0]) != 0:
            fails.add(ST_Q_PADDING)
    if not fails and sum(counts) != M:
        fails.add(ST_Q_MASS)
    if token is not None:
        t = int(token)
        if not (0 <= t < vocab) or counts[t] == 0:
            fails.add(ST_Q_TOKEN)
    if fails:
        return min(fails), np.zeros(vocab, np.uint32)
    return ST_OK, np.array(counts, dtype=np.uint32)


def check_sparse(ids, vals, length: int, topk: int, k_max: int, vocab: int,
                 token=None) -> tuple[int, np.ndarray]:
    """Receiver check of one sparse wire row: ``length`` entries (ids, vals)
    out of a row of at most ``topk`` (1 <= topk <= min(k_max, vocab)).
    Returns (status, counts[k_max]) with the recovered count of entry i at
    position i and zeros past ``length``; all zero unless the status is OK."""
    zero = np.zeros(k_max, np.uint32)
    if not (1 <= topk <= min(k_max, vocab)):
        return ST_BAD_TOPK, zero
    length = int(length)
    if not (0 <= length <= topk):
        return ST_Q_BAD_LEN, zero
    ids = [int(i) for i in np.asarray(ids)[:length].tolist()]
    vals = np.asarray(vals, dtype=np.float32)[:length]
    fails = set()
    counts = [0] * length
    for i in range(length):
        if not (0 <= ids[i] < vocab):
            fails.add(ST_Q_BAD_ID)
        if i > 0 and ids[i] <= ids[i - 1]:
            fails.add(ST_Q_UNSORTED)
        st, c = _entry(vals[i])
        if st is not None:
            fails.add(st)
        else:
            counts[i] = c
    if not fails and sum(counts) != M:
        fails.add(ST_Q_MASS)
    if token is not None:
        t = int(token)
        hit = [counts[i] for i in range(length) if ids[i] == t]
        if not (0 <= t < vocab) or not hit or hit[0] == 0:
            fails.add(ST_Q_TOKEN)
    if fails:
        return min(fails), zero
    out = zero.copy()
    out[:length] = counts
    return ST_OK, out


# --------------------------------------------------------------------------
# the margin of a reply entry
# --------------------------------------------------------------------------
FLT_MAX = np.float32(np.finfo(np.float32).max)


def margin(x) -> np.float32:
    """Margin of one logit row ("Remote DSpark drafter -- wire and state
    contract", section 6.3, HAS_MARGIN: top1 - top2 of the logits; the reply
    must carry a finite value >= 0, and a failed entry carries 0).

    Readings: top2 is the second entry of the row sorted by value, so a
    repeated maximum gives 0; the difference is rounded to binary32 and a
    zero is +0.0; when no second finite logit exists (V = 1, or every other
    logit is -inf) or the difference overflows, the margin is the largest
    finite binary32.  A row the validity rule refuses (NaN, +inf, all -inf)
    has margin 0.
    """
    x = np.asarray(x, dtype=np.float32)
    if row_status(x) != ST_OK:
        return np.float32(0.0)
    v = sorted((float(t) for t in x), reverse=True)
    m1 = v[0]
    m2 = v[1] if len(v) > 1 else float("-inf")
    if m2 == float("-inf"):
        return FLT_MAX
    with np.errstate(over="ignore"):
        d = np.float32(m1) - np.float32(m2)
    if np.isinf(d):
        return FLT_MAX
    return np.float32(0.0) if d == 0 else d
