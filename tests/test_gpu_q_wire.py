"""GPU parity of q on the wire through the C ABI: the binary32 encoder and
the receiver's check ("PP1 q transport and scheduling design", sections
"Distribution contract and precision" and "Versioned v2 message design"),
against ``oracle.q_wire`` row by row, bit for bit.  Inputs are seeded: q rows
come from the oracle's allocation of synthetic logit rows, and every refused
row is one of them with rule-breaking edits made on the host."""
import numpy as np
import pytest
import torch

from oracle import dyadic24 as O
from oracle import q_wire as Q
from vocab_wide_draft_amd import binding as B

from gpu_helpers import dev

pytestmark = pytest.mark.gpu
M = 1 << 24


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def _u32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to(dev())


def _f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


@pytest.mark.parametrize("n,offset", [(50_004, 0), (50_003, 0), (4096, 1)])
def test_encode(n, offset):
    """Every count maps to the oracle's binary32 value, bit for bit, on the
    vector path (aligned, n % 4 == 0) and the scalar path."""
    rng = np.random.default_rng(n + offset)
    c = rng.integers(0, M + 1, n + offset, dtype=np.int64)
    edges = [0, 1, 2, 3, M - 1, M, M + 1, M + 3, 2 ** 25 + 1, 2 ** 32 - 1]
    c[offset:offset + len(edges)] = edges
    c = c.astype(np.uint32)
    dc = _u32(c)[offset:]
    got = B.q_encode(dc).cpu().numpy()
    want = Q.wire_f32(c[offset:])
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # in place
    buf = _u32(c[offset:]) if offset == 0 else None
    if buf is not None:
        B.q_encode(buf, out=buf.view(torch.float32))
        assert np.array_equal(buf.cpu().numpy().view(np.uint32), want.view(np.uint32))


def _valid_dense(V, rng):
    x = (rng.standard_normal(V) * 2).astype(np.float32)
    st, _, c = O.q_row(x, 0)
    assert st == O.ST_OK
    return c.astype(np.int64)


def _valid_sparse(V, k, rng):
    x = (rng.standard_normal(V) * 2).astype(np.float32)
    st, ids, c = O.q_row(x, k)
    assert st == O.ST_OK
    return ids.astype(np.int64), c.astype(np.int64)


def _dense_case(V, P, kind, rng):
    """One dense wire row (P values) with edit `kind`, and a proposed token."""
    c = _dense_valid_cache(V, rng)
    vals = np.concatenate([Q.wire_f32(c), np.zeros(P - V, np.float32)])
    nz = np.flatnonzero(c)
    tok = int(nz[rng.integers(0, nz.size)])
    at = int(rng.integers(0, V))
    if kind == "nan":
        vals[at] = np.nan
    elif kind == "inf":
        vals[at] = np.inf if rng.integers(0, 2) else -np.inf
    elif kind == "neg":
        vals[at] = -vals[at] if vals[at] != 0 else np.float32(-0.0)
    elif kind == "negzero":
        z = np.flatnonzero(c == 0)
        if z.size:
            vals[z[0]] = np.float32(-0.0)
        else:
            vals[at] = np.float32(-0.0)
    elif kind == "offgrid":
        vals[at] = np.nextafter(vals[at], np.float32(1))
    elif kind == "big":
        vals[at] = np.float32(2.0)
    elif kind == "plus1":
        vals[at] = Q.wire_value(int(c[at]) + 1)
    elif kind == "minus1":
        vals[tok] = Q.wire_value(int(c[tok]) - 1)
    elif kind == "pad" and P > V:
        vals[V + int(rng.integers(0, P - V))] = np.float32(2 ** -24) if rng.integers(0, 2) else np.float32(-0.0)
    elif kind == "zerotok":
        s = int(nz[0] if nz[0] != tok else nz[-1])
        vals[s] = Q.wire_value(int(c[s]) + int(c[tok]))
        vals[tok] = 0
    elif kind == "badtok":
        tok = V + int(rng.integers(0, 3)) if rng.integers(0, 2) else -1
    elif kind == "two":
        vals[at] = np.float32(1.5)
        vals[(at + 7) % V] = np.float32(3e-9)
    return vals, tok


_CACHE = {}


def _dense_valid_cache(V, rng):
    key = (V, int(rng.integers(0, 4)))
    if key not in _CACHE:
        _CACHE[key] = _valid_dense(V, np.random.default_rng(key[1] * 1000 + V))
    return _CACHE[key]


DENSE_KINDS = ["ok", "nan", "inf", "neg", "negzero", "offgrid", "big", "plus1", "minus1", "pad", "zerotok",
               "badtok", "two"]


@pytest.mark.parametrize("V,P", [(3001, 3001), (3001, 3003), (3001, 3012), (1, 4), (257, 260), (4096, 4096)])
def test_validate_dense_rows(V, P):
    """Dense rows of every refusal kind, several tiles and a ragged tail,
    padding included; status and recovered counts against the oracle."""
    rng = np.random.default_rng(V * 7 + P)
    rows, toks = [], []
    for kind in DENSE_KINDS * 2:
        v, t = _dense_case(V, P, kind, rng)
        rows.append(v)
        toks.append(t)
    n = len(rows)
    stride = -(-P // 4) * 4 + 4
    buf = np.full((n, stride), np.nan, np.float32)           # past `padded`: never looked at
    buf[:, :P] = np.stack(rows)
    d = _f32(buf)
    out = B.q_validate(V, dense=d, tokens=_i32(toks), padded=P, want_counts=True)
    st, cnt = out["status"].cpu().numpy(), out["dense_counts"].cpu().numpy().view(np.uint32)
    kinds = []
    for j in range(n):
        ws, wc = Q.check_dense(rows[j], V, token=toks[j])
        assert int(st[j]) == ws, (j, DENSE_KINDS[j % len(DENSE_KINDS)], int(st[j]), ws)
        assert np.array_equal(cnt[j], wc), j
        kinds.append(ws)
    # without tokens the token rule is skipped
    out = B.q_validate(V, dense=d, padded=P)
    st2 = out["status"].cpu().numpy()
    for j in range(n):
        assert int(st2[j]) == Q.check_dense(rows[j], V)[0], j
    if V > 1:
        assert {O.ST_OK, Q.ST_Q_NONFINITE, Q.ST_Q_NEGATIVE, Q.ST_Q_NOT_DYADIC, Q.ST_Q_MASS, Q.ST_Q_TOKEN} <= set(kinds)


SPARSE_KINDS = ["ok", "len_hi", "len_neg", "len0", "badid", "negid", "swap", "dup", "dupzero", "zero_ok", "nan",
                "neg", "offgrid", "drop", "zerotok", "notok", "badtok", "two"]


def _sparse_case(V, k, kmax, kind, rng):
    ids, c = _valid_sparse(V, k, rng)
    vals = Q.wire_f32(c)
    ids = ids.copy()
    n = len(ids)
    tok = int(ids[rng.integers(0, n)])
    length = n
    at = int(rng.integers(0, n))
    topk = k
    if kind == "len_hi":
        length = k + 1
    elif kind == "len_neg":
        length = -3
    elif kind == "len0":
        length = 0
    elif kind == "badid":
        ids[-1] = V
    elif kind == "negid" and n > 1:
        ids[0] = -5
        tok = int(ids[1])
    elif kind == "swap" and n > 2:
        ids[0], ids[1] = ids[1], ids[0]
    elif kind in ("dup", "dupzero") and n > 1:
        ids[at if at > 0 else 1] = ids[(at if at > 0 else 1) - 1]
        if kind == "dupzero":
            ids = np.concatenate([ids[:at + 1], ids[at:at + 1], ids[at + 1:]])[: n + 1]
            vals = np.concatenate([vals[:at + 1], np.zeros(1, np.float32), vals[at + 1:]])[: n + 1]
            length, topk = n + 1, min(kmax, V)
    elif kind == "zero_ok":
        free = np.setdiff1d(np.arange(V), ids)
        if free.size and n < min(kmax, V):
            ids = np.sort(np.concatenate([ids, free[:1]]))
            nv = np.zeros(n + 1, np.float32)
            nv[np.searchsorted(ids, ids[np.isin(ids, free[:1], invert=True)])] = vals
            vals, length, topk = nv, n + 1, min(kmax, V)
    elif kind == "nan":
        vals[at] = np.nan
    elif kind == "neg":
        vals[at] = -vals[at]
    elif kind == "offgrid":
        vals[at] = np.float32(1e-9)
    elif kind == "drop":
        length = n - 1
    elif kind == "zerotok" and n > 1:
        o = (at + 1) % n
        vals[o] = Q.wire_value(int(c[o]) + int(c[at]))
        vals[at] = 0
        tok = int(ids[at])
    elif kind == "notok":
        free = np.setdiff1d(np.arange(V), ids)
        if free.size:
            tok = int(free[-1])
    elif kind == "badtok":
        tok = V
    elif kind == "two":
        vals[at] = np.inf
        ids[-1] = V + 1
    ids_row = np.zeros(kmax, np.int32)
    val_row = np.full(kmax, np.nan, np.float32)            # past the length: never looked at
    m = max(0, min(length, len(ids), kmax))
    ids_row[:m] = ids[:m]
    val_row[:m] = vals[:m]
    return ids_row, val_row, length, topk, tok


@pytest.mark.parametrize("V,k,kmax", [(3001, 32, 64), (3001, 1024, 1024), (200, 200, 256), (1, 1, 8)])
def test_validate_sparse_rows(V, k, kmax):
    rng = np.random.default_rng(V + k)
    cases = [_sparse_case(V, k, kmax, kind, rng) for kind in SPARSE_KINDS * 2]
    ids = np.stack([c[0] for c in cases])
    vals = np.stack([c[1] for c in cases])
    lens = np.array([c[2] for c in cases], np.int32)
    topk = np.array([c[3] for c in cases], np.int32)
    toks = np.array([c[4] for c in cases], np.int32)
    out = B.q_validate(V, topk=topk, k_max=kmax, sp_ids=_i32(ids), sp_val=_f32(vals), sp_len=_i32(lens),
                       tokens=_i32(toks), want_counts=True)
    st, cnt = out["status"].cpu().numpy(), out["sp_counts"].cpu().numpy().view(np.uint32)
    seen = set()
    for j in range(len(cases)):
        ws, wc = Q.check_sparse(ids[j], vals[j], int(lens[j]), int(topk[j]), kmax, V, token=int(toks[j]))
        assert int(st[j]) == ws, (j, SPARSE_KINDS[j % len(SPARSE_KINDS)], int(st[j]), ws)
        assert np.array_equal(cnt[j], wc), j
        seen.add(ws)
    if V > 1:
        assert {O.ST_OK, Q.ST_Q_BAD_LEN, Q.ST_Q_BAD_ID, Q.ST_Q_UNSORTED, Q.ST_Q_NONFINITE, Q.ST_Q_MASS} <= seen


def test_validate_mixed_and_bad_topk():
    """Dense and sparse rows in one call, with bad topk values and a dense row
    declared without dense storage in a sparse-only call."""
    V, kmax = 1000, 64
    rng = np.random.default_rng(5)
    dense_rows, sp = [], []
    topk = np.array([0, 32, 0, 64, -1, kmax + 1, 0, 16], np.int32)
    n = len(topk)
    dbuf = np.zeros((n, 1004), np.float32)
    ids = np.zeros((n, kmax), np.int32)
    vals = np.zeros((n, kmax), np.float32)
    lens = np.zeros(n, np.int32)
    toks = np.zeros(n, np.int32)
    for r, k in enumerate(topk.tolist()):
        if k == 0:
            c = _valid_dense(V, rng)
            dbuf[r, :V] = Q.wire_f32(c)
            toks[r] = int(np.argmax(c))
        elif 0 < k <= kmax:
            i, c = _valid_sparse(V, k, rng)
            ids[r, :len(i)] = i
            vals[r, :len(i)] = Q.wire_f32(c)
            lens[r] = len(i)
            toks[r] = int(i[np.argmax(c)])
    out = B.q_validate(V, topk=topk, k_max=kmax, dense=_f32(dbuf), sp_ids=_i32(ids), sp_val=_f32(vals),
                       sp_len=_i32(lens), tokens=_i32(toks), want_counts=True)
    st = out["status"].cpu().numpy()
    dc = out["dense_counts"].cpu().numpy().view(np.uint32)
    sc = out["sp_counts"].cpu().numpy().view(np.uint32)
    for r, k in enumerate(topk.tolist()):
        if k == 0:
            ws, wc = Q.check_dense(dbuf[r], V, token=toks[r])
            assert st[r] == ws and np.array_equal(dc[r], wc)
        else:
            ws, wc = Q.check_sparse(ids[r], vals[r], lens[r], k, kmax, V, token=toks[r])
            assert st[r] == ws and np.array_equal(sc[r], wc)
            if not (1 <= k <= kmax):
                assert ws == O.ST_BAD_TOPK and not dc[r].any()
    # a dense row in a call without dense storage
    out = B.q_validate(V, topk=topk, k_max=kmax, sp_ids=_i32(ids), sp_val=_f32(vals), sp_len=_i32(lens))
    st = out["status"].cpu().numpy()
    assert all(st[r] == O.ST_BAD_TOPK for r in range(n) if topk[r] == 0)


def test_full_chain_at_full_vocabulary():
    """At V = 129,280 (bf16 rows of the mixed workload's kinds): the library's
    own q rows, encoded and checked by the library, all pass with the sampled
    tokens and give back the counts exactly; sampled rows also match the
    oracle's check of the same wire values, and a one-count edit per row is
    refused."""
    from vocab_wide_draft_amd import workloads as W
    V = 129280
    rng = np.random.default_rng(77)
    n = 20
    x = (rng.standard_normal((n, V)) * 2).astype(np.float32)
    x[3] = -np.inf
    x[3, V - 1] = 1.0                                        # one-hot
    bits = W.f32_to_bf16_bits(x)
    d = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev())
    topk = np.array([0, 32, 1024, 0] * 5, np.int32)
    q = B.q_alloc(d, topk=topk, k_max=1024)
    draws = torch.from_numpy(rng.integers(0, M, (n, 1), dtype=np.int64).astype(np.int32)).to(dev())
    st = q["status"].clone()
    tok = B.sample(q, draws, st, V)[:, 0]
    assert (st == 0).all()
    dense_w = B.q_encode(q["dense"])
    sp_w = B.q_encode(q["sp_cnt"])
    out = B.q_validate(V, topk=topk, k_max=1024, dense=dense_w, sp_ids=q["sp_ids"], sp_val=sp_w,
                       sp_len=q["sp_len"], tokens=tok, want_counts=True)
    assert (out["status"] == 0).all()
    dm = torch.from_numpy(topk == 0).to(dev())
    assert torch.equal(out["dense_counts"][dm], q["dense"][dm])
    sm = ~dm
    L = q["sp_len"][sm].long()
    col = torch.arange(1024, device=dev())[None, :]
    keep = col < L[:, None]
    assert torch.equal(out["sp_counts"][sm][keep], q["sp_cnt"][sm][keep])
    assert (out["sp_counts"][sm][~keep] == 0).all()
    # oracle check of a few of the same wire rows
    hw = dense_w.cpu().numpy()
    ht = tok.cpu().numpy()
    for r in (0, 3):
        ws, wc = Q.check_dense(hw[r], V, token=int(ht[r]))
        assert ws == O.ST_OK and np.array_equal(wc, q["dense"][r].cpu().numpy().view(np.uint32))
    # one count moved by 2^-24 in every dense row: refused as a wrong total
    bad = dense_w.clone()
    idx = torch.from_numpy(rng.integers(0, V, n)).to(dev())
    rows = torch.arange(n, device=dev())
    bad[rows, idx] = bad[rows, idx] + 2.0 ** -24
    out = B.q_validate(V, topk=topk, k_max=1024, dense=bad, sp_ids=q["sp_ids"], sp_val=sp_w, sp_len=q["sp_len"],
                       tokens=tok)
    s = out["status"].cpu().numpy()
    assert all(s[r] == Q.ST_Q_MASS for r in range(n) if topk[r] == 0)
    assert all(s[r] == O.ST_OK for r in range(n) if topk[r] != 0)


def _margin_rows(V, rng):
    """Logit rows (binary32 values) for every margin case: ordinary, a
    repeated maximum, one finite logit, +0/-0 maxima, extreme values, the
    maximum in the ragged tail, and the refused kinds."""
    base = (rng.standard_normal(V) * 2).astype(np.float32)
    rows = [base.copy()]
    r = base.copy(); r[V // 2] = r.max(); rows.append(r)
    r = np.full(V, -np.inf, np.float32); r[V - 1] = 2.5; rows.append(r)
    r = np.full(V, -1.0, np.float32); r[0] = -0.0; r[V - 1] = 0.0; rows.append(r)
    r = base.copy(); r[1 % V] = 3e38; r[0] = -3e38; rows.append(r)
    r = base.copy(); r[V - 1] = 50.0; rows.append(r)
    r = np.round(base).astype(np.float32); rows.append(r)                   # many ties
    r = base.copy(); r[V // 3] = np.nan; rows.append(r)
    r = base.copy(); r[V - 1] = np.inf; rows.append(r)
    rows.append(np.full(V, -np.inf, np.float32))
    r = base.copy(); r[::3] = -np.inf; rows.append(r)
    return np.stack(rows)


@pytest.mark.parametrize("V", [1, 2, 7, 257, 3001, 129280, 129283])
def test_margin(V):
    from vocab_wide_draft_amd import workloads as W
    from gpu_helpers import to_dev
    rng = np.random.default_rng(V + 99)
    x = _margin_rows(V, rng)
    for dtype in ("f32", "bf16"):
        raw = W.f32_to_bf16_bits(x) if dtype == "bf16" else x
        got = B.margin(to_dev(raw, dtype)).cpu().numpy()
        for j in range(x.shape[0]):
            f = O.to_f32(raw[j], dtype)
            want = Q.margin(f)
            assert got[j].view(np.uint32) == want.view(np.uint32), (dtype, V, j, got[j], want)


def test_empty_batches():
    """No rows: every new entry point succeeds and launches nothing."""
    V = 1000
    e = torch.empty((0, V), dtype=torch.float32, device=dev())
    assert B.q_encode(torch.empty(0, dtype=torch.int32, device=dev())).numel() == 0
    out = B.q_validate(V, dense=e, want_counts=True)
    assert out["status"].numel() == 0 and out["dense_counts"].numel() == 0
    assert B.margin(torch.empty((0, V), dtype=torch.bfloat16, device=dev())).numel() == 0
    s = B.verify_stochastic(torch.empty((0, V), dtype=torch.bfloat16, device=dev()),
                            torch.empty((0, 5), dtype=torch.int32, device=dev()),
                            torch.empty((0, 6), dtype=torch.int64, device=dev()))
    torch.cuda.synchronize()
    assert s["accept_len"].numel() == 0


def test_largest_vocabulary():
    """Wire rows and margins at V = 2^20 (the largest vocabulary accepted),
    with the most padding accepted, against the oracle."""
    V = 1 << 20
    P = V + 64
    rng = np.random.default_rng(2024)
    pos = rng.choice(V, 3, replace=False)
    c = np.zeros(V, np.int64)
    c[pos] = [M // 2, M // 4, M // 4]
    base = Q.wire_f32(c[pos])
    rows = np.zeros((3, P), np.float32)
    rows[:, pos] = base
    rows[1, V - 1] = np.nan                                  # the last vocabulary entry
    rows[2, P - 1] = np.float32(2 ** -24)                    # the last padding entry
    toks = np.array([pos[0], pos[0], pos[1]], np.int32)
    out = B.q_validate(V, dense=_f32(rows), tokens=_i32(toks), padded=P, want_counts=True)
    st = out["status"].cpu().numpy()
    cnt = out["dense_counts"].cpu().numpy().view(np.uint32)
    for j in range(3):
        ws, wc = Q.check_dense(rows[j], V, token=int(toks[j]))
        assert int(st[j]) == ws and np.array_equal(cnt[j], wc), j
    assert list(st) == [0, Q.ST_Q_NONFINITE, Q.ST_Q_PADDING]
    # margins of full-size rows, the maximum and the runner-up at the far end
    from vocab_wide_draft_amd import workloads as W
    from gpu_helpers import to_dev
    x = (rng.standard_normal((2, V)) * 2).astype(np.float32)
    x[0, V - 1] = 40.0
    x[0, V - 2] = 39.0
    x[1, :] = -np.inf
    x[1, V - 1] = 1.0
    for dtype in ("bf16", "f32"):
        raw = W.f32_to_bf16_bits(x) if dtype == "bf16" else x
        got = B.margin(to_dev(raw, dtype)).cpu().numpy()
        for j in range(2):
            want = Q.margin(O.to_f32(raw[j], dtype))
            assert got[j].view(np.uint32) == want.view(np.uint32), (dtype, j)
