"""GPU parity: the HIP library (through its C ABI) against the CPU oracle,
element by element.  Argmax, tokens, counts, samples, statuses and accept
lengths must match bit-exactly; confidences within 1e-6 relative."""
import math

import numpy as np
import pytest
import torch

from oracle import dyadic24 as O
from vocab_wide_draft_amd import binding as B
from vocab_wide_draft_amd import workloads as W

from gpu_helpers import check_draft_row, check_workload, dev, host, run_fused, to_dev, u32_dev

pytestmark = pytest.mark.gpu

F32, BF16 = "f32", "bf16"


def _bits_bf16(x32):
    return W.f32_to_bf16_bits(np.asarray(x32, np.float32))


# ------------------------------------------------------------ small configs
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("V", [257, 3000, 20011])
def test_configs_small(cfg, V):
    R = {1: 2, 2: 4, 3: 3, 4: 4, 5: 8}[cfg]
    w = W.make(cfg, V=V, R=R, seed=1000 + cfg * 7 + V)
    h = run_fused(w)
    check_workload(w, h, label=f"cfg{cfg} V{V}")


# ------------------------------------------------------------- edge rows
def _edge_rows(V, rng):
    """Constructed draft rows (binary32 values) with a label each."""
    rows = []
    base = (rng.standard_normal(V) * 2).astype(np.float32)
    r = base.copy(); r[V // 2] = np.nan; rows.append(("nan", r))
    r = base.copy(); r[3 % V] = np.inf; rows.append(("posinf", r))
    r = base.copy(); r[3 % V] = np.inf; r[7 % V] = np.nan; rows.append(("nan_and_inf", r))
    rows.append(("all_neginf", np.full(V, -np.inf, np.float32)))
    r = np.full(V, -np.inf, np.float32); r[V - 1] = -3.5; rows.append(("onehot_last", r))
    r = np.zeros(V, np.float32); r[::3] = -0.0; rows.append(("signed_zeros", r))
    r = np.full(V, -np.inf, np.float32); r[0] = -0.0; r[V - 1] = 0.0; rows.append(("zero_pair", r))
    vals = np.array([1.5, 0.25], np.float32)
    rows.append(("two_values", vals[rng.integers(0, 2, V)]))
    rows.append(("constant", np.full(V, 7.0, np.float32)))
    r = np.full(V, -200.0, np.float32); r[0] = 0.0
    tail = np.array([-88.0, -90.5, -100.0, -103.9, -104.5, -87.4, -95.25], np.float32)
    r[1:1 + min(len(tail), V - 1)] = tail[:V - 1]; rows.append(("subnormal_weights", r))
    r = base.copy(); r[rng.random(V) < 0.9] = -np.inf; r[0] = 1.0; rows.append(("mostly_masked", r))
    return rows


def _midpoint_d():
    """A binary32 d whose weight RN32(exp(d)) is an odd multiple of 2^-53 below
    2^-40, so that S = 1 + w is exactly halfway between two binary64 values."""
    for j in range(0, 4000):
        target = (2 * j + 1) * 2.0**-53
        d0 = np.float32(math.log(target))
        ds = d0 + np.arange(-64, 65, dtype=np.float32) * np.spacing(d0)
        w = O.cr_exp_f32(ds.astype(np.float32)).astype(np.float64)
        hit = np.flatnonzero(w == target)
        if hit.size:
            return np.float32(ds[hit[0]])
    raise AssertionError("no binary32 d found")


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("V", [1, 5, 64, 1000, 4099])
def test_edge_rows(dtype, V):
    rng = np.random.default_rng(V)
    rows = [(n, r) for n, r in _edge_rows(V, rng)]
    if dtype == F32 and V >= 2:
        r = np.full(V, -np.inf, np.float32); r[0] = 0.0; r[1] = _midpoint_d(); rows.append(("midpoint_sum", r))
    names = [n for n, _ in rows]
    x = np.stack([r for _, r in rows]).astype(np.float32)
    raw = x if dtype == F32 else _bits_bf16(x)
    ks = [0, min(5, V), min(1024, V), 1]
    for k in ks:
        topk = np.full(len(rows), k, np.int32)
        draws = rng.integers(0, 1 << 24, len(rows), dtype=np.uint32)
        draws[1] = (1 << 24) + 5  # out of range on a row that is invalid anyway
        d = to_dev(raw, dtype)
        q = B.q_alloc(d, topk=topk, k_max=1024)
        pr = B.propose(d)
        torch.cuda.synchronize()
        hq = host(q)
        hp = host(pr)
        for j, name in enumerate(names):
            ref = O.draft_row(raw[j], dtype, k)
            h = {"status": hq["status"], "argmax": hp["argmax"] * (hq["status"] == 0),
                 "conf": hp["conf"] * (hq["status"] == 0), "q": hq}
            check_draft_row(h, j, ref, k, label=f"{dtype} V{V} k{k} {name}")
            st_p = O.row_status(O.to_f32(raw[j], dtype))
            assert int(hp["status"][j]) == st_p


def test_draw_range_and_bad_topk():
    V = 300
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((5, V)) * 2).astype(np.float32)
    t = (rng.standard_normal((6, V)) * 2).astype(np.float32)
    draws = np.array([1, (1 << 24), 5, 0xFFFFFFFF, 7], np.uint32)
    topk = np.array([0, 0, V + 1, 3, -1], np.int32)
    out = B.fused(to_dev(x, F32), to_dev(t, F32), B.SAMPLED, topk=topk, k_max=8, draws=u32_dev(draws))
    torch.cuda.synchronize()
    h = host(out)
    assert h["status"].tolist() == [0, O.ST_DRAW_RANGE, O.ST_BAD_TOPK, O.ST_DRAW_RANGE, O.ST_BAD_TOPK]
    assert h["sample"][1:].tolist() == [0, 0, 0, 0]
    assert not h["q"]["dense"][1].any()
    assert int(h["accept_len"][0]) <= 1


def test_large_tie_groups_dense_f32():
    """More than 2048 equal remainders in one bucket: the refinement passes and
    the index cut by locate."""
    V = 20000
    rng = np.random.default_rng(9)
    vals = np.array([0.0, -0.6931472, -1.25], np.float32)
    x = vals[rng.integers(0, 3, (3, V))]
    x[1, :] = 0.0  # all equal: remainders all equal
    x[2, rng.random(V) < 0.3] = -np.inf
    d = to_dev(x, F32)
    q = host(B.q_alloc(d, topk=None))
    for j in range(3):
        ref = O.draft_row(x[j], F32, 0)
        assert q["status"][j] == 0
        assert (q["dense"][j] == ref["counts"]).all(), j


# --------------------------------------------------- standalone entry points
def test_sample_entry_many_draws():
    V = 1000
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((4, V)) * 2).astype(np.float32)
    x[3, 10:] = -np.inf
    topk = np.array([0, 16, 0, 4], np.int32)
    d = to_dev(x, F32)
    q = B.q_alloc(d, topk=topk, k_max=16)
    st = q["status"].clone()
    draws = rng.integers(0, 1 << 24, (4, 64), dtype=np.uint32)
    draws[:, 0] = 0
    draws[:, 1] = (1 << 24) - 1
    tok = B.sample(q, u32_dev(draws), st, V).cpu().numpy()
    hq = host(q)
    for r in range(4):
        ref = O.draft_row(x[r], F32, int(topk[r]))
        for j in range(64):
            assert tok[r, j] == O.sample(ref["ids"], ref["counts"], int(draws[r, j]))[1]
    # an out-of-range draw and a corrupted count row
    dense = q["dense"]
    dense[2, 5] += 1
    st = q["status"].clone()
    draws[0, 3] = 1 << 24
    tok = B.sample(q, u32_dev(draws), st, V).cpu().numpy()
    assert st.cpu().tolist() == [O.ST_DRAW_RANGE, 0, O.ST_ALLOC_INCONSISTENT, 0]
    assert not tok[0].any() and not tok[2].any()


@pytest.mark.parametrize("k", [0, 1024])
def test_sample_entry_all_2_24_draws(k):
    """Every one of the 2^24 draws, on a full-vocabulary q row (16 copies of
    the row, 2^20 draws each): the token histogram equals the counts
    exactly, for a dense and a sparse row."""
    V = 129280
    rng = np.random.default_rng(27 + k)
    x = (rng.standard_normal((1, V)) * 2).astype(np.float32)
    x[0, 7:40] = -np.inf
    d = to_dev(np.repeat(x, 16, axis=0), F32)
    q = B.q_alloc(d, topk=np.full(16, k, np.int32), k_max=max(k, 1))
    st = q["status"].clone()
    assert (st == 0).all()
    draws = torch.arange(1 << 24, dtype=torch.int64, device=dev()).to(torch.int32).view(16, 1 << 20)
    tok = B.sample(q, draws, st, V)
    torch.cuda.synchronize()
    assert (st == 0).all()
    hist = torch.bincount(tok.view(-1).to(torch.int64), minlength=V).cpu().numpy()
    ref = O.draft_row(x[0], F32, k)
    want = np.zeros(V, np.int64)
    want[ref["ids"]] = ref["counts"]
    assert np.array_equal(hist, want)


def _shared_key_rows(V=3000):
    """Rows whose threshold remainder is shared by distinct table entries:
    the maximum 10.0 (binary32 ulp 2^-20) and values x with
    2^-23 <= |x| <= 2^-21, which are distinct bf16 values above the
    collapse bound 2^-23 but all give RN32(x - 10) = -10, so every one of
    their entries has the weight, the floor and the remainder of the
    collapsed entry.  The largest-remainder cut falls inside that shared key
    and splits it across entries: 2 and 3 entries (the candidate path's tie
    of several entries) and 515 entries (more than a threshold bucket holds:
    the exact path), both handed to the general per-value path."""
    rng = np.random.default_rng(31)
    above = [b | sg for b in range(0x3400, 0x3501) for sg in (0, 0x8000)]
    rows = []
    for distinct, copies in (([0, 0x3480], 60), ([0x3480, 0x3481, 0x3482], 50), ([0] + above, 3)):
        row = np.full(V, 0xFF80, np.uint16)
        pos = rng.permutation(V)
        row[pos[0]] = 0x4120  # 10.0
        k = 1
        for v in distinct:
            for _ in range(copies):
                row[pos[k]] = v
                k += 1
        rows.append(row)
    return np.stack(rows)


@pytest.mark.parametrize("k", [0, 100])
def test_shared_remainder_key_rows(k):
    raw = _shared_key_rows()
    for i in range(raw.shape[0]):  # the oracle splits the shared key across distinct values
        x = O.to_f32(raw[i], BF16)
        st, ids, c = O.q_row(x, 0)
        grp = (raw[i] != 0xFF80) & (x != 10.0)
        up, lo = raw[i][grp & (c == c[grp].max())], raw[i][grp & (c == c[grp].min())]
        assert c[grp].max() == c[grp].min() + 1 and len(set(up.tolist())) >= 2 and len(set(lo.tolist())) >= 2
    draft = np.concatenate([raw, raw[:2]])  # one request of 5 draft rows
    target = np.repeat(raw[:1], 6, axis=0)
    rng = np.random.default_rng(37)
    draws = rng.integers(0, 1 << 24, 5, dtype=np.uint32)
    topk = np.full(5, k, np.int32)
    out = B.fused(to_dev(draft, BF16), to_dev(target, BF16), B.SAMPLED, topk=topk, k_max=max(k, 1),
                  draws=u32_dev(draws))
    torch.cuda.synchronize()
    h = host(out)
    for j in range(5):
        ref = O.draft_row(draft[j], BF16, k, int(draws[j]))
        check_draft_row(h, j, ref, k, f"shared key k={k}")


@pytest.mark.parametrize("dtype,V", [(F32, 129280), (F32, 3001), (BF16, 140001)])
def test_split_streamed_rows_equal_one_workgroup_rows(dtype, V):
    """Streamed dense rows split over several workgroups (a workspace given)
    equal the one-workgroup path and the oracle: q, argmax, confidence,
    sample, verification, with a refused row, a constant row (every id in
    the crossing bin) and sparse rows beside them; target rows (whose
    argmax comes from shard heads then) with NaN, +inf, no finite entry and
    a maximum tied across the first and last shard."""
    R = 2
    rng = np.random.default_rng(V + 3)
    dr = (rng.standard_normal((5 * R, V)) * 2).astype(np.float32)
    dr[3, V // 2] = np.nan
    dr[6, :V // 3] = -np.inf
    dr[7] = 1.25
    tg = (rng.standard_normal((6 * R, V)) * 2).astype(np.float32)
    tg[1, V // 2] = np.nan
    tg[4] = -np.inf
    tg[7, V - 1] = np.inf
    tg[9, [0, V - 1]] = tg[9].max() + 1
    raw_d = W.f32_to_bf16_bits(dr) if dtype == BF16 else dr
    raw_t = W.f32_to_bf16_bits(tg) if dtype == BF16 else tg
    topk = np.array([0, 0, 16, 0, 0, 0, 0, 0, 64, 0], np.int32)
    draws = rng.integers(0, 1 << 24, 5 * R, dtype=np.uint32)
    d, t = to_dev(raw_d, dtype), to_dev(raw_t, dtype)
    a = host(B.fused(d, t, B.SAMPLED, topk=topk, k_max=64, draws=u32_dev(draws), split=True))
    b = host(B.fused(d, t, B.SAMPLED, topk=topk, k_max=64, draws=u32_dev(draws), split=False))
    torch.cuda.synchronize()
    for k in ("argmax", "status", "sample", "target_argmax", "target_status", "accept_len", "bonus", "req_status"):
        assert np.array_equal(a[k], b[k]), k
    for i in range(6 * R):
        x = O.to_f32(raw_t[i], dtype)
        st = O.row_status(x)
        assert a["target_status"][i] == st, i
        assert a["target_argmax"][i] == (O.argmax_first(x)[1] if st == O.ST_OK else 0), i
    assert a["target_argmax"][9] == 0 and a["target_status"][1] != 0 and a["target_status"][4] != 0
    for j in range(5 * R):
        ref = O.draft_row(raw_d[j], dtype, int(topk[j]), int(draws[j]))
        check_draft_row(a, j, ref, int(topk[j]), "split")
    dense = topk == 0
    assert np.array_equal(a["q"]["dense"][dense], b["q"]["dense"][dense])


def test_verify_entry():
    V = 500
    rng = np.random.default_rng(23)
    R = 6
    t = (rng.standard_normal((R * 6, V)) * 2).astype(np.float32)
    t[6 * 2 + 4, 0] = np.nan  # request 2: invalid target row
    tam = np.array([O.argmax_first(r)[1] if O.row_status(r) == 0 else 0 for r in t])
    dt = np.zeros((R, 5), np.int32)
    ds = np.zeros((R, 5), np.int32)
    for r in range(R):
        L = r % 6
        for i in range(5):
            dt[r, i] = tam[r * 6 + i] if i < L else (tam[r * 6 + i] + 1) % V
    ds[4, 1] = O.ST_ROW_NAN  # invalid draft row stops acceptance
    dt[5, 3] = V + 3  # valid row, token out of range
    out = host(B.verify_greedy(to_dev(t, F32), torch.from_numpy(dt).to(dev()), torch.from_numpy(ds).to(dev())))
    for r in range(R):
        tst = [O.row_status(t[r * 6 + i]) for i in range(6)]
        tgt = [0 if s else int(tam[r * 6 + i]) for i, s in enumerate(tst)]
        ref = O.verify_greedy(dt[r].tolist(), ds[r].tolist(), tgt, tst, V)
        assert (int(out["req_status"][r]), int(out["accept_len"][r]), int(out["bonus"][r])) == ref, r
        assert out["target_argmax"][r * 6:(r + 1) * 6].tolist() == tgt


def test_q_alloc_weights_entry():
    rng = np.random.default_rng(29)
    n = 2500
    rows = [
        O.cr_exp_f32(-rng.exponential(3.0, n).astype(np.float32)),
        np.concatenate([[1.0, 2.0**-53], np.zeros(n - 2)]).astype(np.float32),  # binary64 tie in S
        np.concatenate([[2.0**-149] * 7, np.zeros(n - 7)]).astype(np.float32),  # subnormals only
        np.concatenate([[1.0, np.nan], np.zeros(n - 2)]).astype(np.float32),
        np.concatenate([[1.0, np.inf], np.zeros(n - 2)]).astype(np.float32),
        np.concatenate([[1.0, -0.5], np.zeros(n - 2)]).astype(np.float32),
        np.concatenate([[1.5], np.zeros(n - 1)]).astype(np.float32),
        np.zeros(n, np.float32),
        np.concatenate([[-0.0, 0.25, 0.25, 0.25], np.zeros(n - 4)]).astype(np.float32),
        np.full(n, 2.0**-30, np.float32),
    ]
    w = np.stack(rows)
    counts, st = B.q_alloc_weights(torch.from_numpy(w).to(dev()))
    counts, st = counts.cpu().numpy(), st.cpu().numpy()
    for j, row in enumerate(rows):
        s, c = O.dyadic24_counts(row)
        assert int(st[j]) == s, j
        assert (counts[j] == c).all(), j


def test_cr_expf_sampled_and_hard_cases():
    rng = np.random.default_rng(31)
    d = np.concatenate([
        rng.uniform(-104.0, 0.0, 1 << 20).astype(np.float32),
        -np.abs(rng.standard_normal(1 << 18)).astype(np.float32) * np.float32(1e-3),
        np.array([0.0, -0.0, -np.inf, -104.0, -103.972, -87.33654, -1e-45, -104.00001, -105.0, -1000.0,
                  -3.4e38], np.float32),
        rng.uniform(-104.0, -86.0, 1 << 16).astype(np.float32),  # subnormal and near-subnormal results
    ])
    y = np.exp(d.astype(np.float64))
    f = y.astype(np.float32).astype(np.float64)
    ulp = np.spacing(y.astype(np.float32)).astype(np.float64)
    hard = d[np.argsort(np.abs(np.abs(y - f) / np.where(ulp > 0, ulp, 1) - 0.5))[:4096]]
    d = np.concatenate([d, hard])
    got = B.cr_expf(torch.from_numpy(d).to(dev())).cpu().numpy()
    ref = O.cr_exp_f32(d)
    bad = np.flatnonzero(got.view(np.uint32) != ref.view(np.uint32))
    assert bad.size == 0, (d[bad[:5]], got[bad[:5]], ref[bad[:5]])


# ------------------------------------------- rows aimed at the value table
def _table_rows(V, rng):
    """bf16 draft rows (as binary32 values) that exercise the compressed value
    table of the bf16 path: near-zero logits sharing one entry, top-k
    thresholds inside that entry, windows that start above zero, maxima on
    both sides of the table's size limit, negative maxima, bf16 subnormals."""
    rows = []
    base = (rng.standard_normal(V) * 2).astype(np.float32)
    tiny = (rng.choice([-1.0, 1.0], V) * np.exp(rng.uniform(np.log(1e-12), np.log(1e-7), V))).astype(np.float32)
    r = base.copy(); sel = rng.random(V) < 0.4; r[sel] = tiny[sel]; r[0] = 8.0; rows.append(("tiny_mass", r))
    r = tiny.copy(); r[V // 3] = 8.0; r[V // 2] = 5.0; rows.append(("tiny_only", r))
    r = rng.uniform(90.0, 200.0, V).astype(np.float32); r[7 % V] = 200.0; rows.append(("window_above_zero", r))
    r = (rng.uniform(-1.0, 1.0, V) * 2.0**-20).astype(np.float32)
    neg = rng.random(V) < 0.5
    r[neg] = -rng.uniform(0.0, 100.0, int(neg.sum())).astype(np.float32)
    r[1 % V] = 2.0**-20; rows.append(("max_2^-20", r))
    r = (-np.abs(rng.standard_normal(V)) * 3).astype(np.float32); r[2 % V] = 1e-30; rows.append(("max_1e-30", r))
    r = rng.uniform(-50.0, -10.0, V).astype(np.float32); rows.append(("negative_max", r))
    r = base.copy(); r[rng.random(V) < 0.3] = np.float32(3e-39); r[rng.random(V) < 0.3] = np.float32(-5e-39)
    rows.append(("subnormals", r))
    vals = np.array([0.0, 1e-9, -1e-9, 2.0, -1e-12], np.float32)
    rows.append(("tiny_dups", vals[rng.integers(0, vals.size, V)]))
    # a tie entry holding a third of the row below a few hundred distinct
    # larger values: top-k thresholds inside a tie too large to list
    r = (rng.standard_normal(V) * 2 - 10).astype(np.float32)
    r[rng.random(V) < 0.33] = 2.0
    hi = rng.choice(V, min(200, V), replace=False)
    r[hi] = rng.uniform(5.0, 10.0, hi.size).astype(np.float32)
    rows.append(("big_tie_positive", r))
    r = np.full(V, -3.0, np.float32)
    hi = rng.choice(V, min(50, V), replace=False)
    r[hi] = rng.uniform(-1.0, 0.0, hi.size).astype(np.float32)
    r[rng.random(V) < 0.2] = -np.inf
    rows.append(("big_tie_negative", r))
    return rows


@pytest.mark.parametrize("V", [300, 5000, 129280])
def test_value_table_rows(V):
    rng = np.random.default_rng(V + 77)
    rows = _table_rows(V, rng)
    names = [n for n, _ in rows]
    raw = _bits_bf16(np.stack([r for _, r in rows]).astype(np.float32))
    d = to_dev(raw, BF16)
    n5 = (len(rows) // 5) * 5
    t = to_dev(np.tile(raw[:6], ((n5 // 5), 1)), BF16)  # target rows for the fused step (5 per 6)
    for k in [0, 1, 5, min(300, V), min(1024, V)]:
        topk = np.full(len(rows), k, np.int32)
        q = host(B.q_alloc(d, topk=topk, k_max=1024))
        pr = host(B.propose(d))
        for j, name in enumerate(names):
            ref = O.draft_row(raw[j], BF16, k)
            h = {"status": q["status"], "argmax": pr["argmax"] * (q["status"] == 0),
                 "conf": pr["conf"] * (q["status"] == 0), "q": q}
            check_draft_row(h, j, ref, k, label=f"table V{V} k{k} {name}")
        # the fused step (confidence taken from the value table on q rows)
        draws = rng.integers(0, 1 << 24, n5, dtype=np.uint32)
        f = host(B.fused(d[:n5], t, B.SAMPLED, topk=topk[:n5], k_max=1024, draws=u32_dev(draws)))
        for j in range(n5):
            ref = O.draft_row(raw[j], BF16, k, int(draws[j]))
            check_draft_row(f, j, ref, k, label=f"table fused V{V} k{k} {names[j]}")


@pytest.mark.parametrize("R", [120, 210])  # 600 draft rows (3 shards per row), 1,050 (one shard per row)
def test_split_many_rows_equal_one_workgroup_rows(R):
    """Batches past a round of the chip still take the split pipeline (one
    shard per row from 1,024 draft rows on; the target rows' heads with it):
    every output equals the one-workgroup path's (the confidence within the
    tolerance), and sampled rows, the edge rows among them, equal the
    oracle's."""
    V = 3000
    rng = np.random.default_rng(R)
    dr = (rng.standard_normal((5 * R, V)) * 3).astype(np.float32)
    dr[7, 11] = np.nan
    dr[300, :V // 2] = -np.inf
    dr[401] = -2.5
    dr[5 * R - 1, [0, V - 1]] = dr[5 * R - 1].max() + 2
    tg = (rng.standard_normal((6 * R, V)) * 3).astype(np.float32)
    tg[5, 7] = np.inf
    tg[6 * R - 1, [1, V - 2]] = tg[6 * R - 1].max() + 2
    topk = np.zeros(5 * R, np.int32)
    draws = rng.integers(0, 1 << 24, 5 * R, dtype=np.uint32)
    d, t = to_dev(dr, F32), to_dev(tg, F32)
    a = host(B.fused(d, t, B.SAMPLED, topk=topk, draws=u32_dev(draws), split=True))
    b = host(B.fused(d, t, B.SAMPLED, topk=topk, draws=u32_dev(draws), split=False))
    torch.cuda.synchronize()
    for k in ("argmax", "status", "sample", "target_argmax", "target_status", "accept_len", "bonus", "req_status"):
        assert np.array_equal(a[k], b[k]), k
    assert np.array_equal(a["q"]["dense"], b["q"]["dense"])
    assert np.allclose(a["conf"], b["conf"], rtol=1e-6, atol=0)
    assert a["target_argmax"][6 * R - 1] == 1 and a["target_status"][5] != 0
    for j in sorted({0, 7, 300, 401, 5 * R - 1, *rng.integers(0, 5 * R, 6).tolist()}):
        ref = O.draft_row(dr[j], F32, 0, int(draws[j]))
        check_draft_row(a, j, ref, 0, "split, many rows")


@pytest.mark.parametrize("cfg", [1, 3])
def test_split_all_dense_rows_verify_in_the_last_row(cfg):
    """Every draft row dense and few rows: the split pipeline takes all rows,
    and the last finishing row of each request verifies it.  Requests with
    planted agreement (accept lengths 0..5), a refused draft row and an
    invalid target row; all outputs equal the one-workgroup path and the
    oracle's requests."""
    R, V = 6, 40000
    w = W.make(cfg, V=V, R=R)
    sampled = w.mode == "sampled"
    for r in range(R):  # target i agrees with draft token i for i < r (r = 5: all five)
        for i in range(min(r, 5)):
            ref = O.draft_row(w.draft[r * 5 + i], w.dtype, 0, int(w.draws[r * 5 + i]))
            tok = ref["sample"] if sampled else ref["argmax"]
            w.target[r * 6 + i, tok] = np.float32(w.target[r * 6 + i].max() + 30.0)
    w.draft[1 * 5 + 3, 17] = np.nan      # request 1: a refused draft row
    w.target[2 * 6 + 4, 99] = np.inf     # request 2: an invalid target row
    d, t = to_dev(w.draft, w.dtype), to_dev(w.target, w.dtype)
    mode = B.SAMPLED if sampled else B.GREEDY
    draws = u32_dev(w.draws)
    a = host(B.fused(d, t, mode, topk=np.zeros(5 * R, np.int32), draws=draws, split=True))
    b = host(B.fused(d, t, mode, topk=np.zeros(5 * R, np.int32), draws=draws, split=False))
    torch.cuda.synchronize()
    for k in ("argmax", "status", "sample", "target_argmax", "target_status", "accept_len", "bonus", "req_status"):
        assert np.array_equal(a[k], b[k]), k
    assert np.array_equal(a["q"]["dense"], b["q"]["dense"])
    check_workload(w, a, label="split, folded verification")
    assert a["accept_len"].tolist() == [0, 1, 0, 3, 4, 5]
