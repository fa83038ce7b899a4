"""The adjacent rows at full size, in the launch configurations the bench
times (the R = 1024 mixed workload: 5,120 draft rows, 6,144 target rows,
V = 129,280): the wire check of the workload's q, the margins, stochastic
verification and the two-shard propose.  Properties are checked on every row
and the oracle recomputes sampled rows one by one."""
import numpy as np
import pytest
import torch

from oracle import dyadic24 as O
from oracle import q_wire as Q
from vocab_wide_draft_amd import binding as B
from vocab_wide_draft_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def step():
    w = W.make(5)
    d = torch.from_numpy(w.draft.view(np.int16)).view(torch.bfloat16).to(DEV)
    t = torch.from_numpy(w.target.view(np.int16)).view(torch.bfloat16).to(DEV)
    draws = torch.from_numpy(w.draws.view(np.int32)).to(DEV)
    out = B.fused(d, t, B.SAMPLED, topk=w.topk, k_max=1024, draws=draws)
    torch.cuda.synchronize()
    return w, d, t, out


def test_wire_check_bench_launch(step):
    w, d, t, out = step
    q = out["q"]
    topk = torch.from_numpy(w.topk.astype(np.int32)).to(DEV)
    dense_w, sp_w = B.q_encode(q["dense"]), B.q_encode(q["sp_cnt"])
    chk = B.q_validate(w.V, topk=topk, k_max=1024, dense=dense_w, sp_ids=q["sp_ids"], sp_val=sp_w,
                       sp_len=q["sp_len"], tokens=out["sample"], want_counts=True)
    st = chk["status"].cpu().numpy()
    ok = out["status"].cpu().numpy() == 0
    assert (st[ok] == 0).all()                                  # every row the library allocated passes
    dm = torch.from_numpy((w.topk == 0) & ok).to(DEV)
    assert torch.equal(chk["dense_counts"][dm], q["dense"][dm])
    rng = np.random.default_rng(1)
    hd, hs, hsl, hsid = dense_w.cpu().numpy(), sp_w.cpu().numpy(), q["sp_len"].cpu().numpy(), q["sp_ids"].cpu().numpy()
    tok = out["sample"].cpu().numpy()
    dense_rows = np.flatnonzero(w.topk == 0)
    sparse_rows = np.flatnonzero(w.topk != 0)
    for j in rng.choice(dense_rows, 2, replace=False):
        assert Q.check_dense(hd[j], w.V, token=int(tok[j]))[0] == st[j]
    for j in rng.choice(sparse_rows, 3, replace=False):
        ws, wc = Q.check_sparse(hsid[j], hs[j], int(hsl[j]), int(w.topk[j]), 1024, w.V, token=int(tok[j]))
        assert ws == st[j]
        assert np.array_equal(chk["sp_counts"][j].cpu().numpy().view(np.uint32), wc)


def test_margin_bench_launch(step):
    w, d, t, out = step
    m = B.margin(d).cpu().numpy()
    ok = out["status"].cpu().numpy() == 0
    assert np.isfinite(m).all() and (m >= 0).all() and (m[~ok] == 0).all()
    rng = np.random.default_rng(2)
    for j in rng.choice(w.R * 5, 4, replace=False):
        want = Q.margin(O.to_f32(w.draft[j], "bf16"))
        assert m[j].view(np.uint32) == want.view(np.uint32), j


def test_stochastic_bench_launch(step):
    w, d, t, out = step
    dtok = out["sample"].view(w.R, 5)
    dst = out["status"].view(w.R, 5)
    rng = np.random.default_rng(0xD5A1F00D)
    tdr = rng.integers(0, 2**63, (w.R, 6), dtype=np.uint64) * np.uint64(2)
    res = B.verify_stochastic(t, dtok, tdr, draft_status=dst)
    acc = res["accept_len"].cpu().numpy()
    assert ((acc >= 0) & (acc <= 5)).all()
    ht, hs = dtok.cpu().numpy(), dst.cpu().numpy()
    for r in rng.choice(w.R, 3, replace=False):
        st, a, b, toks, sts = O.verify_stochastic(list(ht[r]), list(hs[r]), w.target[6 * r:6 * r + 6], "bf16",
                                                  [int(u) for u in tdr[r]])
        assert (int(res["req_status"][r]), int(res["accept_len"][r]), int(res["bonus"][r])) == (st, a, b)
        assert res["target_sample"][6 * r:6 * r + 6].cpu().tolist() == toks


def test_ratio_bench_launch(step):
    """Probability-ratio verification in the bench's launch configuration
    (the R = 1024 mixed workload's sampled drafts and q): valid ranges for
    every request, sampled requests against the oracle."""
    from oracle import ratio as RT
    w, d, t, out = step
    dtok = out["sample"].view(w.R, 5)
    dst = out["status"].view(w.R, 5)
    qd = out["q"]
    rng = np.random.default_rng(0xD5A1F00E)
    ad = rng.integers(0, 2**63, (w.R, 5), dtype=np.uint64) * np.uint64(2)
    fd = rng.integers(0, 2**63, w.R, dtype=np.uint64) * np.uint64(2) + np.uint64(1)
    res = B.verify_ratio(t, dtok, qd, ad, fd, draft_status=dst)
    acc, tok, rst = (res[k].cpu().numpy() for k in ("accept_len", "token", "req_status"))
    assert ((acc >= 0) & (acc <= 5)).all() and ((tok >= 0) & (tok < w.V)).all()
    assert (rst == 0).all()
    ht, hs = dtok.cpu().numpy(), dst.cpu().numpy()
    topk = np.asarray(w.topk)
    hq = {k: (v.cpu().numpy() if hasattr(v, "cpu") else v) for k, v in qd.items()}
    for r in rng.choice(w.R, 3, replace=False):
        qs = []
        for i in range(5):
            j = 5 * r + i
            if topk[j] == 0:
                qs.append((np.arange(w.V), hq["dense"][j].view(np.uint32)))
            else:
                n = int(hq["sp_len"][j])
                qs.append((hq["sp_ids"][j, :n], hq["sp_cnt"][j, :n].view(np.uint32)))
        want = RT.verify_ratio(list(ht[r]), list(hs[r]), qs, w.target[6 * r:6 * r + 6], "bf16",
                               [int(u) for u in ad[r]], int(fd[r]))
        assert (int(rst[r]), int(acc[r]), int(tok[r])) == want[:3], (r, want)


def test_sharded_bench_launch(step):
    w, d, t, out = step
    s = B.sharded_propose(d, 2)
    am = s["argmax"].cpu().numpy()
    assert np.array_equal(am, out["argmax"].cpu().numpy())      # the same argmax as the fused step, every row
    assert np.array_equal(s["status"].cpu().numpy() == 0, out["status"].cpu().numpy() == 0)
    rng = np.random.default_rng(3)
    s64 = s["s64"].cpu().numpy()
    for j in rng.choice(w.R * 5, 3, replace=False):
        st, a, want = O.propose_sum(w.draft[j], "bf16")
        assert (st, a) == (int(s["status"][j]), int(am[j])) and s64[j] == want, j
