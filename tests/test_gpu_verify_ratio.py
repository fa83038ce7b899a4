"""GPU parity of probability-ratio verification with the dyadic q and
full-vocabulary residual sampling ("PP1 q transport and scheduling design",
"Distribution contract and precision", last paragraph) through the C ABI
against oracle/ratio.py: accept length, correction / bonus token and status
of every request, bit for bit.  Target rows are perturbed copies of the
draft rows so that every accept length occurs; q is dense or sparse (k = 32,
1024); requests cover refused draft and target rows, zero q at the proposed
token, draws at the ends of the range, the value-table and per-element
weight paths, register-resident and streamed rows."""
import numpy as np
import pytest
import torch

from oracle import dyadic24 as O
from oracle import ratio as RT
from vocab_wide_draft_amd import binding as B
from vocab_wide_draft_amd import workloads as W

from gpu_helpers import dev, to_dev

pytestmark = pytest.mark.gpu
M = 1 << 24


def _u64(rng, shape):
    return rng.integers(0, 2**63, shape, dtype=np.uint64) * np.uint64(2) + rng.integers(0, 2, shape, dtype=np.uint64)


def _case(V, R, dtype, seed, ks):
    rng = np.random.default_rng(seed)
    dr = (rng.standard_normal((5 * R, V)) * 2).astype(np.float32)
    tg = np.repeat(dr.reshape(R, 5, V), [1, 1, 1, 1, 2], axis=1).reshape(6 * R, V).copy()
    # target row i predicts draft position i: a perturbed copy, closer for later requests
    for r in range(R):
        tg[6 * r:6 * r + 6] += (rng.standard_normal((6, V)) * (0.05 + 0.4 * (r % 4))).astype(np.float32)
    dr[5 * 0 + 1] = (rng.standard_normal(V) * 3e-4).astype(np.float32)        # maximum near 0
    tg[6 * 0 + 1] = (rng.standard_normal(V) * 3e-4).astype(np.float32)
    if R > 2:
        dr[5 * 2 + 3, V // 4] = np.nan                                         # a refused draft row
    if R > 3:
        tg[6 * 3 + 0, 7 % V] = np.inf                                          # a refused target row, read first
    if R > 4:
        dr[5 * 4 + 2, V // 5] = -np.inf                                        # q = 0 there: proposed below
    draw_raw = W.f32_to_bf16_bits(dr) if dtype == "bf16" else dr
    tg_raw = W.f32_to_bf16_bits(tg) if dtype == "bf16" else tg
    topk = np.array([ks[(r + i) % len(ks)] for r in range(R) for i in range(5)], np.int32)
    return rng, draw_raw, tg_raw, topk


def _oracle_q(draw_raw, dtype, topk):
    qs, sts = [], []
    for j in range(draw_raw.shape[0]):
        x = O.to_f32(draw_raw[j], dtype)
        st = O.row_status(x)
        if st == O.ST_OK:
            st, ids, c = O.q_row(x, int(topk[j]))
        if st != O.ST_OK:
            ids, c = np.zeros(0, np.int64), np.zeros(0, np.int64)
        qs.append((ids, c))
        sts.append(st)
    return qs, sts


def _run_case(V, R, dtype, seed, ks):
    rng, draw_raw, tg_raw, topk = _case(V, R, dtype, seed, ks)
    d, t = to_dev(draw_raw, dtype), to_dev(tg_raw, dtype)
    qd = B.q_alloc(d, topk=topk, k_max=max(ks) if max(ks) > 0 else 0)
    qs, sts = _oracle_q(draw_raw, dtype, topk)
    gst = qd["status"].cpu().numpy()
    assert list(gst) == sts
    # proposals drawn from q; one request proposes a token outside its q's support
    dtok = np.zeros((R, 5), np.int32)
    for r in range(R):
        for i in range(5):
            j = 5 * r + i
            if sts[j] == O.ST_OK:
                dtok[r, i] = O.sample(*qs[j], int(rng.integers(0, M)))[1]
    if R > 4:
        j = 5 * 4 + 2
        held = {int(v) for v, c in zip(qs[j][0].tolist(), qs[j][1].tolist()) if c > 0}
        dtok[4, 2] = next(v for v in range(V) if v not in held)
    ad, fd = _u64(rng, (R, 5)), _u64(rng, R)
    ad[0, 0], fd[0] = 0, np.uint64(2**64 - 1)
    fd[1 % R] = 0
    dst = torch.from_numpy(gst.reshape(R, 5)).to(dev())
    out = B.verify_ratio(t, torch.from_numpy(dtok).to(dev()), qd, ad, fd, draft_status=dst)
    torch.cuda.synchronize()
    acc, tok, rst = (out[k].cpu().numpy() for k in ("accept_len", "token", "req_status"))
    got = []
    for r in range(R):
        want = RT.verify_ratio(list(dtok[r]), sts[5 * r:5 * r + 5], qs[5 * r:5 * r + 5], tg_raw[6 * r:6 * r + 6],
                               dtype, [int(u) for u in ad[r]], int(fd[r]))
        assert (int(rst[r]), int(acc[r]), int(tok[r])) == want[:3], (r, want)
        got.append(want)
    return got


@pytest.mark.parametrize("dtype,V,ks", [("f32", 3001, (0,)), ("bf16", 3001, (0, 32)), ("bf16", 2999, (1024, 0)),
                                        ("f32", 1500, (32, 0, 1024))])
def test_ratio_small(dtype, V, ks):
    R = 12
    got = _run_case(V, R, dtype, V + len(ks), ks)
    lens = {g[1] for g in got if g[0] == O.ST_OK}
    assert len(lens) >= 3, lens
    assert {g[0] for g in got} >= {O.ST_OK, O.ST_TARGET_INVALID, O.ST_DRAFT_INVALID}


@pytest.mark.parametrize("dtype,ks", [("bf16", (0, 32, 1024)), ("f32", (0,))])
def test_ratio_full_vocabulary(dtype, ks):
    _run_case(129280, 4, dtype, 77, ks)


def test_ratio_every_proposal_accepted_when_q_equals_p():
    """Four equal logits: p is dyadic and q equals it, so every proposal is
    accepted and the bonus is the draw from p of target row 5."""
    V, R = 64, 5
    x = np.full((V,), -np.inf, np.float32)
    x[[3, 17, 40, 63]] = 2.0
    draw_raw = np.stack([x] * (5 * R))
    tg_raw = np.stack([x] * (6 * R))
    d, t = to_dev(draw_raw, "f32"), to_dev(tg_raw, "f32")
    qd = B.q_alloc(d, topk=np.zeros(5 * R, np.int32), k_max=0)
    rng = np.random.default_rng(5)
    dtok = rng.choice([3, 17, 40, 63], (R, 5)).astype(np.int32)
    ad, fd = _u64(rng, (R, 5)), _u64(rng, R)
    ad[:, 0] = np.uint64(2**64 - 1)
    out = B.verify_ratio(t, torch.from_numpy(dtok).to(dev()), qd, ad, fd)
    torch.cuda.synchronize()
    assert (out["accept_len"].cpu().numpy() == 5).all() and (out["req_status"].cpu().numpy() == 0).all()
    for r in range(R):
        assert int(out["token"][r]) == O.target_draw_row(x, "f32", int(fd[r]))[1]
