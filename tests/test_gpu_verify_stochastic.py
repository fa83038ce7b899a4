"""GPU parity of stochastic verification ("DeepSeek-V4.1 DSpark", "State and
sampling contracts") through the C ABI against the oracle: every target row's
dense dyadic24 q, its own draw, and the accept length and bonus of each
request, bit for bit.  Draft tokens are planted from the oracle's target
draws so that every accept length occurs."""
import numpy as np
import pytest
import torch

from oracle import dyadic24 as O
from vocab_wide_draft_amd import binding as B
from vocab_wide_draft_amd import workloads as W

from gpu_helpers import dev, to_dev

pytestmark = pytest.mark.gpu
M = 1 << 24


def _case(V, R, dtype, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((6 * R, V)) * 1.5).astype(np.float32)
    x[6 * 1 + 2, V // 2] = np.nan                         # request 1: a refused target row
    x[6 * 2 + 4] = -np.inf
    x[6 * 2 + 4, V - 1] = 3.0                             # request 2: a one-hot target row
    raw = W.f32_to_bf16_bits(x) if dtype == "bf16" else x
    draws = rng.integers(0, M, (R, 6)).astype(np.uint32)
    draws[3 % R, 1] = M + 5                               # a draw out of range
    tt = [[O.target_sample_row(raw[6 * r + i], dtype, int(draws[r, i])) for i in range(6)] for r in range(R)]
    dtok = np.zeros((R, 5), np.int32)
    dst = np.zeros((R, 5), np.int32)
    for r in range(R):
        L = r % 6                                         # planted prefix
        for i in range(5):
            t = tt[r][i][1]
            dtok[r, i] = t if i < L else (t + 1 + int(rng.integers(0, V - 1))) % V if V > 1 else 0
    dst[R - 1, 2] = O.ST_ROW_NAN                          # an invalid draft row stops acceptance
    return raw, draws, dtok, dst


def _check(raw, draws, dtok, dst, dtype, out, V, R, q_rows):
    ts = out["target_sample"].cpu().numpy()
    tst = out["target_status"].cpu().numpy()
    acc, bon, rst = (out[k].cpu().numpy() for k in ("accept_len", "bonus", "req_status"))
    tq = out["target_q"].cpu().numpy().view(np.uint32)
    for r in range(R):
        st, a, b, toks, sts = O.verify_stochastic(list(dtok[r]), list(dst[r]), raw[6 * r:6 * r + 6], dtype,
                                                  [int(u) for u in draws[r]])
        assert list(tst[6 * r:6 * r + 6]) == sts, r
        want_t = [t if s == O.ST_OK else 0 for t, s in zip(toks, sts)]
        assert list(ts[6 * r:6 * r + 6]) == want_t, r
        assert (int(rst[r]), int(acc[r]), int(bon[r])) == (st, a, b), r
        for i in range(6):
            j = 6 * r + i
            if j in q_rows and sts[i] == O.ST_OK:
                _, _, c = O.q_row(O.to_f32(raw[j], dtype), 0)
                assert np.array_equal(tq[j], c.astype(np.uint32)), j


@pytest.mark.parametrize("dtype,V", [("f32", 3001), ("bf16", 3001), ("bf16", 257)])
def test_stochastic_small(dtype, V):
    R = 8
    raw, draws, dtok, dst = _case(V, R, dtype, V + (1 if dtype == "bf16" else 2))
    out = B.verify_stochastic(to_dev(raw, dtype), torch.from_numpy(dtok).to(dev()),
                              torch.from_numpy(draws.view(np.int32)).to(dev()),
                              draft_status=torch.from_numpy(dst).to(dev()))
    torch.cuda.synchronize()
    _check(raw, draws, dtok, dst, dtype, out, V, R, q_rows=set(range(6 * R)))
    acc = out["accept_len"].cpu().numpy()
    assert set(int(a) for a in acc) >= {0, 2, 4, 5}


def test_stochastic_full_vocabulary():
    V, R = 129280, 4
    raw, draws, dtok, dst = _case(V, R, "bf16", 123)
    out = B.verify_stochastic(to_dev(raw, "bf16"), torch.from_numpy(dtok).to(dev()),
                              torch.from_numpy(draws.view(np.int32)).to(dev()),
                              draft_status=torch.from_numpy(dst).to(dev()))
    torch.cuda.synchronize()
    _check(raw, draws, dtok, dst, "bf16", out, V, R, q_rows={0, 5, 13})


@pytest.mark.parametrize("V", [3001, 129280])
def test_stochastic_without_counts(V):
    """With no count storage the draws, accept lengths and bonuses are the
    same as with it (and as the oracle's)."""
    R = 6
    raw, draws, dtok, dst = _case(V, R, "bf16", V + 7)
    args = (to_dev(raw, "bf16"), torch.from_numpy(dtok).to(dev()), torch.from_numpy(draws.view(np.int32)).to(dev()))
    a = B.verify_stochastic(*args, draft_status=torch.from_numpy(dst).to(dev()))
    b = B.verify_stochastic(*args, draft_status=torch.from_numpy(dst).to(dev()), store_q=False)
    torch.cuda.synchronize()
    assert b["target_q"] is None
    for k in ("target_sample", "target_status", "accept_len", "bonus", "req_status"):
        assert torch.equal(a[k], b[k]), k
    if V < 10000:
        _check(raw, draws, dtok, dst, "bf16", {**b, "target_q": a["target_q"]}, V, R, q_rows=set())


def test_stochastic_without_counts_needs_resident_rows():
    x = np.zeros((6, 64), np.float32)
    with pytest.raises(B.DsparkError):
        B.verify_stochastic(to_dev(x, "f32"), torch.zeros((1, 5), dtype=torch.int32, device=dev()),
                            torch.zeros((1, 6), dtype=torch.int32, device=dev()), store_q=False)
