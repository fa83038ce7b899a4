"""GPU parity of stochastic verification ("DeepSeek-V4.1 DSpark", "State and
sampling contracts") through the C ABI against the oracle: every target
row's exact inverse-CDF draw from the full p at T = 1 with its 64-bit draw,
and each request's accept length and bonus, bit for bit.  Rows cover the
value-table path, the per-element path (maxima near zero), tiny weights,
one-hot and refused rows, the register-resident and the streamed sources,
and draws at the ends of the range and exactly at a token boundary."""
import numpy as np
import pytest
import torch

from oracle import dyadic24 as O
from vocab_wide_draft_amd import binding as B
from vocab_wide_draft_amd import workloads as W

from gpu_helpers import dev, to_dev

pytestmark = pytest.mark.gpu


def _boundary_draw(raw, dtype, v):
    """The smallest 64-bit draw whose token is v (> 0): ceil(C_(v-1) 2^64 / A)."""
    st, a, A = O.weight_ints(raw, dtype)
    c = sum(a[:v])
    return -((-c << 64) // A)


def _case(V, R, dtype, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((6 * R, V)) * 1.5).astype(np.float32)
    x[6 * 0 + 1] = (rng.standard_normal(V) * 3e-4).astype(np.float32)   # maximum near 0: per-element path
    x[6 * 0 + 2] = (-rng.gumbel(size=V) * 12.0).astype(np.float32)       # weights down to subnormals
    x[6 * 0 + 3] -= 40.0                                                 # negative maximum
    if R > 1:
        x[6 * 1 + 2, V // 2] = np.nan                                    # request 1: a refused target row
    if R > 2:
        x[6 * 2 + 4] = -np.inf
        x[6 * 2 + 4, V - 1] = 3.0                                        # request 2: a one-hot target row
    raw = W.f32_to_bf16_bits(x) if dtype == "bf16" else x
    draws = rng.integers(0, 2**63, (R, 6), dtype=np.uint64) * np.uint64(2) + rng.integers(0, 2, (R, 6), dtype=np.uint64)
    draws[0, 0] = 0
    draws[0, 5] = np.uint64(2**64 - 1)
    if V >= 8:  # draws exactly at a token boundary, and one below the next
        draws[R - 1, 0] = np.uint64(_boundary_draw(raw[6 * (R - 1)], dtype, V // 3))
        draws[R - 1, 1] = np.uint64(_boundary_draw(raw[6 * (R - 1) + 1], dtype, V // 2) - 1)
    tt = [[O.target_draw_row(raw[6 * r + i], dtype, int(draws[r, i])) for i in range(6)] for r in range(R)]
    if V >= 8:
        assert tt[R - 1][0][1] == V // 3 and tt[R - 1][1][1] == V // 2 - 1
    dtok = np.zeros((R, 5), np.int32)
    dst = np.zeros((R, 5), np.int32)
    for r in range(R):
        L = r % 6                                                        # planted prefix
        for i in range(5):
            t = tt[r][i][1]
            dtok[r, i] = t if i < L else (t + 1 + int(rng.integers(0, V - 1))) % V if V > 1 else 0
    dst[R - 1, 2] = O.ST_ROW_NAN                                         # an invalid draft row stops acceptance
    return raw, draws, dtok, dst


def _check(raw, draws, dtok, dst, dtype, out, R):
    ts = out["target_sample"].cpu().numpy()
    tst = out["target_status"].cpu().numpy()
    acc, bon, rst = (out[k].cpu().numpy() for k in ("accept_len", "bonus", "req_status"))
    for r in range(R):
        st, a, b, toks, sts = O.verify_stochastic(list(dtok[r]), list(dst[r]), raw[6 * r:6 * r + 6], dtype,
                                                  [int(u) for u in draws[r]])
        assert list(tst[6 * r:6 * r + 6]) == sts, r
        assert list(ts[6 * r:6 * r + 6]) == toks, r
        assert (int(rst[r]), int(acc[r]), int(bon[r])) == (st, a, b), r


def _run(raw, draws, dtok, dst, dtype):
    out = B.verify_stochastic(to_dev(raw, dtype), torch.from_numpy(dtok).to(dev()), draws,
                              draft_status=torch.from_numpy(dst).to(dev()))
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dtype,V", [("f32", 3001), ("bf16", 3001), ("bf16", 257), ("bf16", 8), ("f32", 1)])
def test_stochastic_small(dtype, V):
    R = 8
    raw, draws, dtok, dst = _case(V, R, dtype, V + (1 if dtype == "bf16" else 2))
    out = _run(raw, draws, dtok, dst, dtype)
    _check(raw, draws, dtok, dst, dtype, out, R)
    if V > 100:
        assert set(int(a) for a in out["accept_len"].cpu().numpy()) >= {0, 2, 4, 5}


@pytest.mark.parametrize("dtype,V", [("bf16", 129280), ("f32", 129280), ("bf16", 140001)])
def test_stochastic_full_vocabulary(dtype, V):
    """bf16 rows held in registers (V = 129280), float32 and long bf16 rows
    streamed."""
    R = 3
    raw, draws, dtok, dst = _case(V, R, dtype, 123 + V % 7)
    out = _run(raw, draws, dtok, dst, dtype)
    _check(raw, draws, dtok, dst, dtype, out, R)


def test_stochastic_empty_and_argument_errors():
    t = torch.empty((0, 64), dtype=torch.bfloat16, device=dev())
    out = B.verify_stochastic(t, torch.empty((0, 5), dtype=torch.int32, device=dev()),
                              np.zeros((0, 6), np.uint64))
    assert out["accept_len"].numel() == 0
    with pytest.raises(B.DsparkError):
        B.verify_stochastic(torch.zeros((7, 64), dtype=torch.bfloat16, device=dev()),
                            torch.zeros((1, 5), dtype=torch.int32, device=dev()), np.zeros((1, 6), np.uint64))
