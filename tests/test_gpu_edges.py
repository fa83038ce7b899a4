"""GPU edge cases through the C ABI: empty batches on every entry point, and
whole requests at vocabularies on both sides of the register-resident limit
(131,072 bf16 values per row) and at the largest vocabulary accepted, each
compared with the CPU oracle row by row."""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

from oracle import dyadic24 as O
from vocab_wide_draft_amd import binding as B
from vocab_wide_draft_amd import workloads as W

from gpu_helpers import check_workload, dev, host, to_dev, u32_dev

pytestmark = pytest.mark.gpu

V_RESIDENT = 131072  # 16 vectors x 1024 threads x 8 bf16 values
V_MAX = 1 << 20


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_empty_batches(dtype):
    """Zero rows or zero requests: every entry point succeeds and launches
    nothing (the outputs are empty)."""
    V = 1000
    d = torch.empty((0, V), dtype=dtype, device=dev())
    t = torch.empty((0, V), dtype=dtype, device=dev())
    no_k = np.zeros(0, np.int32)
    pr = B.propose(d)
    q = B.q_alloc(d, topk=no_k, k_max=8)
    qd = B.q_alloc(d)
    tok = B.sample(q, torch.zeros((0, 1), dtype=torch.int32, device=dev()), q["status"], V)
    vf = B.verify_greedy(t, torch.zeros((0, 5), dtype=torch.int32, device=dev()))
    f = B.fused(d, t, B.SAMPLED, topk=no_k, k_max=8, draws=u32_dev(np.zeros(0, np.uint32)))
    g = B.fused(d, t, B.GREEDY, with_q=False)
    torch.cuda.synchronize()
    assert pr["argmax"].numel() == 0 and q["status"].numel() == 0 and qd["dense"].numel() == 0
    assert tok.numel() == 0 and vf["accept_len"].numel() == 0
    assert f["accept_len"].numel() == 0 and g["bonus"].numel() == 0


def _request(V, dtype, seed):
    """One request (5 draft rows, 6 target rows) with a dense, two sparse, a
    duplicated-value and a one-hot draft row."""
    rng = np.random.default_rng(seed)
    d = (rng.standard_normal((5, V)) * 2).astype(np.float32)
    t = (rng.standard_normal((6, V)) * 2).astype(np.float32)
    vals = np.array([-1.5, 0.25, 2.0, 2.5], np.float32)
    d[1] = vals[rng.integers(0, vals.size, V)]           # long runs of equal values
    d[3] = -np.inf
    d[3, V - 1] = 1.75                                    # one-hot at the last id
    t[2] = d[0]                                           # a target row equal to a draft row
    if dtype == "bf16":
        d, t = W.f32_to_bf16_bits(d), W.f32_to_bf16_bits(t)
    topk = np.array([0, 1024, 32, 256, 0], np.int32)
    draws = rng.integers(0, 1 << 24, size=5, dtype=np.uint32)
    return SimpleNamespace(R=1, V=V, dtype=dtype, mode="sampled", draft=d, target=t, topk=topk, draws=draws)


@pytest.mark.parametrize("dtype,V", [("bf16", V_RESIDENT), ("bf16", V_RESIDENT + 8), ("bf16", V_MAX),
                                     ("f32", V_RESIDENT + 8), ("f32", V_MAX)])
def test_vocabulary_limits(dtype, V):
    w = _request(V, dtype, seed=V + (1 if dtype == "bf16" else 2))
    dd, td = to_dev(w.draft, dtype), to_dev(w.target, dtype)
    out = B.fused(dd, td, B.SAMPLED, topk=w.topk, k_max=1024, draws=u32_dev(w.draws))
    torch.cuda.synchronize()
    check_workload(w, host(out), label=f"{dtype} V{V}")


def _special_target_rows(V, rng):
    """Target rows (binary32 values) for every status and every kind of
    maximum: NaN, +inf, all -inf, -0 before +0, all negative, constant,
    one-hot at the last id, ordinary."""
    base = (rng.standard_normal(V) * 2).astype(np.float32)
    rows = []
    r = base.copy(); r[V // 3] = np.nan; rows.append(r)
    r = base.copy(); r[V - 1] = np.inf; rows.append(r)
    rows.append(np.full(V, -np.inf, np.float32))
    r = np.full(V, -1.0, np.float32); r[1 % V] = -0.0; r[V // 2] = 0.0; rows.append(r)
    rows.append(-np.abs(base) - 0.5)
    rows.append(np.full(V, 3.0, np.float32))
    r = np.full(V, -np.inf, np.float32); r[V - 1] = -7.25; rows.append(r)
    rows.append(base)
    r = base.copy(); r[::7] = -np.inf; rows.append(r)
    r = np.zeros(V, np.float32); r[::2] = -0.0; rows.append(r)
    r = base.copy(); r[5 % V] = r.max(); r[V - 2] = r.max(); rows.append(r)
    rows.append((base - 200.0).astype(np.float32))
    return np.stack(rows)


@pytest.mark.parametrize("V", [129280, 129283, 5001, 64])
def test_target_rows_every_maximum(V):
    """Target argmax and status for rows of every kind of maximum, through
    the verify entry point and the fused step (bf16 and fp32)."""
    rng = np.random.default_rng(V + 11)
    x = _special_target_rows(V, rng)
    R = x.shape[0] // 6
    for dtype in ("bf16", "f32"):
        raw = W.f32_to_bf16_bits(x) if dtype == "bf16" else x
        t = to_dev(raw, dtype)
        dtok = torch.from_numpy(rng.integers(0, V, size=(R, 5), dtype=np.int32)).to(dev())
        out = host(B.verify_greedy(t, dtok))
        for j in range(x.shape[0]):
            f = O.to_f32(raw[j], dtype)
            st = O.row_status(f)
            assert int(out["target_status"][j]) == st, (dtype, V, j)
            want = O.argmax_first(f)[1] if st == O.ST_OK else 0
            assert int(out["target_argmax"][j]) == want, (dtype, V, j)
        # the fused step with ordinary draft rows
        d = (rng.standard_normal((5 * R, V)) * 2).astype(np.float32)
        draw = W.f32_to_bf16_bits(d) if dtype == "bf16" else d
        w = SimpleNamespace(R=R, V=V, dtype=dtype, mode="greedy", draft=draw, target=raw, topk=None, draws=None)
        f = host(B.fused(to_dev(draw, dtype), t, B.GREEDY, with_q=False))
        check_workload(w, f, label=f"targets {dtype} V{V}")
