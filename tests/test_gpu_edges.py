"""GPU edge cases through the C ABI: empty batches on every entry point, and
whole requests at vocabularies on both sides of the register-resident limit
(131,072 bf16 values per row) and at the largest vocabulary accepted, each
compared with the CPU oracle row by row."""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

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
