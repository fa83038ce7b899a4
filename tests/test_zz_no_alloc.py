"""The allocation-free sharded propose (dspark_sharded_propose_noalloc, for
callers that cannot allocate device memory) against the workspace entry
point dspark_sharded_propose, through the C ABI: bit-identical outputs on
two calls in a row (the second smaller, so that it runs on the scratch the
first one left behind), and the size limit refused on the host."""
import ctypes

import numpy as np
import pytest
import torch

from vocab_wide_draft_amd import binding as B
from vocab_wide_draft_amd import workloads as W

from gpu_helpers import dev, to_dev

pytestmark = pytest.mark.gpu


def _rows(n, V, rng, dtype):
    x = (rng.standard_normal((n, V)) * 2).astype(np.float32)
    x[1, V // 3] = np.nan
    x[2, :] = -np.inf
    x[3, :] = -np.inf
    x[3, V - 1] = 4.0
    x[4, V // 2] = x[4].max() + 1
    x[4, 0] = x[4, V // 2]
    return W.f32_to_bf16_bits(x) if dtype == "bf16" else x


def _same(a, b):
    for k in ("argmax", "status", "s64", "conf"):
        ha, hb = a[k].cpu().numpy(), b[k].cpu().numpy()
        assert np.array_equal(ha.view(np.uint8), hb.view(np.uint8)), k


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_entry_two_calls(dtype):
    rng = np.random.default_rng(101)
    big = to_dev(_rows(96, 129280, rng, dtype), dtype)
    small = to_dev(_rows(7, 3001, rng, dtype), dtype)
    a1 = B.sharded_propose_noalloc(big, 8)
    torch.cuda.synchronize()
    b1 = B.sharded_propose(big, 8)
    torch.cuda.synchronize()
    _same(a1, b1)
    assert int((a1["status"] == 0).sum()) == 94
    a2 = B.sharded_propose_noalloc(small, 3)
    torch.cuda.synchronize()
    b2 = B.sharded_propose(small, 3)
    torch.cuda.synchronize()
    _same(a2, b2)


def test_noalloc_refuses_calls_beyond_its_scratch():
    lib = B.load_library()
    x = torch.zeros((1366, 64), dtype=torch.bfloat16, device=dev())
    r = B._rows(x)
    out = torch.zeros(1366, dtype=torch.int32, device=dev())
    rc = lib.dspark_sharded_propose_noalloc(ctypes.byref(r), 64, B._p(out), None, None, B._p(out), B._stream())
    assert rc == -3 and "exceeds" in lib.dspark_last_error().decode()
    ok = B.sharded_propose_noalloc(x[:1365], 64)  # 87,360 row-shards: inside the limit
    torch.cuda.synchronize()
    assert (ok["status"] == 0).all() and (ok["s64"] == 64.0).all()
