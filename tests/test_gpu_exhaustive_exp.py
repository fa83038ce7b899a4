"""The library's weight function RN32(exp(d)) against the oracle for every
binary32 d in [-104, 0] (1,120,927,745 values, in eight slices)."""
import numpy as np
import pytest
import torch

from oracle import dyadic24 as O
from vocab_wide_draft_amd import binding as B

pytestmark = pytest.mark.gpu

LO = np.float32(-104.0).view(np.uint32)  # bit patterns 0x80000000 (-0.0) .. LO
NEG_ZERO = np.uint32(0x80000000)
CHUNK = 1 << 25


@pytest.mark.parametrize("part", range(8))
def test_weight_function_exhaustive(part):
    total = int(LO) - int(NEG_ZERO) + 1
    per = (total + 7) // 8
    start = int(NEG_ZERO) + part * per
    stop = min(int(NEG_ZERO) + (part + 1) * per, int(LO) + 1)
    bad = 0
    for a in range(start, stop, CHUNK):
        bits = np.arange(a, min(a + CHUNK, stop), dtype=np.uint32)
        d = bits.view(np.float32)
        got = B.cr_expf(torch.from_numpy(d).to("cuda:0")).cpu().numpy().view(np.uint32)
        ref = O.cr_exp_f32(d).view(np.uint32)
        bad += int(np.count_nonzero(got != ref))
        assert bad == 0, (part, a, d[got != ref][:5])
