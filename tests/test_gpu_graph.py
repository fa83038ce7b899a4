"""The fused step captured into a HIP graph and replayed: every replay, with
eager work and synchronisations between replays, equals the eager step bit
for bit (the library records no memsets and no allocations inside the step,
so a captured step is the same kernels on the same buffers)."""
import numpy as np
import pytest
import torch

from vocab_wide_draft_amd import binding as B
from vocab_wide_draft_amd import workloads as W

from gpu_helpers import dev

pytestmark = pytest.mark.gpu


def _tensors(o, pre=""):
    for k, v in o.items():
        if isinstance(v, torch.Tensor):
            yield pre + k, v
        elif isinstance(v, dict):
            yield from _tensors(v, pre + k + ".")


INPUTS = ("draws", "q.topk")  # tensors the output dict holds as inputs of the step


def _fill(out):
    """Every output byte set to 0xF9, so that a replay has to rewrite it."""
    for k, v in _tensors(out):
        if k not in INPUTS:
            v.view(torch.uint8).fill_(0xF9)


@pytest.mark.parametrize("cfg,V,R", [(1, 129280, 1),      # dense float32 rows split over vocabulary shards
                                     (3, 20000, 26),      # 130 streamed dense rows, one workgroup each
                                     (5, 3000, 8),        # register-resident bf16 rows, mixed dense / sparse
                                     (4, 129280, 2)])     # sparse top-k rows, sampled
def test_graph_replay_equals_eager(cfg, V, R):
    w = W.make(cfg, V=V, R=R)

    def up(a):
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev())
        return torch.from_numpy(a).to(dev())

    d, t = up(w.draft), up(w.target)
    draws = None if w.draws is None else torch.from_numpy(w.draws.view(np.int32)).to(dev())
    mode = B.SAMPLED if w.mode == "sampled" else B.GREEDY
    with_q = w.topk is not None
    out = B.fused(d, t, mode, topk=w.topk, k_max=1024 if with_q else 0, draws=draws, with_q=with_q)
    _fill(out)
    B.fused(d, t, mode, draws=draws, out=out)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in _tensors(out)}
    assert int((ref["status"] == 0).sum()) > 0.8 * ref["status"].numel()  # the step ran on valid rows

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.fused(d, t, mode, draws=draws, out=out)
    other = B.fused(d, t, mode, topk=w.topk, k_max=1024 if with_q else 0, draws=draws, with_q=with_q)
    for rep in range(3):
        _fill(out)
        torch.cuda.synchronize()
        graph.replay()
        B.fused(d, t, mode, draws=draws, out=other)  # eager work on other buffers between replays
        torch.cuda.synchronize()
        now = dict(_tensors(out))
        for k, v in ref.items():
            assert torch.equal(now[k], v), (cfg, rep, k)
        bad = [k for k, v in _tensors(other) if k in ref and k not in INPUTS and not k.startswith("q.")
               and not torch.equal(v, ref[k])]
        assert not bad, (cfg, rep, "eager", bad, {k: (dict(_tensors(other))[k][:8].tolist(), ref[k][:8].tolist())
                                                  for k in bad})
