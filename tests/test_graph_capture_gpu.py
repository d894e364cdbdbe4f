"""HIP graph capture of the allocating entry points.

attn_fwd takes its split-KV partials stream-ordered from the library's
memory pool (hipMallocFromPoolAsync / hipFreeAsync on the caller's stream)
and attn_bwd forks
its dQ kernel onto a second stream of the library's (event record and wait)
except at D = 128.  Both must be capturable by a caller (torch.cuda.graph,
as torch.compile's CUDA-graph mode does): each captured call is replayed
several times, with the outputs cleared and unrelated eager work in
between, and every replay must reproduce the eager call bit for bit.
"""
import numpy as np
import pytest

from memory_efficient_tiled_amd import binding, inputs
from tests.parity import log, to_device

pytestmark = pytest.mark.gpu


def _replays(graph, outs, refs, what):
    import torch
    for r in range(4):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _ = float(refs[0].float().abs().sum())   # eager work between replays
        assert all(torch.equal(o, ref) for o, ref in zip(outs, refs)), f"{what}: replay {r}"
    log(f"  {what}: 4 replays bit-identical to the eager call")


def test_capture_split_forward(gpu_device):
    import torch
    x = inputs.make_inputs(1, 4, 2, 100, 3000, 128, inputs.BF16, seed=1)
    assert binding.attn_fwd_plan(1, 4, 2, 100, 3000, 128, False,
                                 binding.ATTN_BF16).workspace_bytes > 0
    q, k, v = (to_device(a, inputs.BF16, gpu_device) for a in (x.q, x.k, x.v))
    out = torch.empty_like(q)
    lse = torch.empty((1, 4, 100), dtype=torch.float32, device=gpu_device)
    binding.attn_fwd(q, k, v, out=out, lse=lse)
    torch.cuda.synchronize()
    refs = (out.clone(), lse.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        binding.attn_fwd(q, k, v, out=out, lse=lse)
    _replays(g, (out, lse), refs, "attn_fwd with split partials")


@pytest.mark.parametrize("D", [64, 128])
def test_capture_gradients(gpu_device, D):
    import torch
    x = inputs.make_inputs(1, 4, 2, 300, 400, D, inputs.F16, seed=2)
    q, k, v = (to_device(a, inputs.F16, gpu_device) for a in (x.q, x.k, x.v))
    do = to_device(inputs.make_dout(x), inputs.F16, gpu_device)
    o, l = binding.attn_fwd(q, k, v, num_splits=1)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    binding.attn_bwd(q, k, v, o, l, do, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    refs = (dq.clone(), dk.clone(), dv.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        binding.attn_bwd(q, k, v, o, l, do, dq=dq, dk=dk, dv=dv)
    _replays(g, (dq, dk, dv), refs,
             f"attn_bwd D={D} ({'forked dQ stream' if D != 128 else 'one stream'})")
