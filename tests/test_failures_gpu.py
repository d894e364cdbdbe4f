"""Failure handling on the GPU: a workspace that cannot be allocated.

The library takes its workspaces stream-ordered (split-KV partials, the
gradients' per-row Delta, the FFN's hidden chunk, the FP8 path's transposed
V).  With ATTN_FAIL_WORKSPACE=1 in the environment every such request fails
as an out-of-memory error would, before anything is launched: each entry
point must return ATTN_ENOMEM (raised as AttnError by the binding), leave
its outputs untouched, and work again once the condition is gone.  Calls
that need no workspace are unaffected, and attn_fwd_noalloc, which never
allocates, runs the same split plan regardless.
"""
import os

import numpy as np
import pytest

from memory_efficient_tiled_amd import binding, inputs
from tests.parity import log, to_device

pytestmark = pytest.mark.gpu


class _FailWorkspace:
    def __enter__(self):
        os.environ["ATTN_FAIL_WORKSPACE"] = "1"

    def __exit__(self, *exc):
        os.environ.pop("ATTN_FAIL_WORKSPACE", None)


def _expect_enomem(fn):
    with pytest.raises(binding.AttnError) as ei:
        fn()
    assert ei.value.code == binding.ATTN_ENOMEM, ei.value


def test_forward_enomem(gpu_device):
    import torch
    # a decode-like shape: every tile is split, so the forward needs a workspace
    x = inputs.make_inputs(1, 14, 2, 3, 20000, 128, inputs.BF16, seed=600)
    q, k, v = (to_device(a, inputs.BF16, gpu_device) for a in (x.q, x.k, x.v))
    assert binding.attn_fwd_plan(1, 14, 2, 3, 20000, 128, False, binding.ATTN_BF16).workspace_bytes > 0
    out = torch.full_like(q, 3.0)
    lse = torch.full((1, 14, 3), 3.0, dtype=torch.float32, device=gpu_device)
    with _FailWorkspace():
        _expect_enomem(lambda: binding.attn_fwd(q, k, v, out=out, lse=lse))
        torch.cuda.synchronize(gpu_device)
        assert bool(torch.all(out == 3.0)) and bool(torch.all(lse == 3.0)), "nothing may run"
        # the allocation-free entry point runs the same plan
        o2 = torch.empty_like(q)
        l2 = torch.empty_like(lse)
        binding.attn_fwd_noalloc(q, k, v, o2, l2)
        # a call that splits nothing needs no workspace
        binding.attn_fwd(q, k, v, out=out, lse=lse, num_splits=1)
    torch.cuda.synchronize(gpu_device)
    ref_o, ref_l = binding.attn_fwd(q, k, v)
    torch.cuda.synchronize(gpu_device)
    assert torch.equal(o2, ref_o) and torch.equal(l2, ref_l)
    assert float((out.float() - ref_o.float()).abs().max()) < 1e-2
    log("  forward: ENOMEM with the injected failure, same results without it")


def test_gradients_enomem(gpu_device):
    import torch
    x = inputs.make_inputs(1, 4, 2, 200, 300, 64, inputs.F16, seed=601)
    q, k, v, g = (to_device(a, inputs.F16, gpu_device)
                  for a in (x.q, x.k, x.v, inputs.make_dout(x)))
    out, lse = binding.attn_fwd(q, k, v, num_splits=1)
    dq, dk, dv = (torch.full_like(t, 3.0) for t in (q, k, v))
    with _FailWorkspace():
        _expect_enomem(lambda: binding.attn_bwd(q, k, v, out, lse, g, dq=dq, dk=dk, dv=dv))
        torch.cuda.synchronize(gpu_device)
        assert all(bool(torch.all(t == 3.0)) for t in (dq, dk, dv)), "nothing may run"
    r = binding.attn_bwd(q, k, v, out, lse, g)
    torch.cuda.synchronize(gpu_device)
    assert all(bool(torch.isfinite(t.float()).all()) for t in r)


def test_ffn_enomem(gpu_device):
    import torch
    from memory_efficient_tiled_amd import ffn_chunked
    xi = inputs.make_ffn_inputs(300, 64, 256, inputs.BF16, seed=602)
    x, w1, b1, w2, b2 = (to_device(a, inputs.BF16, gpu_device)
                         for a in (xi.x, xi.w1, xi.b1, xi.w2, xi.b2))
    y = torch.full_like(x, 3.0)
    with _FailWorkspace():
        _expect_enomem(lambda: ffn_chunked(x, w1, b1, w2, b2, chunk_rows=100, out=y))
        _expect_enomem(lambda: ffn_chunked(x, w1, b1, w2, b2, chunk_rows=100, verify=True))
        torch.cuda.synchronize(gpu_device)
        assert bool(torch.all(y == 3.0)), "nothing may run"
    ffn_chunked(x, w1, b1, w2, b2, chunk_rows=100, out=y, verify=True)
    torch.cuda.synchronize(gpu_device)
    assert bool(torch.isfinite(y.float()).all())


def test_fp8_enomem(gpu_device):
    import torch
    x = inputs.make_inputs(1, 2, 2, 100, 300, 128, inputs.FP8, seed=603)
    q, k, v = (torch.from_numpy(np.ascontiguousarray(a)).to(gpu_device)
               .view(torch.float8_e4m3fn) for a in (x.q, x.k, x.v))
    with _FailWorkspace():
        _expect_enomem(lambda: binding.attn_fwd_fp8(q, k, v, x.q_descale, x.k_descale,
                                                    x.v_descale))
    o, _ = binding.attn_fwd_fp8(q, k, v, x.q_descale, x.k_descale, x.v_descale)
    torch.cuda.synchronize(gpu_device)
    assert bool(torch.isfinite(o.float()).all())


def test_workspace_pool_keeps_memory(gpu_device):
    """The library's workspace pool keeps what it handed out across a device
    synchronisation (release threshold at the maximum), can be trimmed by
    the caller, and serves the next call afterwards."""
    import ctypes
    import torch
    path = next(ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64.so" in ln)
    hip = ctypes.CDLL(path)
    pool = ctypes.c_void_p(binding.workspace_pool())
    assert pool.value == binding.workspace_pool(), "one pool per device"

    def reserved():
        v = ctypes.c_uint64(0)
        assert hip.hipMemPoolGetAttribute(pool, 0x5, ctypes.byref(v)) == 0  # ReservedMemCurrent
        return int(v.value)

    x = inputs.make_inputs(1, 14, 2, 3, 20000, 128, inputs.BF16, seed=604)
    q, k, v = (to_device(a, inputs.BF16, gpu_device) for a in (x.q, x.k, x.v))
    ws = binding.attn_fwd_plan(1, 14, 2, 3, 20000, 128, False, binding.ATTN_BF16).workspace_bytes
    assert ws > 0
    o1, l1 = binding.attn_fwd(q, k, v)
    torch.cuda.synchronize(gpu_device)
    assert reserved() >= ws, "the workspace was returned at the synchronisation"
    assert hip.hipMemPoolTrimTo(pool, ctypes.c_size_t(0)) == 0
    o2, l2 = binding.attn_fwd(q, k, v)
    torch.cuda.synchronize(gpu_device)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    log(f"  workspace pool: {reserved()} bytes reserved after the call (plan {ws})")
