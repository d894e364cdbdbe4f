"""The allocation-free forward (attn_fwd_noalloc) through the C ABI.

attn_fwd_noalloc runs attn_fwd_split's plan and kernels with the split-KV
partials in the library's per-device scratch array instead of a
stream-ordered allocation, so for the same arguments its output and
log-sum-exp must equal attn_fwd_split's bit for bit.  The calls run in a row
on one device with shrinking shapes (the array keeps the previous call's
contents), the first one at the 17160-token video shape, whose plan needs
most of the array; every split call is also checked against the oracle on
sampled rows.  A plan that needs more than the array returns ATTN_ESCRATCH
before anything is launched.
"""
import ctypes

import numpy as np
import pytest

from memory_efficient_tiled_amd import binding, inputs
from tests.parity import LSE_ERR, MAX_ERR, MEAN_ERR, half_ulp, log, oracle_rows, to_device

pytestmark = pytest.mark.gpu


def _launch(fn, q, k, v, out, lse, shape, scale, causal, dtype, splits):
    import torch
    B, Hq, Hkv, Nq, Nkv, D = shape
    stream = torch.cuda.current_stream(q.device).cuda_stream
    return fn(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
              ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(out.data_ptr()),
              ctypes.c_void_p(lse.data_ptr()), B, Hq, Hkv, Nq, Nkv, D, ctypes.c_float(scale),
              causal, dtype, splits, ctypes.c_void_p(stream))


def _compare(device, shape, dtype, causal, splits, seed, k_offset=None, check_rows=64):
    """One attn_fwd_noalloc call and one attn_fwd_split call on the same
    inputs; returns the plan's workspace bytes."""
    import torch
    lib = binding.load_library()
    B, Hq, Hkv, Nq, Nkv, D = shape
    dcode = binding.ATTN_BF16 if dtype == inputs.BF16 else binding.ATTN_F16
    plan = binding.attn_fwd_plan(B, Hq, Hkv, Nq, Nkv, D, causal, dcode, splits,
                                 torch.cuda.get_device_properties(device).multi_processor_count)
    log(f"noalloc B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nkv={Nkv} D={D} {dtype} causal={causal} "
        f"splits={splits}: plan {plan.num_splits} pieces, {plan.workspace_bytes} bytes")
    x = inputs.make_inputs(B, Hq, Hkv, Nq, Nkv, D, dtype, seed=seed, k_offset_std=k_offset)
    q, k, v = (to_device(a, dtype, device) for a in (x.q, x.k, x.v))
    outs = [torch.full((B, Hq, Nq, D), 7.0, dtype=q.dtype, device=device) for _ in range(2)]
    lses = [torch.full((B, Hq, Nq), 7.0, dtype=torch.float32, device=device) for _ in range(2)]
    scale = 1.0 / np.sqrt(D)
    rc_a = _launch(lib.attn_fwd_noalloc, q, k, v, outs[0], lses[0], shape, scale, int(causal),
                   dcode, splits)
    rc_b = _launch(lib.attn_fwd_split, q, k, v, outs[1], lses[1], shape, scale, int(causal),
                   dcode, splits)
    torch.cuda.synchronize(device)
    assert rc_a == binding.ATTN_OK, lib.attn_strerror(rc_a)
    assert rc_b == binding.ATTN_OK, lib.attn_strerror(rc_b)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), \
        "output differs from attn_fwd_split"
    assert torch.equal(lses[0].view(torch.int32), lses[1].view(torch.int32)), \
        "log-sum-exp differs from attn_fwd_split"
    # the oracle on sampled rows (first, last, seeded interior)
    rng = np.random.Generator(np.random.PCG64([seed, 7]))
    pick = np.unique(np.concatenate([[0, Nq - 1], rng.choice(Nq, min(Nq, check_rows),
                                                             replace=False)]))
    rows = np.tile(pick, (Hq, 1))
    o_ref, l_ref = oracle_rows(x, None, bool(causal), rows=rows)
    o = outs[0].float().cpu().numpy().astype(np.float64)[:, :, pick]
    ls = lses[0].cpu().numpy().astype(np.float64)[:, :, pick]
    err = np.abs(o - o_ref)
    lerr = np.abs(ls - l_ref)
    log(f"  max|err| {err.max():.3e} mean|err| {err.mean():.3e} lse {lerr.max():.3e}")
    assert np.all(err <= MAX_ERR + half_ulp(o_ref, dtype)) and err.mean() <= MEAN_ERR
    assert lerr.max() <= LSE_ERR
    return plan.workspace_bytes


def test_noalloc_matches_split_entry_point(gpu_device):
    # 1. the video shape: three rounds of 512-row tiles plus 48 tiles cut
    #    into key ranges, the largest workspace here (under 64 MiB)
    ws1 = _compare(gpu_device, (1, 24, 24, 17160, 17160, 128), inputs.BF16, 0, 0, seed=1,
                   k_offset=0.5, check_rows=16)
    assert 32 << 20 < ws1 <= binding.ATTN_NOALLOC_SCRATCH_BYTES
    # 2. smaller: a few query rows of 14/2 GQA over 20000 keys, every tile split
    ws2 = _compare(gpu_device, (1, 14, 2, 3, 20000, 128), inputs.BF16, 0, 0, seed=2)
    assert 0 < ws2 < ws1
    # 3. smaller again: causal, fp16, D = 64, three key ranges forced
    ws3 = _compare(gpu_device, (1, 2, 2, 130, 1500, 64), inputs.F16, 1, 3, seed=3)
    assert 0 < ws3 < ws2
    # 4. a plan that splits nothing leaves the array alone
    assert _compare(gpu_device, (1, 32, 32, 2048, 2048, 128), inputs.BF16, 0, 0, seed=4) == 0


def test_noalloc_rejects_oversized_plan(gpu_device):
    """16 forced key ranges over 16 heads x 8192 rows need ~1 GiB of
    partials: ATTN_ESCRATCH, and nothing is written."""
    import torch
    lib = binding.load_library()
    shape = (1, 16, 16, 8192, 8192, 128)
    plan = binding.attn_fwd_plan(*shape, False, binding.ATTN_BF16, 16, 256)
    assert plan.workspace_bytes > binding.ATTN_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((1, 16, 8192, 128), dtype=torch.bfloat16, device=gpu_device)
    out = torch.full_like(q, 3.0)
    lse = torch.full((1, 16, 8192), 3.0, dtype=torch.float32, device=gpu_device)
    rc = _launch(lib.attn_fwd_noalloc, q, q, q, out, lse, shape, 0.1, 0, binding.ATTN_BF16, 16)
    torch.cuda.synchronize(gpu_device)
    assert rc == binding.ATTN_ESCRATCH
    assert "scratch" in lib.attn_strerror(rc).decode()
    assert bool(torch.all(out == 3.0)) and bool(torch.all(lse == 3.0))
    # the Python wrapper raises with the same code
    with pytest.raises(binding.AttnError) as ei:
        binding.attn_fwd_noalloc(q, q, q, out, lse, num_splits=16)
    assert ei.value.code == binding.ATTN_ESCRATCH


def test_noalloc_graph_replays(gpu_device):
    """attn_fwd_noalloc captured in a HIP graph (the case it exists for: a
    capture may not allocate): three replays, with eager work, new query
    values copied into the captured buffer and a synchronisation between
    them; every replay equals attn_fwd_split on the same inputs bit for bit.
    Decode over 20000 keys with 14/2 GQA, so the plan splits and merges."""
    import torch
    shape = (1, 14, 2, 1, 20000, 128)
    B, Hq, Hkv, Nq, Nkv, D = shape
    x = inputs.make_inputs(B, Hq, Hkv, Nq, Nkv, D, inputs.BF16, seed=11)
    q, k, v = (to_device(a, inputs.BF16, gpu_device) for a in (x.q, x.k, x.v))
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=gpu_device)
    binding.attn_fwd_noalloc(q, k, v, out, lse)          # first call on the device
    torch.cuda.synchronize(gpu_device)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        binding.attn_fwd_noalloc(q, k, v, out, lse)
    torch.cuda.synchronize(gpu_device)
    lib = binding.load_library()
    for rep in range(3):
        qn = inputs.make_inputs(B, Hq, Hkv, Nq, Nkv, D, inputs.BF16, seed=100 + rep).q
        q.copy_(to_device(qn, inputs.BF16, gpu_device))  # eager work between replays
        torch.cuda.synchronize(gpu_device)
        g.replay()
        torch.cuda.synchronize(gpu_device)
        ref_o, ref_l = torch.full_like(out, 5.0), torch.full_like(lse, 5.0)
        rc = _launch(lib.attn_fwd_split, q, k, v, ref_o, ref_l, shape, 1.0 / np.sqrt(D), 0,
                     binding.ATTN_BF16, 0)
        torch.cuda.synchronize(gpu_device)
        assert rc == binding.ATTN_OK
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), f"replay {rep}"
        assert torch.equal(lse.view(torch.int32), ref_l.view(torch.int32)), f"replay {rep}"
        log(f"  graph replay {rep}: equal to the eager split entry point")
