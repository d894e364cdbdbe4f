"""GPU parity of strided layouts and of the SDPA front end against the oracle.

Inputs are the seeded generator's [B, H, N, D] arrays; on the device they
are stored in another layout and handed over as views, so the kernels read
them through strides.  Expected values come from the CPU oracle on the
logical arrays.
"""
import numpy as np
import pytest

from memory_efficient_tiled_amd import binding, inputs
from tests.parity import compare, gather_rows, log, oracle_rows, to_device

pytestmark = pytest.mark.gpu


def _view(a, dtype, device, layout):
    """Device view of logical [B, H, N, D] array `a` stored as `layout`."""
    if layout == "bhnd":
        return to_device(a, dtype, device)
    if layout == "bnhd":       # sequence-major storage, heads interleaved
        return to_device(np.ascontiguousarray(a.transpose(0, 2, 1, 3)), dtype,
                         device).transpose(1, 2)
    if layout == "padded":     # rows of D + 8 elements
        pad = np.zeros(a.shape[:3] + (8,), dtype=a.dtype)
        return to_device(np.concatenate([a, pad], axis=3), dtype, device)[..., :a.shape[3]]
    raise ValueError(layout)


def _empty_out(B, H, N, D, like, layout):
    import torch
    if layout == "bnhd":
        return torch.empty(B, N, H, D, dtype=like.dtype, device=like.device).transpose(1, 2)
    return torch.empty(B, H, N, D, dtype=like.dtype, device=like.device)


def _case(device, B, Hq, Hkv, Nq, Nkv, D, dtype, causal, layout, out_layout,
          seed, rows=None, num_splits=0):
    import torch
    log(f"strided case {layout}->{out_layout} B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} "
        f"Nkv={Nkv} D={D} {dtype} causal={causal} splits={num_splits}")
    x = inputs.make_inputs(B, Hq, Hkv, Nq, Nkv, D, dtype, seed=seed, sampled_rows=rows)
    q, k, v = (_view(a, dtype, device, layout) for a in (x.q, x.k, x.v))
    assert layout == "bhnd" or not q.is_contiguous()
    out = _empty_out(B, Hq, Nq, D, q, out_layout)
    o, l = binding.attn_fwd(q, k, v, causal=causal, out=out, num_splits=num_splits)
    torch.cuda.synchronize(device)
    o = o.float().cpu().numpy().astype(np.float64)
    l = l.cpu().numpy().astype(np.float64)
    r = None if rows is None else x.rows
    o_ref, l_ref = oracle_rows(x, None, causal, rows=r)
    if r is not None:
        o, l = gather_rows(o, r), gather_rows(l, r)
    compare(o, l, o_ref, l_ref, dtype, rounding_allowance=True,
            what=f"{layout} N={Nq}x{Nkv} D={D} {dtype} causal={causal}")


def test_strided_wide_d128_with_last_round_split(gpu_device):
    # 512-row tiles, 64 x 5 = 320 tiles: the last 64 are split and merged,
    # the merge writing through the output's strides
    _case(gpu_device, 1, 64, 8, 2100, 1000, 128, inputs.BF16, False, "bnhd", "bnhd",
          seed=21, rows=24)


@pytest.mark.parametrize("causal", [False, True])
def test_strided_narrow_d128(gpu_device, causal):
    _case(gpu_device, 2, 4, 2, 300, 300, 128, inputs.BF16, causal, "bnhd", "bhnd", seed=22)


def test_padded_rows_gqa_causal_d64(gpu_device):
    _case(gpu_device, 1, 14, 2, 1000, 1000, 64, inputs.F16, True, "padded", "padded",
          seed=23, rows=64)


def test_strided_wide_d64(gpu_device):
    _case(gpu_device, 2, 32, 8, 2100, 2000, 64, inputs.F16, False, "bnhd", "bnhd",
          seed=24, rows=24)


@pytest.mark.parametrize("splits", [3, 8])
def test_strided_forced_splits(gpu_device, splits):
    _case(gpu_device, 1, 3, 1, 200, 1500, 64, inputs.F16, True, "bnhd", "bnhd",
          seed=25, num_splits=splits)


# -- the SDPA front end --------------------------------------------------------

def _oracle_out(x, causal):
    o_ref, _ = oracle_rows(x, None, causal)
    return o_ref


def test_sdpa_matches_oracle(gpu_device):
    import torch
    import memory_efficient_tiled_amd as mta
    x = inputs.make_inputs(2, 8, 2, 333, 333, 128, inputs.BF16, seed=26)
    q, k, v = (_view(a, inputs.BF16, gpu_device, "bnhd") for a in (x.q, x.k, x.v))
    o = mta.sdpa(q, k, v, is_causal=True, enable_gqa=True)
    torch.cuda.synchronize(gpu_device)
    assert o.shape == q.shape and o.is_contiguous()
    compare(o.float().cpu().numpy().astype(np.float64), None, _oracle_out(x, True), None,
            inputs.BF16, rounding_allowance=True, what="sdpa 4-D")


def test_sdpa_three_dimensional(gpu_device):
    import torch
    import memory_efficient_tiled_amd as mta
    x = inputs.make_inputs(1, 4, 4, 100, 260, 64, inputs.F16, seed=27)
    q, k, v = (to_device(a, inputs.F16, gpu_device)[0] for a in (x.q, x.k, x.v))
    o = mta.sdpa(q, k, v)
    torch.cuda.synchronize(gpu_device)
    assert o.shape == q.shape
    compare(o.float().cpu().numpy().astype(np.float64)[None], None, _oracle_out(x, False),
            None, inputs.F16, rounding_allowance=True, what="sdpa 3-D")


def test_patched_torch_sdpa(gpu_device):
    import torch
    import torch.nn.functional as F
    import memory_efficient_tiled_amd as mta
    x = inputs.make_inputs(1, 4, 4, 150, 150, 64, inputs.F16, seed=28)
    q, k, v = (to_device(a, inputs.F16, gpu_device) for a in (x.q, x.k, x.v))
    try:
        mta.patch(fallback=True)
        s0 = mta.sdpa_stats()
        o = F.scaled_dot_product_attention(q, k, v, is_causal=True)
        torch.cuda.synchronize(gpu_device)
        s1 = mta.sdpa_stats()
        assert s1["native"] == s0["native"] + 1
        compare(o.float().cpu().numpy().astype(np.float64), None, _oracle_out(x, True),
                None, inputs.F16, rounding_allowance=True, what="patched sdpa")
        # float32 is not served: handed to PyTorch's own (float32) attention
        qf, kf, vf = q.float(), k.float(), v.float()
        F.scaled_dot_product_attention(qf, kf, vf)
        torch.cuda.synchronize(gpu_device)
        assert mta.sdpa_stats()["fallback"] == s1["fallback"] + 1
    finally:
        mta.unpatch()


def test_auto_patch_follows_the_backend_probe(gpu_device):
    """With PyTorch's flash and memory-efficient kernels switched off, the
    probe finds no fused backend and auto_patch routes SDPA here; with them
    on, it patches exactly when the probe still finds none."""
    import torch
    import torch.nn.functional as F
    import memory_efficient_tiled_amd as mta
    orig = F.scaled_dot_product_attention
    flash, eff = (torch.backends.cuda.flash_sdp_enabled(),
                  torch.backends.cuda.mem_efficient_sdp_enabled())
    x = inputs.make_inputs(1, 2, 2, 70, 70, 64, inputs.F16, seed=29)
    q, k, v = (to_device(a, inputs.F16, gpu_device) for a in (x.q, x.k, x.v))
    try:
        torch.backends.cuda.enable_flash_sdp(False)
        torch.backends.cuda.enable_mem_efficient_sdp(False)
        assert mta.efficient_backend_available(gpu_device) is False
        assert mta.auto_patch(device=gpu_device) is True
        s0 = mta.sdpa_stats()["native"]
        o = F.scaled_dot_product_attention(q, k, v)
        torch.cuda.synchronize(gpu_device)
        assert mta.sdpa_stats()["native"] == s0 + 1
        compare(o.float().cpu().numpy().astype(np.float64), None, _oracle_out(x, False),
                None, inputs.F16, rounding_allowance=True, what="auto-patched sdpa")
        mta.unpatch()
        torch.backends.cuda.enable_flash_sdp(True)
        torch.backends.cuda.enable_mem_efficient_sdp(True)
        fused = mta.efficient_backend_available(gpu_device)
        log(f"  PyTorch fused SDPA kernel on this device: {fused}")
        assert mta.auto_patch(device=gpu_device) is (not fused)
        assert (F.scaled_dot_product_attention is not orig) is (not fused)
    finally:
        mta.unpatch()
        torch.backends.cuda.enable_flash_sdp(flash)
        torch.backends.cuda.enable_mem_efficient_sdp(eff)
    assert F.scaled_dot_product_attention is orig


def test_sdpa_causal_lower_right_bias(gpu_device):
    """PyTorch's lower-right causal bias as attn_mask: bottom-right alignment
    in the forward and under autograd."""
    import torch
    from torch.nn.attention.bias import causal_lower_right
    import oracle
    import memory_efficient_tiled_amd as mta
    from tests.test_backward_gpu import check_grad, delta_terms
    x = inputs.make_inputs(1, 4, 2, 96, 400, 64, inputs.BF16, seed=29)
    do = inputs.make_dout(x)
    leaves = [to_device(a, inputs.BF16, gpu_device).requires_grad_(True)
              for a in (x.q, x.k, x.v)]
    o = mta.sdpa(*leaves, attn_mask=causal_lower_right(96, 400), enable_gqa=True)
    o.backward(to_device(do, inputs.BF16, gpu_device))
    torch.cuda.synchronize(gpu_device)
    o_ref, _ = oracle_rows(x, None, True, causal_offset=304)
    compare(o.detach().float().cpu().numpy().astype(np.float64), None, o_ref, None,
            inputs.BF16, rounding_allowance=True, what="sdpa lower-right")
    dec = [oracle.decode(a, inputs.BF16) for a in (x.q, x.k, x.v, do)]
    ref = oracle.attention_backward(*dec, oracle.scale_value(None, 64), True,
                                    causal_offset=304)
    terms = delta_terms(x, do, ref, True, 304)
    for name, leaf, r, t in zip(("dq", "dk", "dv"), leaves, ref, terms):
        check_grad(name, leaf.grad.float().cpu().numpy().astype(np.float64), r,
                   inputs.BF16, "sdpa lower-right autograd", None, t)


def test_custom_ops_opcheck(gpu_device):
    """torch.library.opcheck: schema, fake implementation and autograd
    registration of the custom ops against real runs."""
    import torch
    import memory_efficient_tiled_amd as mta
    att, bwd = mta.torch_ops()
    assert mta.available()
    x = inputs.make_inputs(1, 4, 2, 130, 200, 64, inputs.BF16, seed=31)
    q, k, v = (to_device(a, inputs.BF16, gpu_device).requires_grad_(True)
               for a in (x.q, x.k, x.v))
    for causal in (0, 1, 2):
        torch.library.opcheck(att, (q, k, v, None, causal, 0.125),
                              test_utils=("test_schema", "test_faketensor",
                                          "test_autograd_registration"))
    keep = torch.rand(1, 1, 130, 200, device=gpu_device) < 0.7
    qd, kd, vd = (t.detach() for t in (q, k, v))
    torch.library.opcheck(att, (qd, kd, vd, keep, 0, 0.125),
                          test_utils=("test_schema", "test_faketensor"))


def test_sdpa_compiles_without_graph_break(gpu_device):
    """torch.compile(fullgraph=True) traces sdpa through the custom op (the
    aot_eager backend: no code generation), forward and backward."""
    import torch
    import memory_efficient_tiled_amd as mta
    x = inputs.make_inputs(1, 4, 4, 120, 120, 64, inputs.F16, seed=32)
    q, k, v = (to_device(a, inputs.F16, gpu_device).requires_grad_(True)
               for a in (x.q, x.k, x.v))
    w = torch.linspace(-1.0, 1.0, 64, device=gpu_device)

    def loss_fn(a, b, c):
        return (mta.sdpa(a, b, c, is_causal=True).float() * w).sum()

    f = torch.compile(loss_fn, fullgraph=True, backend="aot_eager")
    loss = f(q, k, v)
    loss.backward()
    grads = [t.grad.clone() for t in (q, k, v)]
    for t in (q, k, v):
        t.grad = None
    ref = loss_fn(q, k, v)           # eager: the same kernels, so the same bits
    ref.backward()
    torch.cuda.synchronize(gpu_device)
    assert torch.equal(loss, ref)
    for g, t in zip(grads, (q, k, v)):
        assert torch.equal(g, t.grad)
    o_ref, _ = oracle_rows(x, None, True)
    want = float((o_ref * np.linspace(-1.0, 1.0, 64)).sum())
    assert abs(float(loss.detach()) - want) <= 2e-3 * o_ref.size ** 0.5


def test_sdpa_tensor_masks(gpu_device):
    """Boolean and additive attn_mask tensors through sdpa and the patched
    PyTorch call (no autograd)."""
    import torch
    import torch.nn.functional as F
    import oracle
    import memory_efficient_tiled_amd as mta
    x = inputs.make_inputs(2, 4, 4, 100, 130, 64, inputs.F16, seed=33)
    q, k, v = (to_device(a, inputs.F16, gpu_device) for a in (x.q, x.k, x.v))
    rng = np.random.Generator(np.random.PCG64(34))
    keep = rng.random((2, 1, 100, 130)) < 0.6
    add = inputs.to_storage(rng.standard_normal((100, 130)).astype(np.float32), inputs.F16)
    sc = oracle.scale_value(None, 64)
    dec = [oracle.decode(a, inputs.F16) for a in (x.q, x.k, x.v)]
    for m, bias in ((torch.from_numpy(keep).to(gpu_device), np.where(keep, 0.0, -np.inf)),
                    (to_device(add, inputs.F16, gpu_device), oracle.decode(add, inputs.F16))):
        o = mta.sdpa(q, k, v, attn_mask=m)
        try:
            mta.patch()
            o2 = F.scaled_dot_product_attention(q, k, v, attn_mask=m)
        finally:
            mta.unpatch()
        torch.cuda.synchronize(gpu_device)
        assert torch.equal(o, o2)
        o_ref, _ = oracle.attention(*dec, sc, False, bias=np.broadcast_to(bias, (2, 4, 100, 130)))
        compare(o.float().cpu().numpy().astype(np.float64), None, o_ref, None, inputs.F16,
                rounding_allowance=True, what=f"sdpa mask {m.dtype}")
