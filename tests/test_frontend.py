"""CPU tests of the SDPA front end and the strided C ABI validation.

No GPU work: the front end's argument screening runs on CPU tensors (every
check before the device check), patch() is exercised with CPU calls that it
hands to PyTorch, and the strided validation entry point makes no HIP call.
"""
import ctypes

import pytest
import torch
import torch.nn.functional as F

import memory_efficient_tiled_amd as mta
from memory_efficient_tiled_amd import binding, frontend

OK, EINVAL = binding.ATTN_OK, binding.ATTN_EINVAL
BF16 = binding.ATTN_BF16
Q, K, V, O, L = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


def t(*shape, dtype=torch.float16, **kw):
    return torch.zeros(*shape, dtype=dtype, **kw)


def reason(q, k, v, **kw):
    return frontend.unsupported_reason(q, k, v, **kw)


def test_cpu_tensors_only_fail_the_device_check():
    q = t(2, 4, 100, 64)
    assert reason(q, q, q) == "inputs must be on one HIP device"
    # [B, N, H, E] storage viewed as [B, H, N, E]: accepted layout
    s = t(2, 100, 4, 128).transpose(1, 2)
    assert reason(s, s, s) == "inputs must be on one HIP device"


@pytest.mark.parametrize("kw,frag", [
    ({"attn_mask": t(100, 100, dtype=torch.float32)}, "attn_mask must be bool"),
    ({"attn_mask": t(3, 100, 100, dtype=torch.bool)}, "broadcast"),
    ({"attn_mask": t(100, 100, dtype=torch.bool), "is_causal": True}, "is_causal"),
    ({"dropout_p": 0.1}, "dropout"),
])
def test_unsupported_arguments(kw, frag):
    q = t(1, 2, 100, 64)
    assert frag in reason(q, q, q, **kw)


def test_unsupported_inputs():
    q = t(1, 2, 100, 64)
    assert "dtype" in reason(q.float(), q.float(), q.float())
    assert "head dimension" in reason(t(1, 2, 10, 72), t(1, 2, 10, 72), t(1, 2, 10, 72))
    for e in (80, 96, 256):
        w = t(1, 2, 10, e)
        assert reason(w, w, w) == "inputs must be on one HIP device"
    wg = t(1, 2, 10, 256).requires_grad_()     # gradients at every head dim
    assert reason(wg, wg, wg) == "inputs must be on one HIP device"
    assert "3-D" in reason(t(2, 100, 64)[0], t(2, 100, 64)[0], t(2, 100, 64)[0])
    k = t(1, 1, 100, 64)
    assert "enable_gqa" in reason(q, k, k)
    assert reason(q, k, k, enable_gqa=True) == "inputs must be on one HIP device"
    assert "multiple" in reason(t(1, 3, 10, 64), t(1, 2, 10, 64), t(1, 2, 10, 64),
                                enable_gqa=True)
    assert "last dimension" in reason(t(1, 2, 64, 100).transpose(2, 3), q, q)
    padded = t(1, 2, 100, 68)[..., :64]          # row stride 68: not a multiple of 8
    assert "multiples of 8" in reason(padded, padded, padded)
    g = t(1, 2, 10, 64).requires_grad_()      # differentiable: served (on a device)
    assert reason(g, g, g) == "inputs must be on one HIP device"
    assert "scale" in reason(q, q, q, scale=float("inf"))


def test_tensor_masks_are_served():
    q = t(2, 4, 100, 64)
    for m in (t(100, 100, dtype=torch.bool), t(2, 1, 100, 100), t(2, 4, 1, 100),
              t(100, 1, dtype=torch.bool)):
        assert reason(q, q, q, attn_mask=m) == "inputs must be on one HIP device"
    g = t(2, 4, 100, 64).requires_grad_()   # masked gradients: served
    assert reason(g, g, g, attn_mask=t(100, 100, dtype=torch.bool)) == \
        "inputs must be on one HIP device"
    g256 = t(2, 4, 100, 256).requires_grad_()
    assert reason(g256, g256, g256, attn_mask=t(100, 100, dtype=torch.bool)) == \
        "inputs must be on one HIP device"


def test_mask_view_broadcasts_without_copies():
    """Broadcast dimensions get stride 0; keys stay contiguous; rows that are
    not a multiple of 4 elements are padded in one copy of the mask's own
    shape."""
    m = torch.ones(1, 1, 10, 64, dtype=torch.bool)
    v, mtype, st = binding.mask_view(m, 2, 3, 10, 64, torch.float16)
    assert mtype == binding.ATTN_MASK_BOOL and tuple(v.shape) == (2, 3, 10, 64)
    assert (st[0], st[1], st[2]) == (0, 0, 64) and v.data_ptr() == m.data_ptr()
    a = torch.randn(3, 10, 30).half()                  # 30 keys: padded to 32
    v, mtype, st = binding.mask_view(a, 2, 3, 10, 30, torch.float16)
    assert mtype == binding.ATTN_MASK_ADD and (st[0], st[1], st[2]) == (0, 320, 32)
    assert torch.equal(v[1], a)
    kp = torch.tensor([True] * 20 + [False] * 10).reshape(1, 1, 1, 30)  # key padding
    v, _, st = binding.mask_view(kp, 2, 3, 10, 30, torch.float16)
    assert (st[0], st[1], st[2]) == (0, 0, 0) and bool(v[1, 2, 7, 19]) and not bool(v[1, 2, 7, 20])
    with pytest.raises(TypeError):
        binding.mask_view(a.float(), 2, 3, 10, 30, torch.float16)


def test_causal_biases_are_served():
    from torch.nn.attention.bias import causal_lower_right, causal_upper_left
    q, k = t(1, 2, 10, 64), t(1, 2, 30, 64)
    assert reason(q, k, k, attn_mask=causal_lower_right(10, 30)) == \
        "inputs must be on one HIP device"
    assert reason(q, k, k, attn_mask=causal_upper_left(10, 30)) == \
        "inputs must be on one HIP device"
    assert "lengths" in reason(q, k, k, attn_mask=causal_lower_right(10, 31))
    assert "is_causal" in reason(q, k, k, attn_mask=causal_lower_right(10, 30),
                                 is_causal=True)
    assert frontend.causal_mode(causal_lower_right(10, 30), False) == "bottom_right"
    assert frontend.causal_mode(causal_upper_left(10, 30), False) == "top_left"
    assert frontend.causal_mode(None, True) == "top_left"
    assert frontend.causal_mode(None, False) is False


def test_causal_codes():
    assert binding.causal_code(False) == 0 and binding.causal_code(True) == 1
    assert binding.causal_code("top_left") == 1
    assert binding.causal_code("bottom_right") == 2
    with pytest.raises(ValueError):
        binding.causal_code("diagonal")


def test_sdpa_raises_for_unsupported_calls():
    q = t(1, 2, 10, 64)
    with pytest.raises(NotImplementedError):
        mta.sdpa(q, q, q, attn_mask=t(10, 10))


def test_patch_routes_and_restores():
    orig = F.scaled_dot_product_attention
    q = torch.randn(1, 2, 10, 64)
    ref = orig(q, q, q)
    try:
        mta.patch(fallback=False)
        assert F.scaled_dot_product_attention is not orig
        with pytest.raises(NotImplementedError):
            F.scaled_dot_product_attention(q, q, q)     # CPU: not served, no fallback
        mta.patch(fallback=True)
        before = mta.sdpa_stats()["fallback"]
        out = F.scaled_dot_product_attention(q, q, q)
        assert torch.equal(out, ref)
        assert mta.sdpa_stats()["fallback"] == before + 1
    finally:
        mta.unpatch()
    assert F.scaled_dot_product_attention is orig


def strides(*s):
    return (ctypes.c_longlong * 3)(*s)


def check(qs=None, ks=None, vs=None, os_=None, B=2, Hq=4, Hkv=2, Nq=100, Nkv=300,
          D=128, out=O):
    lib = mta.load_library()
    return lib.attn_fwd_strided_check(Q, K, V, out, L, B, Hq, Hkv, Nq, Nkv, D,
                                      qs, ks, vs, os_, 0.088, 0, BF16)


def test_strided_check_accepts_common_layouts():
    assert check() == OK                                           # NULL: contiguous
    # [B, N, H, D] storage of every tensor
    assert check(strides(100 * 4 * 128, 128, 4 * 128), strides(300 * 2 * 128, 128, 2 * 128),
                 strides(300 * 2 * 128, 128, 2 * 128), strides(100 * 4 * 128, 128, 4 * 128)) == OK
    # padded rows, broadcast batch stride of K/V (B > 1, stride 0 for reads only)
    assert check(qs=strides(4 * 100 * 136, 100 * 136, 136), ks=strides(0, 300 * 128, 128)) == OK
    # contiguous layout spelled out equals NULL
    lib = mta.load_library()
    assert lib.attn_fwd_check(Q, K, V, O, L, 2, 4, 2, 100, 300, 128, 0.088, 0, BF16) == OK


@pytest.mark.parametrize("kw", [
    {"qs": strides(4 * 100 * 128, 100 * 128, 64)},         # row stride < D
    {"ks": strides(0, 300 * 128, 132)},                     # not a multiple of 8
    {"vs": strides(-8, 300 * 128, 128)},                     # negative
    {"ks": strides(0, 0, 1 << 25)},                          # row stride > 2^24
    {"os_": strides(4 * 100 * 128, 0, 128)},                 # output heads overlap
    {"os_": strides(4 * 100 * 128, 128, 128)},               # output rows overlap heads
    {"os_": strides(4 * 100 * 128, 100 * 128, 128), "out": Q + 256},  # out overlaps q
])
def test_strided_check_rejects(kw):
    assert check(**kw) == EINVAL


def test_custom_op_fake_shapes():
    """The custom ops' fake implementations give the output shapes on meta
    tensors (what tracing sees); no kernel runs."""
    mta.torch_ops()
    q = torch.empty(2, 4, 10, 64, device="meta", dtype=torch.bfloat16)
    k = torch.empty(2, 2, 30, 64, device="meta", dtype=torch.bfloat16)
    o, lse = torch.ops.memory_efficient_tiled_amd.attention(q, k, k, None, 1, 0.125)
    assert o.shape == q.shape and o.dtype == q.dtype and o.is_contiguous()
    assert lse.shape == (2, 4, 10) and lse.dtype == torch.float32
    dq, dk, dv = torch.ops.memory_efficient_tiled_amd.attention_backward(
        o, q, k, k, o, lse, None, 2, 0.125)
    assert dq.shape == q.shape and dk.shape == k.shape and dv.shape == k.shape


def test_backend_probe_without_gpu():
    assert mta.available() is False
    assert mta.efficient_backend_available() is False


@pytest.mark.parametrize("usable,fused,patched", [(False, False, False), (False, True, False),
                                                 (True, True, False), (True, False, True)])
def test_auto_patch_rule(monkeypatch, usable, fused, patched):
    """Patched exactly when the library can run on the device and PyTorch has
    no fused SDPA kernel there; calls it cannot serve then fall back."""
    from memory_efficient_tiled_amd import frontend
    orig = F.scaled_dot_product_attention
    monkeypatch.setattr(frontend, "available", lambda device=None: usable)
    monkeypatch.setattr(frontend, "efficient_backend_available", lambda device=None: fused)
    try:
        assert frontend.auto_patch() is patched
        assert (F.scaled_dot_product_attention is not orig) is patched
        if patched:
            q = torch.randn(1, 2, 10, 64)       # CPU tensors: handed to PyTorch
            assert torch.equal(F.scaled_dot_product_attention(q, q, q), orig(q, q, q))
    finally:
        mta.unpatch()
    assert F.scaled_dot_product_attention is orig


def test_value_head_dimension():
    """Query/key head dim 192 with value head dim 128 is served, with or
    without gradients; other pairs go elsewhere."""
    q, v = t(1, 2, 10, 192), t(1, 2, 10, 128)
    assert reason(q, q, v) == "inputs must be on one HIP device"
    assert "head dimension" in reason(t(1, 2, 10, 128), t(1, 2, 10, 128), t(1, 2, 10, 64))
    assert "head dimension" in reason(q, q, t(1, 2, 10, 192 + 64))
    assert "head dimension" in reason(v, q, v)                 # key width differs from query
    qg = t(1, 2, 10, 192).requires_grad_()
    assert reason(qg, q, v) == "inputs must be on one HIP device"
    assert "one shape" in reason(q, q, t(1, 2, 11, 128))
    # value rows strided by the value's width: [B, N, H, 128] storage
    vs = t(1, 10, 2, 128).transpose(1, 2)
    assert reason(q, q, vs) == "inputs must be on one HIP device"


def test_custom_op_fake_shapes_value_width():
    mta.torch_ops()
    q = torch.empty(1, 4, 10, 192, device="meta", dtype=torch.bfloat16)
    v = torch.empty(1, 4, 30, 128, device="meta", dtype=torch.bfloat16)
    k = torch.empty(1, 4, 30, 192, device="meta", dtype=torch.bfloat16)
    o, lse = torch.ops.memory_efficient_tiled_amd.attention(q, k, v, None, 0, 0.07)
    assert o.shape == (1, 4, 10, 128) and lse.shape == (1, 4, 10)
    dq, dk, dv = torch.ops.memory_efficient_tiled_amd.attention_backward(
        o, q, k, v, o, lse, None, 1, 0.07)
    assert dq.shape == q.shape and dk.shape == k.shape and dv.shape == v.shape
