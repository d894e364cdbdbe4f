"""GPU parity of the attention gradients (dQ, dK, dV) against the oracle.

The forward runs on the GPU (its output and log-sum-exp feed the gradient
kernels, as in training); the oracle computes the exact float64 gradients
from the same 16-bit inputs and the same seeded output gradient.

Tolerance.  Each gradient row (the D values of one query row of dQ, or of
one key row of dK, dV) is a sum over keys (dQ) or queries (dK, dV) of terms
x_t in which one 16-bit operand was rounded from fp32 by the kernel (P or
dS, relative error <= u = 2^-8 for bf16, 2^-11 for fp16), the other an exact
input, accumulated in fp32.  The rounding errors are independent from term
to term, so an element's error has a standard deviation of about
u / sqrt(3) * sqrt(sum_t x_t^2).  The other factor of every term (dO, Q or
K) is an input of zero mean, so sqrt(sum_t x_t^2) is also about the
root-mean-square of that gradient row, rms_row(ref).  Delta = <dO, O> is
read from the 16-bit output, whose elements are off by about u |O|: Delta_i
is off by about u b_i, b_i = sqrt(sum_d (dO_id O_id)^2), and every dS_ij of
row i by P_ij u b_i.  In dQ_i that adds scale u b_i |sum_j P_ij K_j| (the
oracle's attention output with K in place of V); in dK_j it adds terms of
random sign whose root sum of squares is at most
scale u max_i(b_i) max|Q| sqrt(sum_i P_ij^2) (causal: the max over the rows
i >= j that see key j), and sqrt(sum_i P_ij^2) is rms_row(dV_j) (dO has unit
variance).  This term dominates in short causal
rows, where dS nearly cancels.  The bounds are max|err| <= 12 u rms_row(ref)
+ 2 u rms(ref) + the Delta term (x12 for dQ, x6 for dK, whose estimate
already takes maxima) + half an ulp of the output type (beyond 6 standard
deviations), and mean|err| <= 1.5 u rms(ref) (the mean of |N(0, s)| is
0.8 s).  Keys that no query may see
(causal, key index >= Nq) must get exactly zero gradients.
"""
import numpy as np
import pytest

import oracle
from memory_efficient_tiled_amd import binding, inputs
from tests.parity import half_ulp, log, to_device

pytestmark = pytest.mark.gpu

U = {inputs.BF16: 2.0 ** -8, inputs.F16: 2.0 ** -11}


def _decode(a, dtype):
    return oracle.decode(a, dtype)


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


def check_grad(name, got, ref, dtype, what, zero_from=None, extra=0.0):
    """Compare one gradient; keys zero_from.. along axis 2 must be exactly 0;
    `extra` (per row or element) is the bound's Delta term."""
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what} {name}: non-finite values"
    err = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    rms_row = np.sqrt(np.mean(ref ** 2, axis=-1, keepdims=True))
    u = U[dtype]
    bound = 12.0 * u * rms_row + 2.0 * u * rms + extra + half_ulp(ref, dtype)
    mbound = 1.5 * u * rms
    ratio = float(np.max(err / (u * rms_row + u * rms + 1e-300)))
    log(f"  {what} {name}: max|err| {err.max():.3e} mean|err| {err.mean():.3e} "
        f"rms(ref) {rms:.3e} (max err/(u (rms_row + rms)) {ratio:.2f}, "
        f"mean/(u rms) {err.mean() / (u * rms + 1e-300):.2f})")
    if zero_from is not None:
        assert np.all(ref[:, :, zero_from:] == 0.0)
        assert np.all(got[:, :, zero_from:] == 0.0), \
            f"{what} {name}: non-zero gradient for keys no query sees"
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), f"{what} {name}: err {err[worst]:.3e} at {worst} > bound"
    # The mean criterion is relative to rms(ref).  An identically zero exact
    # gradient (one key: dS = P (dP - Delta) = 0) leaves only rounding noise
    # of dP - Delta, which the element bound's Delta term covers.
    if rms > 0.0:
        assert err.mean() <= mbound, f"{what} {name}: mean err {err.mean():.3e} > {mbound:.3e}"


def delta_terms(x, do, ref, causal, causal_offset=0, bias=None):
    """Per-row Delta terms of the bound for (dq, dk, dv) (see the header),
    for the inputs ``x`` and output gradient ``do``."""
    dec = [_decode(a, x.dtype) for a in (x.q, x.k, x.v, do)]
    return delta_terms_dec(dec, ref, x.dtype, causal, causal_offset, bias)


def delta_terms_dec(dec, ref, dtype, causal, causal_offset=0, bias=None):
    """Delta terms from decoded (q, k, v, dO).  ``bias`` (broadcastable to
    [B, Hq, Nq, Nkv], -inf removes a key) enters the oracle's attention
    exactly as in the forward; the dK term then takes, for each key, the
    maximum of b_i over the rows of its group that see it."""
    q, k, v, g = dec
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    sc = oracle.scale_value(None, D)
    u = U[dtype]
    o, _ = oracle.attention(q, k, v, sc, causal, causal_offset=causal_offset, bias=bias)
    pk, _ = oracle.attention(q, k, k, sc, causal, causal_offset=causal_offset,
                             bias=bias)                                  # sum_j P_ij K_j
    b = np.sqrt(np.sum((g * o) ** 2, axis=-1, keepdims=True))         # [B,Hq,Nq,1]
    t_dq = 12.0 * sc * u * b * np.abs(pk)
    if bias is not None:
        # rows i of the group that see key j: bias finite (and causal order)
        vis = np.isfinite(np.broadcast_to(bias, (B, Hq, Nq, Nkv)))
        if causal:
            i = np.arange(Nq)[:, None]
            j = np.arange(Nkv)[None, :]
            vis = vis & (j <= i + causal_offset)
        bmax = np.max(np.where(vis, b, 0.0).reshape(B, Hkv, G * Nq, Nkv), axis=2)
        bmax = bmax[..., None]                                           # [B,Hkv,Nkv,1]
    elif causal:   # rows i >= j - offset see key j
        bg = b[..., 0].reshape(B, Hkv, G, Nq).max(axis=2)             # [B,Hkv,Nq]
        suffix = np.maximum.accumulate(bg[:, :, ::-1], axis=-1)[:, :, ::-1]
        bmax = np.zeros((B, Hkv, Nkv))
        for j in range(Nkv):
            i0 = max(0, j - causal_offset)
            if i0 < Nq:
                bmax[:, :, j] = suffix[:, :, i0]
        bmax = bmax[..., None]
    else:
        bg = b[..., 0].reshape(B, Hkv, G, Nq).max(axis=2)
        bmax = bg.max(axis=-1)[:, :, None, None]
    qmax = np.abs(q).reshape(B, Hkv, -1).max(axis=-1)[:, :, None, None]
    rms_dv = np.sqrt(np.mean(ref[2] ** 2, axis=-1, keepdims=True))
    t_dk = 6.0 * sc * u * bmax * qmax * rms_dv
    return t_dq, t_dk, 0.0


def run_case(device, B, Hq, Hkv, Nq, Nkv, D, dtype, causal, seed, Dv=None):
    """``causal``: False, True (top-left) or "bottom_right"; ``Dv``: V's
    head dimension (default D)."""
    import torch
    what = (f"bwd B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nkv={Nkv} D={D} Dv={Dv} {dtype} "
            f"causal={causal} seed={seed}")
    log(what)
    x = inputs.make_inputs(B, Hq, Hkv, Nq, Nkv, D, dtype, seed=seed, Dv=Dv)
    do = inputs.make_dout(x)
    q, k, v, g = (to_device(a, dtype, device) for a in (x.q, x.k, x.v, do))
    out, lse = binding.attn_fwd(q, k, v, causal=causal)
    dq, dk, dv = binding.attn_bwd(q, k, v, out, lse, g, causal=causal)
    torch.cuda.synchronize(device)
    sc = oracle.scale_value(None, D)
    off = Nkv - Nq if causal == "bottom_right" else 0
    ref = oracle.attention_backward(_decode(x.q, dtype), _decode(x.k, dtype),
                                    _decode(x.v, dtype), _decode(do, dtype), sc, bool(causal),
                                    causal_offset=off)
    # keys no query may see: past the last row's reach
    unseen = Nq + off if causal and Nkv > Nq + off else None
    terms = delta_terms(x, do, ref, bool(causal), off)
    if off < 0:   # rows that see no key
        assert torch.all(dq[:, :, :-off] == 0), "dq of rows without keys must be 0"
    for name, got, r, t in zip(("dq", "dk", "dv"), (dq, dk, dv), ref, terms):
        check_grad(name, _host(got), r, dtype, what, None if name == "dq" else unseen, t)


@pytest.mark.parametrize("dtype", [inputs.F16, inputs.BF16])
@pytest.mark.parametrize("causal", [False, True])
def test_mha_d64_ragged(gpu_device, dtype, causal):
    # neither length a multiple of the 64-query, 128-key or 128-row tiles
    run_case(gpu_device, 1, 3, 3, 333, 270, 64, dtype, causal, seed=41)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_d128(gpu_device, causal):
    run_case(gpu_device, 2, 6, 2, 300, 300, 128, inputs.BF16, causal, seed=42)


def test_more_keys_than_queries_causal(gpu_device):
    # keys past the last query row receive exactly zero gradient
    run_case(gpu_device, 1, 2, 1, 130, 600, 64, inputs.F16, True, seed=43)


@pytest.mark.parametrize("D", [128, 64])
def test_more_queries_than_keys(gpu_device, D):
    run_case(gpu_device, 1, 4, 4, 700, 90, D, inputs.F16, True, seed=44)


@pytest.mark.parametrize("D", [128, 64, 96])
@pytest.mark.parametrize("nq,nkv", [(100, 700), (500, 130)])
def test_bottom_right(gpu_device, nq, nkv, D):
    # queries after a cache of keys; more queries than keys (the first rows
    # see no key and get zero gradients); the wave-pair dK/dV kernel (128)
    # and the one-wave kernel (64, 96)
    run_case(gpu_device, 1, 4, 2, nq, nkv, D, inputs.BF16, "bottom_right", seed=nq + D)


@pytest.mark.parametrize("D", [64, 96])
@pytest.mark.parametrize("n", [1, 7, 64, 129])
def test_short_sequences(gpu_device, n, D):
    run_case(gpu_device, 1, 2, 2, n, n, D, inputs.BF16, False, seed=45 + n)


@pytest.mark.parametrize("D,dtype,Nq,bm", [(128, inputs.BF16, 2000, 128),
                                            (64, inputs.F16, 4000, 256)])
def test_dq_last_round_split(gpu_device, D, dtype, Nq, bm):
    """33 heads x 16 query tiles of bm rows (128; 256 at D = 64) = 528 dQ
    workgroups on 512 slots (256 CUs x 2): the 16 tiles of the last, partial
    round are cut into 8 key ranges of 128 keys, whose fp32 partials the
    reduce kernel adds.  Element-wise parity of dQ, dK and dV; the workspace
    pool's peak holds the partials (8 x 16 x bm rows x D fp32) besides Delta
    and the base-2 LSE."""
    import torch
    from tests.parity import PoolPeak
    B, H, Nkv = 1, 33, 1024
    run_case(gpu_device, B, H, H, Nq, Nkv, D, dtype, False, seed=60 + D)
    x = inputs.make_inputs(B, H, H, Nq, Nkv, D, dtype, seed=61)
    do = inputs.make_dout(x)
    q, k, v, g = (to_device(a, dtype, gpu_device) for a in (x.q, x.k, x.v, do))
    out, lse = binding.attn_fwd(q, k, v)
    binding.attn_bwd(q, k, v, out, lse, g)
    torch.cuda.synchronize(gpu_device)
    pool = PoolPeak(gpu_device.index or 0)
    pool.reset()
    binding.attn_bwd(q, k, v, out, lse, g)
    torch.cuda.synchronize(gpu_device)
    rows_bytes = (B * H * Nq * 4 + 255) // 256 * 256
    partials = 8 * 16 * bm * D * 4
    assert pool.read() >= 2 * rows_bytes + partials


def test_long_d128_several_tiles(gpu_device):
    run_case(gpu_device, 1, 4, 4, 1500, 1500, 128, inputs.BF16, False, seed=46)


@pytest.mark.parametrize("D", [128, 64, 96])
def test_deterministic(gpu_device, D):
    # the wave-pair dK/dV kernel (128) and the one-wave kernel (64, 96), both
    # with head-split partials summed by the reduce kernel
    import torch
    x = inputs.make_inputs(1, 4, 2, 500, 500, D, inputs.BF16, seed=47)
    q, k, v, g = (to_device(a, inputs.BF16, gpu_device)
                  for a in (x.q, x.k, x.v, inputs.make_dout(x)))
    out, lse = binding.attn_fwd(q, k, v)
    a = binding.attn_bwd(q, k, v, out, lse, g)
    b = binding.attn_bwd(q, k, v, out, lse, g)
    torch.cuda.synchronize(gpu_device)
    for x1, x2 in zip(a, b):
        assert torch.equal(x1, x2)


def test_sdpa_autograd(gpu_device):
    """sdpa() under autograd: strided (bnhd) inputs, GQA, causal."""
    import torch
    import memory_efficient_tiled_amd as mta
    dtype = inputs.BF16
    x = inputs.make_inputs(1, 4, 2, 200, 200, 64, dtype, seed=48)
    do = inputs.make_dout(x)
    leaves = []
    for a in (x.q, x.k, x.v):
        t = to_device(np.ascontiguousarray(a.transpose(0, 2, 1, 3)), dtype, gpu_device)
        t.requires_grad_(True)
        leaves.append(t)
    q, k, v = (t.transpose(1, 2) for t in leaves)
    o = mta.sdpa(q, k, v, is_causal=True, enable_gqa=True)
    o.backward(to_device(do, dtype, gpu_device))
    torch.cuda.synchronize(gpu_device)
    sc = oracle.scale_value(None, 64)
    ref = oracle.attention_backward(_decode(x.q, dtype), _decode(x.k, dtype),
                                    _decode(x.v, dtype), _decode(do, dtype), sc, True)
    terms = delta_terms(x, do, ref, True)
    for name, leaf, r, t in zip(("dq", "dk", "dv"), leaves, ref, terms):
        got = _host(leaf.grad.transpose(1, 2))
        check_grad(name, got, r, dtype, "sdpa autograd", None, t)


@pytest.mark.parametrize("kind", ["bool", "add"])
@pytest.mark.parametrize("D", [64, 128])
def test_masked_gradients(gpu_device, kind, D):
    """Gradients of a masked forward: a per-head boolean mask (one row left
    with no key) or an additive mask with -inf entries, GQA, ragged sizes."""
    import torch
    dtype = inputs.BF16
    B, Hq, Hkv, Nq, Nkv = 1, 4, 2, 150, 230
    x = inputs.make_inputs(B, Hq, Hkv, Nq, Nkv, D, dtype, seed=D + len(kind))
    do = inputs.make_dout(x)
    rng = np.random.Generator(np.random.PCG64([D, 9]))
    if kind == "bool":
        keep = rng.random((1, Hq, Nq, Nkv)) < 0.7
        keep[0, 1, 5] = False
        mt, bias = torch.from_numpy(keep).to(gpu_device), np.where(keep, 0.0, -np.inf)
    else:
        a = rng.standard_normal((Nq, Nkv)).astype(np.float32)
        a[rng.random((Nq, Nkv)) < 0.2] = -np.inf
        st = inputs.to_storage(a, dtype)
        mt, bias = to_device(st, dtype, gpu_device), _decode(st, dtype)
    q, k, v, g = (to_device(a, dtype, gpu_device) for a in (x.q, x.k, x.v, do))
    out, lse = binding.attn_fwd(q, k, v, mask=mt)
    dq, dk, dv = binding.attn_bwd(q, k, v, out, lse, g, mask=mt)
    torch.cuda.synchronize(gpu_device)
    sc = oracle.scale_value(None, D)
    bias4 = np.broadcast_to(bias, (B, Hq, Nq, Nkv))
    dec = [_decode(a, dtype) for a in (x.q, x.k, x.v, do)]
    ref = oracle.attention_backward(*dec, sc, False, bias=bias4)
    terms = delta_terms_dec(dec, ref, dtype, False, bias=bias4)
    what = f"masked {kind} D={D}"
    for name, got, r, t in zip(("dq", "dk", "dv"), (dq, dk, dv), ref, terms):
        check_grad(name, _host(got), r, dtype, what, None, t)
    if kind == "bool":
        assert torch.all(dq[0, 1, 5] == 0), "a row with no key has no gradient"


@pytest.mark.parametrize("D", [64, 128])
def test_sdpa_masked_autograd(gpu_device, D):
    # a boolean key-padding mask: batch 0 keeps every key (the kernels' paths
    # for tiles that keep all keys), batch 1 drops keys 100..119
    import torch
    import memory_efficient_tiled_amd as mta
    dtype = inputs.F16
    x = inputs.make_inputs(2, 4, 4, 90, 120, D, dtype, seed=61)
    do = inputs.make_dout(x)
    keep = np.ones((2, 1, 1, 120), dtype=bool)
    keep[1, ..., 100:] = False                        # key padding of batch 1
    leaves = [to_device(a, dtype, gpu_device).requires_grad_(True) for a in (x.q, x.k, x.v)]
    o = mta.sdpa(*leaves, attn_mask=torch.from_numpy(keep).to(gpu_device))
    o.backward(to_device(do, dtype, gpu_device))
    torch.cuda.synchronize(gpu_device)
    bias = np.broadcast_to(np.where(keep, 0.0, -np.inf), (2, 4, 90, 120))
    dec = [_decode(a, dtype) for a in (x.q, x.k, x.v, do)]
    ref = oracle.attention_backward(*dec, oracle.scale_value(None, D), False, bias=bias)
    terms = delta_terms_dec(dec, ref, dtype, False, bias=bias)
    for name, leaf, r, t in zip(("dq", "dk", "dv"), leaves, ref, terms):
        check_grad(name, _host(leaf.grad), r, dtype, f"sdpa masked autograd D={D}", None, t)
    assert torch.all(leaves[1].grad[1, :, 100:] == 0) and torch.all(leaves[2].grad[1, :, 100:] == 0)


@pytest.mark.parametrize("D", [80, 96])
@pytest.mark.parametrize("causal", [False, True, "bottom_right"])
def test_head_dims_80_96(gpu_device, D, causal):
    # D = 80 runs the D = 96 kernels with two zero chunks per row
    run_case(gpu_device, 1, 6, 2, 211, 300, D, inputs.BF16 if D == 96 else inputs.F16,
             causal, seed=D + 3)


def test_masked_gradients_d96(gpu_device):
    import torch
    dtype = inputs.F16
    x = inputs.make_inputs(1, 2, 2, 130, 140, 96, dtype, seed=97)
    do = inputs.make_dout(x)
    keep = np.random.Generator(np.random.PCG64(98)).random((130, 140)) < 0.75
    mt = torch.from_numpy(keep).to(gpu_device)
    q, k, v, g = (to_device(a, dtype, gpu_device) for a in (x.q, x.k, x.v, do))
    out, lse = binding.attn_fwd(q, k, v, mask=mt)
    dq, dk, dv = binding.attn_bwd(q, k, v, out, lse, g, mask=mt)
    torch.cuda.synchronize(gpu_device)
    bias = np.broadcast_to(np.where(keep, 0.0, -np.inf), (1, 2, 130, 140))
    dec = [_decode(a, dtype) for a in (x.q, x.k, x.v, do)]
    ref = oracle.attention_backward(*dec, oracle.scale_value(None, 96), False, bias=bias)
    terms = delta_terms_dec(dec, ref, dtype, False, bias=bias)
    for name, got, r, t in zip(("dq", "dk", "dv"), (dq, dk, dv), ref, terms):
        check_grad(name, _host(got), r, dtype, "masked D=96", None, t)


@pytest.mark.parametrize("causal", [False, True])
def test_head_dim_256(gpu_device, causal):
    # 32-row query tiles in the dK/dV kernel, one wave per SIMD in the dQ kernel
    run_case(gpu_device, 1, 4, 2, 200, 260, 256, inputs.BF16, causal, seed=256)


# -- V rows of another width: (D, Dv) = (192, 128) ----------------------------
# 32-row query tiles in the dK/dV kernel (the P wave holds K and accumulates
# dV over 128 columns, the dS wave holds V and accumulates dK over 192), one
# wave per SIMD in the dQ kernel.  GQA 3 (dK/dV over head-split partials)
# and MHA (written directly).

@pytest.mark.parametrize("causal", [False, True, "bottom_right"])
def test_value_width_gqa(gpu_device, causal):
    run_case(gpu_device, 1, 6, 2, 211, 300, 192, inputs.BF16, causal, seed=192, Dv=128)


@pytest.mark.parametrize("dtype", [inputs.F16, inputs.BF16])
def test_value_width_mha(gpu_device, dtype):
    run_case(gpu_device, 2, 2, 2, 300, 170, 192, dtype, True, seed=193, Dv=128)


def test_value_width_masked(gpu_device):
    import torch
    dtype = inputs.BF16
    x = inputs.make_inputs(1, 4, 2, 130, 150, 192, dtype, seed=194, Dv=128)
    do = inputs.make_dout(x)
    keep = np.random.Generator(np.random.PCG64(195)).random((130, 150)) < 0.75
    mt = torch.from_numpy(keep).to(gpu_device)
    q, k, v, g = (to_device(a, dtype, gpu_device) for a in (x.q, x.k, x.v, do))
    out, lse = binding.attn_fwd(q, k, v, mask=mt)
    dq, dk, dv = binding.attn_bwd(q, k, v, out, lse, g, mask=mt)
    torch.cuda.synchronize(gpu_device)
    bias = np.broadcast_to(np.where(keep, 0.0, -np.inf), (1, 4, 130, 150))
    dec = [_decode(a, dtype) for a in (x.q, x.k, x.v, do)]
    ref = oracle.attention_backward(*dec, oracle.scale_value(None, 192), False, bias=bias)
    terms = delta_terms_dec(dec, ref, dtype, False, bias=bias)
    for name, got, r, t in zip(("dq", "dk", "dv"), (dq, dk, dv), ref, terms):
        check_grad(name, _host(got), r, dtype, "masked D=192 Dv=128", None, t)


def test_value_width_sdpa_autograd(gpu_device):
    """sdpa() under autograd with query/key head dim 192 and value 128."""
    import torch
    import memory_efficient_tiled_amd as mta
    dtype = inputs.BF16
    x = inputs.make_inputs(1, 4, 4, 180, 180, 192, dtype, seed=196, Dv=128)
    do = inputs.make_dout(x)
    leaves = [to_device(a, dtype, gpu_device).requires_grad_(True) for a in (x.q, x.k, x.v)]
    o = mta.sdpa(*leaves, is_causal=True)
    assert o.shape == (1, 4, 180, 128)
    o.backward(to_device(do, dtype, gpu_device))
    torch.cuda.synchronize(gpu_device)
    ref = oracle.attention_backward(*(_decode(a, dtype) for a in (x.q, x.k, x.v, do)),
                                    oracle.scale_value(None, 192), True)
    terms = delta_terms(x, do, ref, True)
    for name, leaf, r, t in zip(("dq", "dk", "dv"), leaves, ref, terms):
        check_grad(name, _host(leaf.grad), r, dtype, "sdpa autograd D=192 Dv=128", None, t)


@pytest.mark.parametrize("D", [64, 96, 128])
def test_broadcast_additive_mask_large_bias(gpu_device, D):
    """A [B, 1, 1, Nkv] additive fp16 mask (row stride 0) with values of
    12..20, with Nq not a multiple of the 64- or 32-row query tile.  Rows past Nq
    in the last tile must get P = 0: exp2 of such a bias alone exceeds the
    fp16 range, and inf * 0 would turn into NaN in dV and dK."""
    import torch
    dtype = inputs.F16
    B, Hq, Hkv, Nq, Nkv = 2, 4, 2, 100, 136
    x = inputs.make_inputs(B, Hq, Hkv, Nq, Nkv, D, dtype, seed=300 + D)
    do = inputs.make_dout(x)
    rng = np.random.Generator(np.random.PCG64([D, 301]))
    a = (12.0 + 8.0 * rng.random((B, 1, 1, Nkv))).astype(np.float32)
    a[rng.random((B, 1, 1, Nkv)) < 0.2] = -np.inf
    st = inputs.to_storage(a, dtype)
    mt = to_device(st, dtype, gpu_device)
    q, k, v, g = (to_device(t, dtype, gpu_device) for t in (x.q, x.k, x.v, do))
    out, lse = binding.attn_fwd(q, k, v, mask=mt)
    dq, dk, dv = binding.attn_bwd(q, k, v, out, lse, g, mask=mt)
    torch.cuda.synchronize(gpu_device)
    bias = np.broadcast_to(_decode(st, dtype), (B, Hq, Nq, Nkv))
    dec = [_decode(t, dtype) for t in (x.q, x.k, x.v, do)]
    ref = oracle.attention_backward(*dec, oracle.scale_value(None, D), False, bias=bias)
    terms = delta_terms_dec(dec, ref, dtype, False, bias=bias)
    what = f"broadcast additive mask 12..20 D={D}"
    for name, got, r, t in zip(("dq", "dk", "dv"), (dq, dk, dv), ref, terms):
        check_grad(name, _host(got), r, dtype, what, None, t)


# -- gradients at several thousand tokens: every element of dQ, dK and dV ----

def test_long_d128_4133(gpu_device):
    # bf16 MHA, 33 query tiles of the dK/dV kernel's 128 keys with a ragged tail
    run_case(gpu_device, 1, 3, 3, 4133, 4133, 128, inputs.BF16, False, seed=4133)


def test_long_gqa_causal_4096(gpu_device):
    # the causal GQA 14/2 shape at 4096 tokens (dK/dV over head-split partials)
    run_case(gpu_device, 1, 14, 2, 4096, 4096, 64, inputs.F16, True, seed=4096)
