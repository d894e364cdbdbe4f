"""GPU parity of the FP8 (E4M3) forward against the oracle.

Inputs are Gaussian tensors quantised per tensor to E4M3 (inputs.py); the
oracle evaluates exact attention on the decoded values times their descale
factors (oracle.attention_fp8).  The outputs are compared element by
element against the bound derived in tests/parity.py (fp8_bounds: the
rounding of the probabilities to E4M3 for P V, and the accumulation of the
8-bit matrix instruction in both products, pinned on the instruction alone
in tests/test_mma_fp8_gpu.py) plus half an ulp of the output type; the
log-sum-exp within 1e-3 plus the score-error term.
"""
import numpy as np
import pytest

import oracle
from memory_efficient_tiled_amd import inputs
from tests.parity import fp8_bounds, gather_rows, half_ulp, log

pytestmark = pytest.mark.gpu


def _dev(a, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device).view(torch.float8_e4m3fn)


def _check(device, x, causal, what, out_dtype="bf16", scale=None, num_splits=0, rows=None):
    import torch
    from memory_efficient_tiled_amd import attn_fwd_fp8
    od = torch.bfloat16 if out_dtype == "bf16" else torch.float16
    q, k, v = (_dev(a, device) for a in (x.q, x.k, x.v))
    out, lse = attn_fwd_fp8(q, k, v, x.q_descale, x.k_descale, x.v_descale, causal=causal,
                            scale=scale, out_dtype=od, num_splits=num_splits)
    torch.cuda.synchronize(device)
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    B, Hq, Nq, D = x.q.shape
    Nkv = x.k.shape[2]
    off = Nkv - Nq if causal == "bottom_right" else 0
    sc = oracle.scale_value(scale, D)
    r = None if rows is None else x.rows
    o_ref = np.empty((B, Hq, Nq if r is None else r.shape[1], D))
    l_ref = np.empty(o_ref.shape[:3])
    G = Hq // x.k.shape[1]
    for h in range(Hq):   # one head at a time (rows of that head)
        oh, lh = oracle.attention_fp8(x.q[:, h:h + 1], x.k[:, h // G:h // G + 1],
                                      x.v[:, h // G:h // G + 1], x.q_descale, x.k_descale,
                                      x.v_descale, sc, bool(causal),
                                      rows=None if r is None else r[h], causal_offset=off)
        o_ref[:, h], l_ref[:, h] = oh[:, 0], lh[:, 0]
    if r is not None:
        o, l = gather_rows(o, r), gather_rows(l, r)
    bound, mbound, lbound = fp8_bounds(x, scale, bool(causal), rows=r, causal_offset=off)
    hu = half_ulp(o_ref, inputs.BF16 if out_dtype == "bf16" else inputs.F16)
    err = np.abs(o - o_ref)
    empty = np.isneginf(l_ref)
    lerr = np.abs(l[~empty] - l_ref[~empty])
    log(f"  {what}: max|err| {err.max():.3e} mean|err| {err.mean():.3e} (bound mean "
        f"{bound.mean():.3e}, worst err/bound {np.max(err / (bound + hu)):.3f}) lse "
        f"{lerr.max() if lerr.size else 0.0:.3e} rms(o) {np.sqrt(np.mean(o_ref ** 2)):.3e}")
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    assert np.all(err <= bound + hu), f"{what}: error above the bound"
    assert err.mean() <= float(np.mean(mbound + hu)), f"{what}: mean error above the bound"
    assert np.all(np.isneginf(l[empty])), f"{what}: key-less rows need lse -inf"
    assert np.all(lerr <= 1e-3 + lbound[~empty]), f"{what}: lse error"
    return err


@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 63, 65, 1000])
def test_fp8_ragged(gpu_device, n, causal, out_dtype):
    x = inputs.make_inputs(2, 4, 2, n, n, 128, inputs.FP8, seed=800 + n)
    _check(gpu_device, x, causal, f"fp8 N={n} causal={causal} {out_dtype}", out_dtype)


@pytest.mark.parametrize("causal", [False, True, "bottom_right"])
@pytest.mark.parametrize("nq,nkv", [(100, 700), (700, 90), (1, 777)])
def test_fp8_nq_ne_nkv(gpu_device, nq, nkv, causal):
    x = inputs.make_inputs(1, 6, 2, nq, nkv, 128, inputs.FP8, seed=nq + 3 * nkv)
    _check(gpu_device, x, causal, f"fp8 {nq}x{nkv} causal={causal}")


@pytest.mark.parametrize("splits", [2, 5])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_forced_splits(gpu_device, splits, causal):
    x = inputs.make_inputs(1, 3, 1, 200, 1500, 128, inputs.FP8, seed=810 + splits)
    _check(gpu_device, x, causal, f"fp8 splits={splits} causal={causal}", num_splits=splits)


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.3])
def test_fp8_scale_values(gpu_device, scale):
    x = inputs.make_inputs(1, 2, 2, 130, 190, 128, inputs.FP8, seed=820)
    _check(gpu_device, x, True, f"fp8 scale={scale}", scale=scale)


def test_fp8_key_offset_long(gpu_device):
    """A per-channel K offset (the video workload's) over 4100 keys, GQA."""
    x = inputs.make_inputs(1, 8, 2, 300, 4100, 128, inputs.FP8, seed=830, k_offset_std=0.5)
    _check(gpu_device, x, False, "fp8 K offset 4100 keys")


def test_fp8_decode_long_keys(gpu_device):
    # one query row over 65536 keys: split pieces and their merge
    x = inputs.make_inputs(1, 4, 1, 1, 65536, 128, inputs.FP8, seed=840)
    _check(gpu_device, x, False, "fp8 decode 64K keys")


@pytest.mark.parametrize("name", ["dit-17160-fp8", "gqa-causal-fp8-8192"])
def test_fp8_workloads(gpu_device, name):
    w = inputs.WORKLOADS[name]
    x = inputs.make_workload_inputs(w, seed=0, sampled_rows=32)
    _check(gpu_device, x, w.causal, name, rows=32)
