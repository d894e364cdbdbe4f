"""Shared helpers for the GPU parity tests: upload, run, oracle, compare.

Inputs come from the seeded generator; expected values come from the CPU
oracle only.  The GPU result is read back as its exact 16-bit values.
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np

import oracle
from memory_efficient_tiled_amd import attn_fwd, inputs

# Tolerances for the named workloads, on outputs and on the log-sum-exp.
MAX_ERR = 4e-3
MEAN_ERR = 5e-4
LSE_ERR = 1e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(a: np.ndarray, dtype: str, device):
    import torch
    if dtype == inputs.F16:
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device) \
        .view(torch.bfloat16)


def half_ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Half a unit in the last place of the output type at |x|: the error that
    rounding the exact result to the output type alone can cause."""
    mant = 10 if dtype == inputs.F16 else 7
    ax = np.maximum(np.abs(x), 2.0 ** -14)
    return 0.5 * 2.0 ** (np.floor(np.log2(ax)) - mant)


@dataclasses.dataclass
class Result:
    max_err: float
    mean_err: float
    lse_err: float
    n: int


def oracle_rows(x: inputs.Inputs, scale, causal, rows=None, causal_offset=0):
    """Oracle output for all rows, or for rows [Hq, R], one head at a time."""
    B, Hq, Nq, D = x.q.shape
    Hkv, Dv = x.k.shape[1], x.v.shape[3]
    G = Hq // Hkv
    R = Nq if rows is None else rows.shape[1]
    o = np.empty((B, Hq, R, Dv))
    lse = np.empty((B, Hq, R))
    sc = oracle.scale_value(scale, D)
    for b in range(B):
        for hk in range(Hkv):
            kh = oracle.decode(x.k[b:b + 1, hk:hk + 1], x.dtype)
            vh = oracle.decode(x.v[b:b + 1, hk:hk + 1], x.dtype)
            for g in range(G):
                h = hk * G + g
                qh = oracle.decode(x.q[b:b + 1, h:h + 1], x.dtype)
                r = None if rows is None else rows[h]
                oh, lh = oracle.attention(qh, kh, vh, sc, causal, rows=r,
                                          causal_offset=causal_offset)
                o[b, h] = oh[0, 0]
                lse[b, h] = lh[0, 0]
    return o, lse


def run_gpu(x: inputs.Inputs, scale, causal, device, num_splits=0,
            return_lse=True):
    """``causal``: False, True / "top_left" or "bottom_right"."""
    import torch
    q = to_device(x.q, x.dtype, device)
    k = to_device(x.k, x.dtype, device)
    v = to_device(x.v, x.dtype, device)
    res = attn_fwd(q, k, v, causal=causal, scale=scale, num_splits=num_splits,
                   return_lse=return_lse)
    torch.cuda.synchronize(device)
    if return_lse:
        out, lse = res
        return out.float().cpu().numpy().astype(np.float64), \
            lse.cpu().numpy().astype(np.float64)
    return res.float().cpu().numpy().astype(np.float64), None


def compare(o_gpu, l_gpu, o_ref, l_ref, dtype, rounding_allowance=False,
            max_err=MAX_ERR, mean_err=MEAN_ERR, lse_err=LSE_ERR, what="", extra=None):
    """Element-wise comparison against the oracle.

    ``extra`` (an array of o's shape) is added to the element bounds (and
    its mean to the mean bound).  With ``rounding_allowance`` the bounds
    also admit half an ulp of the output type at |ref| (used for edge shapes with few keys, where |o| is
    of order 1 and the output rounding alone can reach 2^-9).
    """
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite outputs"
    err = np.abs(o_gpu - o_ref)
    bound = np.full_like(err, max_err)
    mbound = mean_err
    if rounding_allowance:
        hu = half_ulp(o_ref, dtype)
        bound = bound + hu
        mbound = mean_err + float(hu.mean())
    if extra is not None:       # per-element allowance derived by the caller
        bound = bound + extra
        mbound = mbound + float(np.mean(extra))
    r = Result(float(err.max()), float(err.mean()), 0.0, err.size)
    if l_gpu is not None:
        empty = np.isneginf(l_ref)      # rows that see no key (bottom-right causal)
        bad = empty & ~np.isneginf(l_gpu)
        assert not bad.any(), (f"{what}: lse of key-less rows not -inf at "
                               f"{np.argwhere(bad)[:4].tolist()}: {l_gpu[bad][:4]}")
        assert np.all(np.isfinite(l_gpu[~empty])), f"{what}: non-finite lse"
        r.lse_err = float(np.abs(l_gpu[~empty] - l_ref[~empty]).max()) if (~empty).any() else 0.0
    log(f"  {what}: max|err| {r.max_err:.3e} mean|err| {r.mean_err:.3e} "
        f"lse {r.lse_err:.3e} over {r.n} values")
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), \
        f"{what}: max err {r.max_err:.3e} at {worst} exceeds bound"
    assert r.mean_err <= mbound, f"{what}: mean err {r.mean_err:.3e} > {mbound:.3e}"
    assert r.lse_err <= lse_err, f"{what}: lse err {r.lse_err:.3e} > {lse_err}"
    return r


def gather_rows(a, rows):
    """a [B, Hq, Nq, ...] -> [B, Hq, R, ...] at per-head rows [Hq, R]."""
    B, Hq = a.shape[:2]
    return np.stack([np.stack([a[b, h, rows[h]] for h in range(Hq)])
                     for b in range(B)])


def _e4m3_units(b: np.ndarray) -> np.ndarray:
    """2^e(x) of E4M3 bytes, e the exponent field minus 7 (field 0 counts as
    1); 0 for the two zero patterns."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    e = (b >> 3) & 15
    unit = np.exp2(np.where(e == 0, 1, e) - 7.0)
    return np.where((b & 0x7F) == 0, 0.0, unit)


def fp8_bounds(x: inputs.Inputs, scale, causal, rows=None, causal_offset=0):
    """Per-element error bound of the FP8 forward against the oracle, and a
    per-row LSE bound, on rows [Hq, R] (all rows when None).

    Both products run on the 8-bit matrix instruction, whose accumulation
    tests/test_mma_fp8_gpu.py pins: per instruction, |D - (C + sum_k a_k b_k)|
    <= 7 * 2^-13 sum_g 2^E_g + 2^-19 max(|C|, 2^(max_g E_g + 1)), with eight
    groups of eight products and E_g the largest e(a_k) + e(b_k) of a group
    (e: exponent field minus 7).  Since 2^E_g <= sum over the group of
    2^(e(a_k) + e(b_k)), and |C| <= 4 sum_k 2^(e(a_k) + e(b_k)) for the second
    of the two chained score instructions (D = 128), the raw score error is
    at most 2^-10 U_ij with U_ij = sum_d 2^(e(q_id) + e(k_jd)):
    dS_ij = 2^-10 U_ij scale q_descale k_descale.  It moves o_id by at most
    max_j dS_ij sum_j p_ij (|v_jd| + |o_id|) and the log-sum-exp by
    max_j dS_ij.

    P V: the kernel rounds each probability P_ij (relative to its running
    reference max, so P_ij >= exp(s_ij - max_j s_ij) and the row sum
    l_i >= L_i = sum_j exp(s_ij - max s) >= 1) to E4M3: an error of at most
    2^-4 P_ij (normal numbers, 3 mantissa bits) or 2^-10 (subnormals, below
    2^-6), i.e. 2^-4 p_ij + 2^-10 / L_i on the normalised weight p_ij.  The
    roundings are independent and uniform, so o_id is off by a sum with
    standard deviation sigma_id = sqrt(sum_j (2^-4 p_ij + 2^-10 / L_i)^2
    v_jd^2 / 3), bounded by 6 sigma.  The instruction's own error on
    V^T P^T adds, in normalised units, 2^-10 sum_j max(1.0625 p_ij, 2^-6 / L_i)
    2^e(v_jd) v_descale (2^e of a rounded probability is at most
    1.0625 P_ij, or 2^-6 for a subnormal) plus 2^-19 per key tile on the
    running accumulator, at most 2^-18 n_tiles sum_j p_ij |v_jd|.  The bound
    is the sum of these terms; half an ulp of the output type is added by
    the caller.  Returns (bound [B,Hq,R,D], mean bound [B,Hq,R,D], lse bound
    [B,Hq,R]).
    """
    q8, k8, v8 = x.q, x.k, x.v
    B, Hq, Nq, D = q8.shape
    Hkv, Nkv = k8.shape[1], k8.shape[2]
    G = Hq // Hkv
    sc = oracle.scale_value(scale, D)
    cn = sc * x.q_descale * x.k_descale
    dec = oracle.decode_fp8_e4m3
    n_tiles = (Nkv + 63) // 64 + 1
    R = Nq if rows is None else rows.shape[1]
    bound = np.empty((B, Hq, R, D))
    mbound = np.empty((B, Hq, R, D))
    lbound = np.empty((B, Hq, R))
    keys = np.arange(Nkv)
    for b in range(B):
        for hk in range(Hkv):
            kk = dec(k8[b, hk])
            uk = _e4m3_units(k8[b, hk])
            vv = dec(v8[b, hk]) * x.v_descale
            uv = _e4m3_units(v8[b, hk]) * x.v_descale
            for g in range(G):
                h = hk * G + g
                ri = np.arange(Nq) if rows is None else rows[h]
                qq = dec(q8[b, h, ri])
                s = cn * (qq @ kk.T)
                ds = 2.0 ** -10 * cn * (_e4m3_units(q8[b, h, ri]) @ uk.T)
                if causal:
                    allowed = keys[None, :] <= ri[:, None] + causal_offset
                    s = np.where(allowed, s, -np.inf)
                    ds = np.where(allowed, ds, 0.0)
                mx = s.max(axis=1, keepdims=True)
                empty = ~np.isfinite(mx)
                e = np.exp(s - np.where(empty, 0.0, mx))
                L = np.where(empty, 1.0, e.sum(axis=1, keepdims=True))
                p = e / L
                w = 2.0 ** -4 * p + 2.0 ** -10 / L * (p > 0)
                sigma = np.sqrt((w ** 2) @ (vv ** 2) / 3.0)
                o = p @ vv
                pabs_v = p @ np.abs(vv)
                dsm = ds.max(axis=1, keepdims=True)
                sterm = dsm * (pabs_v + np.abs(o))
                pu = np.where(p > 0, np.maximum(1.0625 * p, 2.0 ** -6 / L), 0.0)
                pvterm = 2.0 ** -10 * (pu @ uv) + 2.0 ** -18 * n_tiles * pabs_v
                bound[b, h] = 6.0 * sigma + sterm + pvterm
                mbound[b, h] = 2.0 * sigma + sterm + pvterm
                lbound[b, h] = dsm[:, 0]
    return bound, mbound, lbound


class PoolPeak:
    """High-water mark of the library's workspace pool on the device
    (attn_workspace_pool), through the HIP runtime this process has already
    loaded."""

    USED_MEM_HIGH = 0x8   # hipMemPoolAttrUsedMemHigh

    def __init__(self, device_index: int = 0):
        import ctypes
        path = next(ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64.so" in ln)
        self.ct = ctypes
        self.hip = ctypes.CDLL(path)
        from memory_efficient_tiled_amd import binding
        import torch
        with torch.cuda.device(device_index):
            self.pool = ctypes.c_void_p(binding.workspace_pool())

    def reset(self):
        zero = self.ct.c_uint64(0)
        assert self.hip.hipMemPoolSetAttribute(self.pool, self.USED_MEM_HIGH,
                                               self.ct.byref(zero)) == 0

    def read(self) -> int:
        v = self.ct.c_uint64(0)
        assert self.hip.hipMemPoolGetAttribute(self.pool, self.USED_MEM_HIGH,
                                               self.ct.byref(v)) == 0
        return int(v.value)
