"""The 8-bit matrix instruction on its own: how it accumulates.

The FP8 forward forms S^T = K Q^T and O^T = V^T P^T with
v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 operands, block scales 2^0).  Its
error bound (tests/parity.py, fp8_bounds) rests on the accumulation property
checked here, one instruction at a time (tests/instr/mma_fp8_probe.hip),
against the exact result: an E4M3 product has at most 8 significant bits
between 2^-18 and 2^17.6, so C plus 64 of them is exact in float64 for
|C| < 2^30.

Property.  Let e(x) be the exponent field of an E4M3 operand minus the bias 7
(field 0, the subnormals, counts as 1), and for products t_k = a_k b_k let
the reduction indices fall into eight groups of eight consecutive ones.  With
E_g the largest e(a_k) + e(b_k) over the nonzero products of group g, the
instruction truncates every product of the group toward zero to a multiple
of 2^(E_g - 13), then adds the group sums to the fp32 accumulator C with an
error of at most 2^-19 max(|C|, 2^(max_g E_g + 1)).  A product with
e(a) + e(b) >= E_g - 7 has at most 6 fraction bits below its exponent and is
a multiple of 2^(E_g - 13) already, so at most seven products of a group
lose anything, each less than 2^(E_g - 13):

  |D - (C + sum_k t_k)| <= 7 * 2^-13 * sum_g 2^(E_g) + 2^-19 max(|C|, 2^(max_g E_g + 1)).

No ISA document for gfx950 is at hand, so the property is a model of the
instruction: the tests below check its parts separately (the grouping, the
truncation width bit for bit, the bound on random, wide-range and
adversarial inputs, and that the width 13 cannot be raised to 14).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import pytest

import oracle
from tests.parity import log

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE = os.path.join(HERE, "instr", "libmma_fp8_probe.so")

DEC = oracle.decode_fp8_e4m3(np.arange(256, dtype=np.uint8))
FINITE = np.array([i for i in range(256) if np.isfinite(DEC[i])], dtype=np.uint8)


def enc(values) -> np.ndarray:
    """E4M3 bytes of values that E4M3 represents exactly (no rounding)."""
    v = np.asarray(values, dtype=np.float64)
    lut = {float(DEC[i]): i for i in range(256) if np.isfinite(DEC[i]) and i != 0x80}
    out = np.vectorize(lambda x: lut[float(x)], otypes=[np.uint8])(v)
    return out.astype(np.uint8)


def round_e4m3(x: np.ndarray) -> np.ndarray:
    """Nearest E4M3 byte (ties to the even mantissa) of |x| <= 448, by search."""
    x = np.asarray(x, dtype=np.float64)
    pos = FINITE[(DEC[FINITE] >= 0) & (FINITE < 0x80)]
    vals = DEC[pos]
    order = np.argsort(vals)
    pos, vals = pos[order], vals[order]
    a = np.abs(x)
    i = np.clip(np.searchsorted(vals, a), 1, len(vals) - 1)
    lo, hi = vals[i - 1], vals[i]
    pick_hi = (a - lo > hi - a) | ((a - lo == hi - a) & (pos[i] % 2 == 0))
    b = np.where(pick_hi, pos[i], pos[i - 1]).astype(np.uint8)
    return np.where((x < 0) & (DEC[b] != 0), b | 0x80, b).astype(np.uint8)


def exp_field(b: np.ndarray) -> np.ndarray:
    e = (b.astype(np.int64) >> 3) & 15
    return np.where(e == 0, 1, e) - 7


def run_probe(device, a: np.ndarray, b: np.ndarray, c: np.ndarray) -> np.ndarray:
    import torch
    if not os.path.exists(PROBE):
        raise RuntimeError(f"{PROBE} is not built (python -m tests.instr.build)")
    lib = ctypes.CDLL(PROBE)
    lib.mma_fp8_probe.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.c_void_p]
    lib.mma_fp8_probe.restype = ctypes.c_int
    n = a.shape[0]
    assert a.shape == (n, 32, 64) and b.shape == (n, 32, 64) and c.shape == (n, 32, 32)
    assert a.dtype == np.uint8 and b.dtype == np.uint8
    ga = torch.from_numpy(np.ascontiguousarray(a)).to(device)
    gb = torch.from_numpy(np.ascontiguousarray(b)).to(device)
    gc = torch.from_numpy(np.ascontiguousarray(c, dtype=np.float32)).to(device)
    gd = torch.empty_like(gc)
    stream = torch.cuda.current_stream(device).cuda_stream
    rc = lib.mma_fp8_probe(ga.data_ptr(), gb.data_ptr(), gc.data_ptr(), gd.data_ptr(), n,
                           ctypes.c_void_p(stream))
    assert rc == 0, f"mma_fp8_probe returned {rc}"
    torch.cuda.synchronize(device)
    return gd.cpu().numpy().astype(np.float64)


def products(a, b):
    """t [n, i, j, k] and e(a) + e(b) (-inf where t = 0)."""
    t = DEC[a][:, :, None, :] * DEC[b][:, None, :, :]
    es = exp_field(a)[:, :, None, :] + exp_field(b)[:, None, :, :]
    return t, np.where(t != 0, es.astype(np.float64), -np.inf)


def exact(a, b, c):
    return c.astype(np.float32).astype(np.float64) + products(a, b)[0].sum(-1)


def group_exponents(es):
    return es.reshape(*es.shape[:-1], 8, 8).max(-1)   # [n, i, j, 8]


def bound(a, b, c, width=13):
    _, es = products(a, b)
    eg = group_exponents(es)
    cc = np.abs(c.astype(np.float32).astype(np.float64))
    return 7.0 * 2.0 ** -width * np.exp2(eg).sum(-1) + \
        2.0 ** -19 * np.maximum(cc, np.exp2(eg.max(-1) + 1))


def truncated_group_sums(a, b, width=13):
    """The model's group sums: products truncated toward zero to 2^(E_g - width)."""
    t, es = products(a, b)
    tg = t.reshape(*t.shape[:-1], 8, 8)
    eg = group_exponents(es)[..., None]
    q = np.where(np.isfinite(eg), np.exp2(np.where(np.isfinite(eg), eg, 0) - width), 1.0)
    return (np.trunc(tg / q) * q).sum(-1)


def ones(n):
    return np.full((n, 32, 64), enc([1.0])[0], np.uint8)


def exact_case(kind: str):
    """Operands (C = 0) of the bit-exact truncation cases."""
    rng = np.random.default_rng({"gaussian": 901, "gaussian-wide": 902, "sparse": 903,
                                 "near-step": 904}[kind])
    n = 48
    if kind.startswith("gaussian"):
        s = 1.0 if kind == "gaussian" else 24.0
        a = round_e4m3(np.clip(rng.standard_normal((n, 32, 64)) * s, -440, 440))
        b = round_e4m3(np.clip(rng.standard_normal((n, 32, 64)) * s, -440, 440))
    elif kind == "sparse":   # two to five nonzero bytes a row, times 1
        a = np.zeros((n, 32, 64), np.uint8)
        for p in range(n):
            for i in range(32):
                ks = rng.choice(64, rng.integers(2, 6), replace=False)
                a[p, i, ks] = FINITE[rng.integers(0, len(FINITE), len(ks))]
        b = ones(n)
    else:   # one large product per row, the rest 2^-9 .. 2^-15 of it
        a = np.zeros((n, 32, 64), np.uint8)
        for p in range(n):
            for i in range(32):
                e = rng.integers(-2, 8)
                a[p, i] = round_e4m3(rng.choice([-1.0, 1.0], 64) *
                                     np.exp2(e - rng.uniform(9, 15, 64)))
                a[p, i, rng.integers(0, 64)] = enc([rng.choice([-1.0, 1.0]) * 2.0 ** e *
                                                    rng.choice([1.0, 1.125, 1.5, 1.875])])[0]
        b = ones(n)
    return a, b


@pytest.mark.gpu
def test_probe_layout_small_integers(gpu_device):
    # integer operands -8..8: every partial sum is exact in any arithmetic
    rng = np.random.default_rng(900)
    ints = enc(np.arange(-8, 9))
    a = ints[rng.integers(0, 17, (16, 32, 64))]
    b = ints[rng.integers(0, 17, (16, 32, 64))]
    c = rng.integers(-1000, 1000, (16, 32, 32)).astype(np.float32)
    d = run_probe(gpu_device, a, b, c)
    assert np.array_equal(d, exact(a, b, c)), "operand or accumulator layout is off"


@pytest.mark.gpu
def test_groups_of_eight(gpu_device):
    # 2^8 at index kb and 2^-6 at kt (times 1): the small product is 2^-14 of
    # the large one, below the truncation step 2^(8 - 13) when the two share
    # a group, and kept exactly otherwise
    pairs = [(kb, kt) for kb in range(64) for kt in range(64) if kb != kt]
    a = np.zeros((len(pairs), 64), np.uint8)
    for r, (kb, kt) in enumerate(pairs):
        a[r, kt] = enc([2.0 ** -6])[0]
        a[r, kb] = enc([256.0])[0]
    n = len(pairs) // 32
    d = run_probe(gpu_device, a.reshape(n, 32, 64), ones(n), np.zeros((n, 32, 32)))
    got = d[:, :, 0].reshape(-1)
    same = np.array([kb // 8 == kt // 8 for kb, kt in pairs])
    want = np.where(same, 256.0, 256.0 + 2.0 ** -6)
    assert np.array_equal(got, want), \
        f"grouping differs at {np.nonzero(got != want)[0][:5]} of {len(pairs)} pairs"


@pytest.mark.gpu
@pytest.mark.parametrize("kind", ["gaussian", "gaussian-wide", "sparse", "near-step"])
def test_truncation_bit_exact(gpu_device, kind):
    """With C = 0, wherever the model's sum is an fp32 number the instruction
    returns exactly that number (so neither a wider nor a narrower step, nor
    rounding instead of truncation, fits)."""
    a, b = exact_case(kind)
    n = a.shape[0]
    d = run_probe(gpu_device, a, b, np.zeros((n, 32, 32)))
    model = truncated_group_sums(a, b).sum(-1)
    rep = model.astype(np.float32).astype(np.float64) == model
    assert rep.mean() > 0.9, f"only {rep.mean():.3f} of the model sums are fp32 numbers"
    mism = rep & (d != model)
    log(f"  {kind}: model exact on {np.mean(d[rep] == model[rep]):.4f} of "
        f"{int(rep.sum())} representable sums; exact sum differs on "
        f"{np.mean(d != exact(a, b, np.zeros((n, 32, 32)))):.3f}")
    assert not mism.any(), f"{int(mism.sum())} results differ from the truncation model"
    for w in (12, 14):   # the neighbouring widths do not fit
        other = truncated_group_sums(a, b, width=w).sum(-1)
        assert np.any(rep & (d != other)), f"width {w} fits as well"


@pytest.mark.gpu
@pytest.mark.parametrize("kind", ["random-bytes", "gaussian", "c-small", "c-large",
                                  "c-huge", "bytes-and-c", "near-step"])
def test_accumulation_bound(gpu_device, kind):
    rng = np.random.default_rng({"random-bytes": 910, "gaussian": 911, "c-small": 912,
                                 "c-large": 913, "c-huge": 914, "bytes-and-c": 915,
                                 "near-step": 916}[kind])
    n = 64
    rnd = lambda: FINITE[rng.integers(0, len(FINITE), (n, 32, 64))]   # noqa: E731
    gau = lambda s=1.0: round_e4m3(np.clip(rng.standard_normal((n, 32, 64)) * s,  # noqa: E731
                                           -440, 440))
    c = np.zeros((n, 32, 32))
    if kind == "random-bytes":
        a, b = rnd(), rnd()
    elif kind == "gaussian":
        a, b = gau(8.0), gau(8.0)
    elif kind.startswith("c-"):
        a, b = gau(), gau()
        c = rng.standard_normal((n, 32, 32)) * {"c-small": 1e-3, "c-large": 8.0,
                                                "c-huge": 1e7}[kind]
    elif kind == "bytes-and-c":
        a, b = rnd(), rnd()
        c = rng.standard_normal((n, 32, 32)) * 1e3
    else:
        a = np.zeros((n, 32, 64), np.uint8)
        for p in range(n):
            for i in range(32):
                e = rng.integers(-2, 8)
                a[p, i] = round_e4m3(rng.choice([-1.0, 1.0], 64) *
                                     np.exp2(e - rng.uniform(7, 14, 64)))
                a[p, i, 8 * np.arange(8) + rng.integers(0, 8, 8)] = enc([2.0 ** e])[0]
        b = ones(n)
    c = c.astype(np.float32)
    d = run_probe(gpu_device, a, b, c)
    err = np.abs(d - exact(a, b, c))
    bd = bound(a, b, c)
    log(f"  {kind}: worst err/bound {np.max(err / bd):.3f}")
    assert np.all(err <= bd), f"{kind}: error above the bound"


@pytest.mark.gpu
def test_truncation_width_is_sharp(gpu_device):
    """Each group: one product 2^8 (mantissas 1) and seven of 1.96875 2^-5
    (mantissas 1.75 and 1.125), all of one sign: each of the seven keeps only
    2^-5 = 2^(8 - 13), so the error is 0.96875 of the bound's group term,
    above what a 14-bit step would allow."""
    rng = np.random.default_rng(905)
    n = 16
    a = np.zeros((n, 32, 64), np.uint8)
    b = np.zeros((n, 32, 64), np.uint8)
    for p in range(n):
        sgn = rng.choice([-1.0, 1.0])   # one sign: the groups' losses add up
        for g in range(8):
            big = 8 * g + rng.integers(0, 8)
            for k in range(8 * g, 8 * g + 8):
                a[p, :, k] = enc([sgn * (2.0 ** 4 if k == big else 1.75 * 2.0 ** -3)])[0]
                b[p, :, k] = enc([2.0 ** 4 if k == big else 1.125 * 2.0 ** -2])[0]
    c = np.zeros((n, 32, 32), np.float32)
    d = run_probe(gpu_device, a, b, c)
    err = np.abs(d - exact(a, b, c))
    assert np.array_equal(d, truncated_group_sums(a, b).sum(-1))
    group_term = 7 * 2.0 ** -13 * 8 * 2.0 ** 8
    frac = err / group_term
    log(f"  sharp: err / group term {frac.min():.4f} .. {frac.max():.4f}")
    assert np.all(err <= bound(a, b, c))
    assert np.all(frac == 0.96875)
    assert np.all(err > bound(a, b, c, width=14)), "a 14-bit step would bound this"


def test_probe_exports():
    """The probe library, when built, exports its one entry point (no GPU call)."""
    if not os.path.exists(PROBE):
        pytest.skip("instruction probe not built")
    lib = ctypes.CDLL(PROBE)
    assert hasattr(lib, "mma_fp8_probe")


def test_bound_helpers_on_the_cpu():
    """The model's helpers agree with hand-computed cases."""
    one, big = enc([1.0])[0], enc([256.0])[0]
    a = np.zeros((1, 32, 64), np.uint8)
    b = np.full((1, 32, 64), one, np.uint8)
    a[0, 0, 0] = big
    a[0, 0, 1] = enc([2.0 ** -6])[0]        # same group: truncated away
    a[0, 0, 9] = enc([2.0 ** -6])[0]        # own group: exact
    s = truncated_group_sums(a, b).sum(-1)
    assert s[0, 0, 0] == 256.0 + 2.0 ** -6
    assert exact(a, b, np.zeros((1, 32, 32)))[0, 0, 0] == 256.0 + 2.0 ** -5
    bd = bound(a, b, np.zeros((1, 32, 32)))
    assert bd[0, 0, 0] == 7 * 2.0 ** -13 * (2.0 ** 8 + 2.0 ** -6) + 2.0 ** -19 * 2.0 ** 9
    # round_e4m3 is nearest-even on exact midpoints and exact on E4M3 values
    assert DEC[round_e4m3(np.array([1.0625]))][0] == 1.0     # between 1 and 1.125
    assert DEC[round_e4m3(np.array([1.1875]))][0] == 1.25    # between 1.125 and 1.25
    assert np.array_equal(round_e4m3(DEC[FINITE]), np.where(FINITE == 0x80, 0, FINITE))
