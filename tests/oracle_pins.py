"""Pins for the CPU oracle: facts fixed by mathematics, not by the oracle.

Every pin takes an ``attn(q, k, v, scale, causal, rows=None) -> (o, lse)``
callable (float64 arrays, q [B,Hq,Nq,D], k/v [B,Hkv,Nkv,D]) and raises
AssertionError when the callable disagrees.  ``test_oracle.py`` runs them on
the oracle; its mutation test runs them on copies of the oracle with a
planted mistake and requires each mistake to be caught.
"""
from __future__ import annotations

import json
import math
import warnings
import os
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")
TOL = 1e-12


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.max(np.abs(a - b) / np.maximum(1.0, np.abs(b))) if a.size else 0.0
    assert err <= tol, f"{what}: max rel err {err:.3e} > {tol:.1e}"


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _dyadic(rng, shape, denom=8, lim=16):
    """Small random multiples of 1/denom: exact in binary floating point."""
    return rng.integers(-lim, lim + 1, size=shape).astype(np.float64) / denom


# ---------------------------------------------------------------------------
# 1. High-precision brute force (exact rational scores, 40-digit exp/log).
# ---------------------------------------------------------------------------

def _bruteforce(q, k, v, scale, causal):
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    o = np.zeros((B, Hq, Nq, D))
    lse = np.zeros((B, Hq, Nq))
    sc = Fraction(scale)
    with localcontext() as ctx:
        ctx.prec = 40
        for b in range(B):
            for h in range(Hq):
                kh = h // G
                for i in range(Nq):
                    keys = [j for j in range(Nkv) if (not causal) or j <= i]
                    ex = []
                    for j in keys:
                        s = sc * sum(Fraction(float(q[b, h, i, d])) *
                                     Fraction(float(k[b, kh, j, d])) for d in range(D))
                        ex.append((Decimal(s.numerator) / Decimal(s.denominator)).exp())
                    total = sum(ex, Decimal(0))
                    lse[b, h, i] = float(total.ln())
                    for d in range(D):
                        acc = sum((e * Decimal(float(v[b, kh, j, d]))
                                   for e, j in zip(ex, keys)), Decimal(0))
                        o[b, h, i, d] = float(acc / total)
    return o, lse


def pin_bruteforce(attn):
    cases = [
        # B, Hq, Hkv, Nq, Nkv, D, causal, scale
        (1, 1, 1, 1, 1, 1, False, 0.5),
        (1, 2, 1, 5, 6, 3, False, 0.7),
        (1, 2, 1, 5, 6, 3, True, 0.7),
        (2, 3, 3, 4, 4, 2, True, 1.25),
        (1, 4, 2, 7, 3, 2, True, 0.375),
        (1, 2, 2, 3, 8, 4, False, 2.0),
    ]
    rng = _rng(11)
    for B, Hq, Hkv, Nq, Nkv, D, causal, scale in cases:
        q = _dyadic(rng, (B, Hq, Nq, D))
        k = _dyadic(rng, (B, Hkv, Nkv, D))
        v = _dyadic(rng, (B, Hkv, Nkv, D))
        o_ref, l_ref = _bruteforce(q, k, v, scale, causal)
        o, l = attn(q, k, v, scale, causal)
        _close(o, o_ref, what=f"bruteforce o {B,Hq,Hkv,Nq,Nkv,D,causal}")
        _close(l, l_ref, what=f"bruteforce lse {B,Hq,Hkv,Nq,Nkv,D,causal}")


# ---------------------------------------------------------------------------
# 2. An independent library implementation (PyTorch's CPU SDPA, float64).
# ---------------------------------------------------------------------------

def pin_torch_sdpa(attn):
    import torch
    import torch.nn.functional as F
    rng = _rng(12)
    cases = [
        (1, 4, 4, 33, 33, 16, False),
        (2, 6, 2, 40, 40, 8, True),
        (1, 7, 1, 17, 29, 8, True),     # Nq < Nkv, top-left causal
        (1, 4, 2, 29, 17, 8, True),     # Nq > Nkv
        (1, 2, 1, 9, 70, 32, False),
    ]
    for B, Hq, Hkv, Nq, Nkv, D, causal in cases:
        q = rng.standard_normal((B, Hq, Nq, D))
        k = rng.standard_normal((B, Hkv, Nkv, D))
        v = rng.standard_normal((B, Hkv, Nkv, D))
        scale = 1.0 / math.sqrt(D)
        ref = F.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            is_causal=causal, scale=scale, enable_gqa=(Hq != Hkv)).numpy()
        o, _ = attn(q, k, v, scale, causal)
        _close(o, ref, tol=1e-11, what=f"torch sdpa {B,Hq,Hkv,Nq,Nkv,D,causal}")


# ---------------------------------------------------------------------------
# 3. Hand-derived worked examples (tests/golden).
# ---------------------------------------------------------------------------

def _eval_expr(expr):
    return float(eval(expr, {"__builtins__": {}},
                      {"e": math.e, "log": math.log, "exp": math.exp}))


def pin_golden(attn):
    with open(GOLDEN) as f:
        data = json.load(f)
    for case in data["cases"]:
        q = np.array(case["q"], dtype=np.float64)[None, None]
        k = np.array(case["k"], dtype=np.float64)[None, None]
        v = np.array(case["v"], dtype=np.float64)[None, None]
        o, lse = attn(q, k, v, case["scale"], case["causal"])
        eo = np.array([[_eval_expr(x) for x in row] for row in case["expected_o"]])
        el = np.array([_eval_expr(x) for x in case["expected_lse"]])
        _close(o[0, 0], eo, what=f"golden {case['name']} o")
        _close(lse[0, 0], el, what=f"golden {case['name']} lse")


# ---------------------------------------------------------------------------
# 4. Closed forms and special cases.
# ---------------------------------------------------------------------------

def pin_q_zero(attn):
    """Q = 0: every allowed key has the same score, so o is the mean of the
    allowed V rows and lse = ln(number of allowed keys)."""
    rng = _rng(13)
    for causal in (False, True):
        B, Hq, Hkv, Nq, Nkv, D = 1, 4, 2, 12, 10, 8
        q = np.zeros((B, Hq, Nq, D))
        k = rng.standard_normal((B, Hkv, Nkv, D))
        v = rng.standard_normal((B, Hkv, Nkv, D))
        o, lse = attn(q, k, v, 0.3, causal)
        for h in range(Hq):
            kh = h // (Hq // Hkv)
            for i in range(Nq):
                n = min(i + 1, Nkv) if causal else Nkv
                _close(o[0, h, i], v[0, kh, :n].mean(axis=0), what="q=0 o")
                _close(lse[0, h, i], math.log(n), what="q=0 lse")


def pin_v_const(attn):
    rng = _rng(14)
    for causal in (False, True):
        B, Hq, Hkv, Nq, Nkv, D = 2, 3, 1, 9, 9, 5
        q = rng.standard_normal((B, Hq, Nq, D)) * 3
        k = rng.standard_normal((B, Hkv, Nkv, D)) * 3
        c = rng.standard_normal(D)
        v = np.broadcast_to(c, (B, Hkv, Nkv, D)).copy()
        o, _ = attn(q, k, v, 0.5, causal)
        _close(o, np.broadcast_to(c, o.shape), what="v const")


def pin_causal_row0(attn):
    """Causal row 0 sees key 0 only: o_0 = v_0, lse_0 = scale*q_0.k_0."""
    rng = _rng(15)
    B, Hq, Hkv, N, D = 2, 4, 2, 6, 4
    q = rng.standard_normal((B, Hq, N, D))
    k = rng.standard_normal((B, Hkv, N, D))
    v = rng.standard_normal((B, Hkv, N, D))
    o, lse = attn(q, k, v, 0.9, True)
    for b in range(B):
        for h in range(Hq):
            kh = h // 2
            _close(o[b, h, 0], v[b, kh, 0], what="causal row 0 o")
            _close(lse[b, h, 0], 0.9 * float(q[b, h, 0] @ k[b, kh, 0]),
                   what="causal row 0 lse")


def pin_single_key(attn):
    rng = _rng(16)
    q = rng.standard_normal((1, 2, 5, 3))
    k = rng.standard_normal((1, 2, 1, 3))
    v = rng.standard_normal((1, 2, 1, 3))
    o, lse = attn(q, k, v, 0.8, False)
    for h in range(2):
        _close(o[0, h], np.broadcast_to(v[0, h, 0], (5, 3)), what="Nkv=1 o")
        _close(lse[0, h], 0.8 * (q[0, h] @ k[0, h, 0]), what="Nkv=1 lse")


def pin_dominant_key(attn):
    """q_i = k_j* = a*u with a large: softmax mass concentrates on j*."""
    rng = _rng(17)
    Nkv, D = 16, 8
    k = rng.standard_normal((1, 1, Nkv, D)) * 0.1
    v = rng.standard_normal((1, 1, Nkv, D))
    u = np.zeros(D)
    u[3] = 1.0
    js = 5
    k[0, 0, js] = 12.0 * u
    q = (12.0 * u)[None, None, None, :]
    o, lse = attn(q, k, v, 1.0, False)
    # every other score is at most 12*max|k_j[3]| < 12*0.5, so the gap is > 70
    _close(o[0, 0, 0], v[0, 0, js], tol=1e-20 + 1e-12, what="dominant key o")
    _close(lse[0, 0, 0], 144.0, what="dominant key lse")


def pin_extreme_scores(attn):
    """Scores spread over thousands of natural-log units (exp of most of them
    over- or underflows float64): softmax is still defined and picks the
    largest, so o_i = v_j* and lse_i = s_ij* to rounding, whichever key
    position holds the maximum (first, middle or last of 40 keys), causal
    or not; only a true row maximum keeps every exponent finite."""
    rng = _rng(18)
    Nkv, D = 40, 4
    v = rng.standard_normal((1, 1, Nkv, D))
    for js in (0, 17, Nkv - 1):
        s = np.linspace(-3000.0, 2000.0, Nkv)          # distinct scores, gaps > 100
        s[[js, Nkv - 1]] = s[[Nkv - 1, js]]             # the maximum at key js
        k = np.zeros((1, 1, Nkv, D))
        k[0, 0, :, 0] = s
        q = np.zeros((1, 1, 1, D))
        q[0, 0, 0, 0] = 1.0
        for causal in (False, True):
            qq = q if not causal else np.repeat(q, Nkv, axis=2)
            o, lse = attn(qq, k, v, 1.0, causal)
            i = Nkv - 1 if causal else 0                 # the last row sees every key
            _close(o[0, 0, i], v[0, 0, js], tol=1e-12, what=f"extreme scores o (j*={js})")
            _close(lse[0, 0, i], 2000.0, tol=1e-12, what=f"extreme scores lse (j*={js})")


# ---------------------------------------------------------------------------
# 5. Invariants.
# ---------------------------------------------------------------------------

def pin_key_shift(attn):
    """K_j += c for every j shifts each score of row i by scale*q_i.c:
    o unchanged, lse_i += scale*q_i.c."""
    rng = _rng(18)
    for causal in (False, True):
        q = rng.standard_normal((1, 2, 7, 6))
        k = rng.standard_normal((1, 2, 9, 6))
        v = rng.standard_normal((1, 2, 9, 6))
        c = rng.standard_normal(6)
        o1, l1 = attn(q, k, v, 0.4, causal)
        o2, l2 = attn(q, k + c, v, 0.4, causal)
        _close(o2, o1, tol=1e-11, what="key shift o")
        _close(l2, l1 + 0.4 * (q @ c), tol=1e-11, what="key shift lse")


def pin_kv_permutation(attn):
    rng = _rng(19)
    q = rng.standard_normal((1, 2, 5, 4))
    k = rng.standard_normal((1, 1, 11, 4))
    v = rng.standard_normal((1, 1, 11, 4))
    p = rng.permutation(11)
    o1, l1 = attn(q, k, v, 0.6, False)
    o2, l2 = attn(q, k[:, :, p], v[:, :, p], 0.6, False)
    _close(o2, o1, tol=1e-11, what="kv permutation o")
    _close(l2, l1, tol=1e-11, what="kv permutation lse")


def pin_query_permutation(attn):
    rng = _rng(20)
    q = rng.standard_normal((1, 3, 8, 4))
    k = rng.standard_normal((1, 3, 6, 4))
    v = rng.standard_normal((1, 3, 6, 4))
    p = rng.permutation(8)
    o1, l1 = attn(q, k, v, 0.6, False)
    o2, l2 = attn(q[:, :, p], k, v, 0.6, False)
    _close(o2, o1[:, :, p], what="query permutation o")
    _close(l2, l1[:, :, p], what="query permutation lse")


def pin_gqa_repeat(attn):
    """GQA equals MHA with each KV head repeated for its G query heads."""
    rng = _rng(21)
    for causal in (False, True):
        B, Hq, Hkv, N, D = 2, 6, 2, 7, 4
        q = rng.standard_normal((B, Hq, N, D))
        k = rng.standard_normal((B, Hkv, N, D))
        v = rng.standard_normal((B, Hkv, N, D))
        G = Hq // Hkv
        o1, l1 = attn(q, k, v, 0.5, causal)
        o2, l2 = attn(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), 0.5, causal)
        _close(o1, o2, what="gqa o")
        _close(l1, l2, what="gqa lse")


def pin_linear_in_v(attn):
    rng = _rng(22)
    q = rng.standard_normal((1, 2, 6, 4))
    k = rng.standard_normal((1, 2, 6, 4))
    v1 = rng.standard_normal((1, 2, 6, 4))
    v2 = rng.standard_normal((1, 2, 6, 4))
    for causal in (False, True):
        oa, _ = attn(q, k, v1, 0.7, causal)
        ob, _ = attn(q, k, v2, 0.7, causal)
        oc, _ = attn(q, k, 2.0 * v1 - 3.0 * v2, 0.7, causal)
        _close(oc, 2.0 * oa - 3.0 * ob, tol=1e-11, what="linearity in v")


def pin_convex_hull(attn):
    rng = _rng(23)
    q = rng.standard_normal((1, 2, 9, 4)) * 2
    k = rng.standard_normal((1, 2, 9, 4)) * 2
    v = rng.standard_normal((1, 2, 9, 4))
    for causal in (False, True):
        o, _ = attn(q, k, v, 1.0, causal)
        for h in range(2):
            for i in range(9):
                n = i + 1 if causal else 9
                lo = v[0, h, :n].min(axis=0) - 1e-12
                hi = v[0, h, :n].max(axis=0) + 1e-12
                assert np.all(o[0, h, i] >= lo) and np.all(o[0, h, i] <= hi), \
                    "convex hull violated"


def pin_rows_subset(attn):
    """Selecting query rows returns exactly those rows of the full result."""
    rng = _rng(24)
    for causal in (False, True):
        q = rng.standard_normal((1, 2, 20, 4))
        k = rng.standard_normal((1, 1, 20, 4))
        v = rng.standard_normal((1, 1, 20, 4))
        rows = np.array([[0, 3, 19], [1, 7, 12]])
        of, lf = attn(q, k, v, 0.5, causal)
        os_, ls = attn(q, k, v, 0.5, causal, rows=rows)
        for h in range(2):
            _close(os_[0, h], of[0, h, rows[h]], what="rows subset o")
            _close(ls[0, h], lf[0, h, rows[h]], what="rows subset lse")


# ---------------------------------------------------------------------------
# 6. Causal alignment with an offset (bottom-right: offset = Nkv - Nq).
# ---------------------------------------------------------------------------

def pin_causal_offset_torch(attn):
    """PyTorch CPU SDPA in float64 with its lower-right causal bias (and an
    explicit boolean tril mask for other offsets) on the rows that see a
    key; rows that see none are o = 0, lse = -inf by definition."""
    import torch
    import torch.nn.functional as F
    from torch.nn.attention.bias import causal_lower_right
    rng = _rng(30)
    for B, Hq, Hkv, Nq, Nkv, D, off in [(1, 4, 2, 17, 29, 8, None), (2, 2, 1, 5, 40, 16, None),
                                       (1, 3, 1, 29, 17, 8, None), (1, 2, 2, 12, 12, 8, 3),
                                       (1, 2, 1, 20, 9, 8, -4)]:
        c = Nkv - Nq if off is None else off
        q = rng.standard_normal((B, Hq, Nq, D))
        k = rng.standard_normal((B, Hkv, Nkv, D))
        v = rng.standard_normal((B, Hkv, Nkv, D))
        scale = 1.0 / math.sqrt(D)
        if off is None:
            mask = causal_lower_right(Nq, Nkv)   # NaN rows when Nq > Nkv: not compared
        else:
            mask = torch.ones(Nq, Nkv, dtype=torch.bool).tril(diagonal=off)
        kt, vt = (torch.from_numpy(np.repeat(a, Hq // Hkv, axis=1)) for a in (k, v))
        with warnings.catch_warnings():
            warnings.simplefilter("ignore", UserWarning)
            ref = F.scaled_dot_product_attention(torch.from_numpy(q), kt, vt, attn_mask=mask,
                                                 scale=scale).numpy()
        o, lse = attn(q, k, v, scale, True, causal_offset=c)
        seen = np.arange(Nq) + c >= 0
        _close(o[:, :, seen], ref[:, :, seen], tol=1e-11,
               what=f"causal offset {c} vs torch {B,Hq,Hkv,Nq,Nkv,D}")
        assert np.all(o[:, :, ~seen] == 0.0), "rows without keys must be 0"
        assert np.all(np.isneginf(lse[:, :, ~seen])), "rows without keys: lse = -inf"
        assert np.all(np.isfinite(lse[:, :, seen]))


def pin_causal_offset_shift(attn):
    """With Nq <= Nkv, bottom-right attention of Q equals the last Nq rows of
    top-left attention of Q placed after Nkv - Nq other query rows."""
    rng = _rng(31)
    for G in (1, 3):
        q = rng.standard_normal((1, 2 * G, 7, 8))
        k = rng.standard_normal((1, 2, 19, 8))
        v = rng.standard_normal((1, 2, 19, 8))
        pad = np.concatenate([rng.standard_normal((1, 2 * G, 12, 8)), q], axis=2)
        o1, l1 = attn(q, k, v, 0.4, True, causal_offset=12)
        o2, l2 = attn(pad, k, v, 0.4, True)
        _close(o1, o2[:, :, 12:], what="offset shift o")
        _close(l1, l2[:, :, 12:], what="offset shift lse")


# ---------------------------------------------------------------------------
# 7. Attention masks (PyTorch SDPA semantics), as an additive bias.
# ---------------------------------------------------------------------------

def pin_mask_torch(attn):
    """PyTorch CPU SDPA in float64 with boolean and float masks of several
    broadcast shapes; rows whose keys are all masked are o = 0, lse = -inf."""
    import torch
    import torch.nn.functional as F
    rng = _rng(32)
    B, Hq, Hkv, Nq, Nkv, D = 2, 4, 2, 13, 21, 8
    q = rng.standard_normal((B, Hq, Nq, D))
    k = rng.standard_normal((B, Hkv, Nkv, D))
    v = rng.standard_normal((B, Hkv, Nkv, D))
    kt, vt = (torch.from_numpy(np.repeat(a, Hq // Hkv, axis=1)) for a in (k, v))
    keep = rng.random((B, 1, Nq, Nkv)) < 0.6
    keep[0, 0, 3] = False                               # a row with no key
    fmask = rng.standard_normal((1, Hq, Nq, Nkv))
    pad = np.ones((B, 1, 1, Nkv), dtype=bool)
    pad[1, 0, 0, 15:] = False                           # key padding of batch 1
    for m in (keep, fmask, pad):
        ref = F.scaled_dot_product_attention(torch.from_numpy(q), kt, vt,
                                             attn_mask=torch.from_numpy(m), scale=0.4).numpy()
        bias = np.where(m, 0.0, -np.inf) if m.dtype == bool else m
        o, lse = attn(q, k, v, 0.4, False, bias=bias)
        empty = np.isneginf(np.broadcast_to(bias, (B, Hq, Nq, Nkv))).all(axis=-1)
        _close(o[~empty], ref[~empty], tol=1e-11, what=f"mask {m.dtype} {m.shape} vs torch")
        assert np.all(o[empty] == 0.0) and np.all(np.isneginf(lse[empty]))


def pin_mask_bias_shift(attn):
    """A bias constant along the keys of a row leaves o unchanged and adds
    to lse; a bias of log(w_j) weights key j like w_j repeated copies."""
    rng = _rng(33)
    q = rng.standard_normal((1, 2, 6, 4))
    k = rng.standard_normal((1, 2, 9, 4))
    v = rng.standard_normal((1, 2, 9, 4))
    c = rng.standard_normal((1, 2, 6, 1))
    o0, l0 = attn(q, k, v, 0.5, False)
    o1, l1 = attn(q, k, v, 0.5, False, bias=np.broadcast_to(c, (1, 2, 6, 9)))
    _close(o1, o0, what="row-constant bias o")
    _close(l1, l0 + c[..., 0], what="row-constant bias lse")
    # key 2 given weight 3 equals key 2 appearing three times
    b = np.zeros((1, 2, 6, 9))
    b[..., 2] = math.log(3.0)
    o2, l2 = attn(q, k, v, 0.5, False, bias=b)
    k3 = np.concatenate([k, k[:, :, 2:3], k[:, :, 2:3]], axis=2)
    v3 = np.concatenate([v, v[:, :, 2:3], v[:, :, 2:3]], axis=2)
    o3, l3 = attn(q, k3, v3, 0.5, False)
    _close(o2, o3, what="log-weight bias o")
    _close(l2, l3, what="log-weight bias lse")


def pin_value_width_torch(attn):
    """V rows of another width than Q and K (Dv != D): PyTorch CPU SDPA in
    float64 (its math path takes such V), non-causal, top-left causal and
    grouped KV heads."""
    import torch
    import torch.nn.functional as F
    rng = _rng(40)
    for B, Hq, Hkv, Nq, Nkv, D, Dv, causal in [(1, 2, 2, 9, 13, 12, 8, False),
                                               (2, 4, 2, 11, 11, 8, 20, True),
                                               (1, 3, 1, 7, 19, 24, 16, True)]:
        q = rng.standard_normal((B, Hq, Nq, D))
        k = rng.standard_normal((B, Hkv, Nkv, D))
        v = rng.standard_normal((B, Hkv, Nkv, Dv))
        scale = 1.0 / math.sqrt(D)
        kt, vt = (torch.from_numpy(np.repeat(a, Hq // Hkv, axis=1)) for a in (k, v))
        ref = F.scaled_dot_product_attention(torch.from_numpy(q), kt, vt, is_causal=causal,
                                             scale=scale).numpy()
        o, lse = attn(q, k, v, scale, causal)
        assert o.shape == (B, Hq, Nq, Dv), f"output shape {o.shape}"
        _close(o, ref, tol=1e-11, what=f"Dv={Dv} vs D={D} against torch")
        _, lse_d = attn(q, k, np.ones((B, Hkv, Nkv, D)), scale, causal)
        _close(lse, lse_d, tol=1e-13, what="lse must not depend on V")


def pin_value_width_columns(attn):
    """Each output column depends on its own V column only: attention with
    V = [V1 V2] is [attention with V1, attention with V2]."""
    rng = _rng(41)
    q = rng.standard_normal((1, 2, 10, 8))
    k = rng.standard_normal((1, 2, 15, 8))
    v = rng.standard_normal((1, 2, 15, 24))
    for causal in (False, True):
        o, lse = attn(q, k, v, 0.4, causal)
        o1, l1 = attn(q, k, v[..., :16], 0.4, causal)
        o2, l2 = attn(q, k, v[..., 16:], 0.4, causal)
        _close(o, np.concatenate([o1, o2], axis=-1), tol=1e-13, what="V column split")
        _close(lse, l1, tol=1e-13, what="lse with part of V")
        _close(lse, l2, tol=1e-13, what="lse with the other part of V")


ALL_PINS = [pin_bruteforce, pin_torch_sdpa, pin_golden, pin_q_zero, pin_v_const,
            pin_causal_row0, pin_single_key, pin_dominant_key, pin_extreme_scores,
            pin_key_shift,
            pin_kv_permutation, pin_query_permutation, pin_gqa_repeat,
            pin_linear_in_v, pin_convex_hull, pin_rows_subset,
            pin_causal_offset_torch, pin_causal_offset_shift, pin_mask_torch,
            pin_mask_bias_shift, pin_value_width_torch, pin_value_width_columns]
