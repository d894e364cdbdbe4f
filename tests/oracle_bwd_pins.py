"""Pins for the oracle's attention gradients: facts fixed by mathematics.

Every pin takes ``bwd(q, k, v, do, scale, causal, causal_offset=0) -> (dq, dk, dv)`` (float64
arrays, q [B,Hq,Nq,D], k [B,Hkv,Nkv,D], v [B,Hkv,Nkv,Dv], do [B,Hq,Nq,Dv])
and raises AssertionError when
it disagrees.  The strongest is the derivative itself: central finite
differences of the (separately pinned) forward oracle along random
directions.  ``test_oracle.py`` runs them on the oracle and on copies of it
with planted mistakes.
"""
from __future__ import annotations

import numpy as np

import oracle


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _inputs(seed, B=1, Hq=2, Hkv=1, Nq=6, Nkv=7, D=4, Dv=None):
    r = _rng(seed)
    Dv = D if Dv is None else Dv
    return (r.standard_normal((B, Hq, Nq, D)), r.standard_normal((B, Hkv, Nkv, D)),
            r.standard_normal((B, Hkv, Nkv, Dv)), r.standard_normal((B, Hq, Nq, Dv)))


def _close(a, b, tol, what):
    err = float(np.max(np.abs(a - b) / np.maximum(1.0, np.abs(b))))
    assert err <= tol, f"{what}: rel err {err:.3e} > {tol:.1e}"


def pin_finite_differences(bwd):
    """<grad, direction> equals the central difference of L = sum(O * dO)."""
    for seed, causal, Nq, Nkv in ((1, False, 6, 7), (2, True, 7, 7), (3, True, 5, 9)):
        q, k, v, do = _inputs(seed, Nq=Nq, Nkv=Nkv)
        scale = 0.7
        dq, dk, dv = bwd(q, k, v, do, scale, causal)
        r = _rng(100 + seed)
        h = 1e-5
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            d = r.standard_normal(x.shape)
            def loss(xx):
                args = {"q": q, "k": k, "v": v}
                args[name] = xx
                o, _ = oracle.attention(args["q"], args["k"], args["v"], scale, causal)
                return float(np.sum(o * do))
            fd = (loss(x + h * d) - loss(x - h * d)) / (2 * h)
            an = float(np.sum(g * d))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), \
                f"d{name} (causal={causal}): finite difference {fd:.10f} vs {an:.10f}"


def pin_causal_row0_dq(bwd):
    """Causal row 0 sees only key 0 (P = 1), so its dS row is exactly 0."""
    q, k, v, do = _inputs(4, Nq=6, Nkv=6)
    dq, _, _ = bwd(q, k, v, do, 0.5, True)
    assert np.all(dq[:, :, 0] == 0.0), "dq of causal row 0 must vanish"


def pin_zero_do(bwd):
    q, k, v, do = _inputs(5)
    for g in bwd(q, k, v, np.zeros_like(do), 0.5, False):
        assert np.all(g == 0.0), "zero output gradient must give zero gradients"


def pin_column_sums(bwd):
    """Rows of P sum to 1 and rows of dS to 0, so summed over keys
    dv = sum of do over the query rows of the group, and dk sums to 0."""
    for causal in (False, True):
        q, k, v, do = _inputs(6, Hq=4, Hkv=2, Nq=8, Nkv=8)
        _, dk, dv = bwd(q, k, v, do, 0.8, causal)
        G = 2
        for hk in range(2):
            want = do[0, hk * G:(hk + 1) * G].sum(axis=(0, 1))
            _close(dv[0, hk].sum(axis=0), want, 1e-12, f"sum of dv (causal={causal})")
            _close(dk[0, hk].sum(axis=0), np.zeros(4), 1e-12, f"sum of dk (causal={causal})")


def pin_linear_in_do(bwd):
    q, k, v, d1 = _inputs(7)
    d2 = _inputs(8)[3]
    g1, g2, g12 = (bwd(q, k, v, d, 0.5, True) for d in (d1, d2, 2.0 * d1 - 3.0 * d2))
    for a, b, c in zip(g1, g2, g12):
        _close(c, 2.0 * a - 3.0 * b, 1e-12, "linearity in do")


def pin_gqa_repeat(bwd):
    """GQA equals MHA on repeated K/V with the K/V gradients summed back."""
    q, k, v, do = _inputs(9, Hq=6, Hkv=2, Nq=5, Nkv=6)
    dq, dk, dv = bwd(q, k, v, do, 0.6, False)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    dq2, dkr, dvr = bwd(q, kr, vr, do, 0.6, False)
    _close(dq, dq2, 1e-12, "gqa dq")
    _close(dk, dkr.reshape(1, 2, 3, 6, 4).sum(axis=2), 1e-12, "gqa dk")
    _close(dv, dvr.reshape(1, 2, 3, 6, 4).sum(axis=2), 1e-12, "gqa dv")


def pin_finite_differences_offset(bwd):
    """The same derivative check with the causal diagonal moved by an offset:
    bottom-right alignment (Nkv - Nq) with more keys than queries, and with
    more queries than keys, where the first rows see no key at all (their
    output is 0 whatever the inputs, so they contribute no gradient)."""
    for seed, Nq, Nkv in ((11, 5, 9), (12, 9, 5)):
        c = Nkv - Nq
        q, k, v, do = _inputs(seed, Hq=2, Hkv=1, Nq=Nq, Nkv=Nkv)
        scale = 0.6
        dq, dk, dv = bwd(q, k, v, do, scale, True, causal_offset=c)
        r = _rng(200 + seed)
        h = 1e-5
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            d = r.standard_normal(x.shape)
            def loss(xx):
                args = {"q": q, "k": k, "v": v}
                args[name] = xx
                o, _ = oracle.attention(args["q"], args["k"], args["v"], scale, True,
                                        causal_offset=c)
                return float(np.sum(o * do))
            fd = (loss(x + h * d) - loss(x - h * d)) / (2 * h)
            an = float(np.sum(g * d))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), \
                f"d{name} (offset {c}): finite difference {fd:.10f} vs {an:.10f}"
        if c < 0:
            assert np.all(dq[:, :, :-c] == 0.0), "rows without keys have no dq"
        else:
            # the last row sees every key; key c + i is the first that row i sees
            assert np.all(np.isfinite(dk)) and np.any(dk[:, :, -1] != 0.0)


def pin_finite_differences_bias(bwd):
    """The derivative check with an additive mask (finite and -inf entries,
    one row left with no key), against the forward oracle with the same
    bias."""
    q, k, v, do = _inputs(13, Hq=2, Hkv=1, Nq=6, Nkv=8)
    r = _rng(213)
    bias = r.standard_normal((1, 2, 6, 8))
    bias[r.random((1, 2, 6, 8)) < 0.3] = -np.inf
    bias[0, 1, 2] = -np.inf
    scale = 0.5
    dq, dk, dv = bwd(q, k, v, do, scale, False, bias=bias)
    h = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        d = r.standard_normal(x.shape)
        def loss(xx):
            args = {"q": q, "k": k, "v": v}
            args[name] = xx
            o, _ = oracle.attention(args["q"], args["k"], args["v"], scale, False, bias=bias)
            return float(np.sum(o * do))
        fd = (loss(x + h * d) - loss(x - h * d)) / (2 * h)
        an = float(np.sum(g * d))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), \
            f"d{name} (bias): finite difference {fd:.10f} vs {an:.10f}"
    assert np.all(dq[0, 1, 2] == 0.0), "a row with no key has no dq"


def pin_finite_differences_value_width(bwd):
    """V (and so O and dO) wider or narrower than Q and K: central
    differences of the forward oracle, GQA, causal and not, and the column
    sums of dv (sum over keys = sum of dO over the group's query rows)."""
    for seed, causal, D, Dv in ((11, False, 4, 7), (12, True, 6, 3)):
        q, k, v, do = _inputs(seed, Hq=4, Hkv=2, Nq=6, Nkv=8, D=D, Dv=Dv)
        scale = 0.6
        dq, dk, dv = bwd(q, k, v, do, scale, causal)
        assert dq.shape == q.shape and dk.shape == k.shape and dv.shape == v.shape
        r = _rng(200 + seed)
        h = 1e-5
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            d = r.standard_normal(x.shape)
            def loss(xx):
                args = {"q": q, "k": k, "v": v}
                args[name] = xx
                o, _ = oracle.attention(args["q"], args["k"], args["v"], scale, causal)
                return float(np.sum(o * do))
            fd = (loss(x + h * d) - loss(x - h * d)) / (2 * h)
            an = float(np.sum(g * d))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), \
                f"d{name} (D={D}, Dv={Dv}): finite difference {fd:.10f} vs {an:.10f}"
        for hk in range(2):
            _close(dv[0, hk].sum(axis=0), do[0, 2 * hk:2 * hk + 2].sum(axis=(0, 1)), 1e-12,
                   f"sum of dv (D={D}, Dv={Dv})")


ALL_PINS = [pin_finite_differences, pin_causal_row0_dq, pin_zero_do, pin_column_sums,
            pin_linear_in_do, pin_gqa_repeat, pin_finite_differences_offset,
            pin_finite_differences_bias, pin_finite_differences_value_width]
