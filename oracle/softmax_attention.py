"""CPU oracle for scaled-dot-product attention forward (float64).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the bench's CPU
baseline leg use it.  It shares no code with the HIP library.

What it computes
----------------
The English noflash-attention post (ai-navigate-news.com, section "The DIY
approach") describes its tiled attention as the same mathematics as full
attention: a query chunk's scores against all keys, a softmax over each row,
and a product with V, with the rows of all chunks put together.  Tiling over
keys with a running max and running sum (the post's "online softmax" tier in
the same section) changes the evaluation order only.  The result of the
method is therefore exactly softmax attention, and this oracle is that
definition written out, one query row at a time, in float64:

    s_ij   = scale * <q_i, k_j>                      for j in J_i
    lse_i  = ln sum_{j in J_i} exp(s_ij)             (natural log)
    o_i    = sum_{j in J_i} exp(s_ij - lse_i) * v_j

evaluated with the row maximum subtracted before exponentiating (the
max-subtraction also appears in the chunked snippet of the ai-manual.ru
article, section 3 "Self-written memory-efficient attention").

Readings where the pages are silent (listed again in the design notes):
  * J_i = all keys, or with ``causal`` the keys j <= i (top-left alignment,
    as PyTorch's scaled_dot_product_attention applies is_causal); with a
    ``causal_offset`` c the keys j <= i + c (c = Nkv - Nq is the bottom-right
    alignment of PyTorch's causal_lower_right bias, where the last query
    row sees every key).  A row whose J_i is empty (bottom-right with
    Nq > Nkv) has o_i = 0 and lse_i = -inf: the sum over an empty set;
  * an attention mask follows PyTorch's scaled_dot_product_attention (the
    API the post patches): a float mask is added to the scaled scores, a
    boolean mask keeps the keys where it is True; the oracle takes both as
    an additive ``bias`` (0 / -inf for a boolean mask).  A row whose every
    allowed key has bias -inf is empty as above;
  * query head hq reads KV head hq // (Hq // Hkv): the post's "flattened GQA"
    groups consecutive query heads on one KV head (section "The DIY
    approach");
  * scale defaults to 1/sqrt(D) (the ai-manual.ru snippet divides by
    sqrt(dim)); it is used as the float32 value the GPU receives;
  * V rows may be wider or narrower than Q and K rows (Dv != D): nothing in
    the definition ties them together, each output column is the weighted
    sum of one V column, and PyTorch's SDPA (the API the post patches) takes
    such V.  The pages' own snippet allocates the output like the query
    (ai-manual.ru, section 3), which assumes Dv = D; D alone sets the
    default scale;
  * no epsilon in the denominator (the ai-manual.ru snippet adds 1e-8; after
    max subtraction the row sum is >= 1, so it is left out) and no flush-to-
    zero threshold (the post's fp16 workaround): the oracle is exact.

Rows are processed in groups of query rows purely to bound memory; the
arithmetic of each row is untouched by the grouping.
"""
from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# Decoding the 16-bit inputs exactly into float64.
# ---------------------------------------------------------------------------


def decode_f16(a: np.ndarray) -> np.ndarray:
    """IEEE binary16 values -> float64 (exact)."""
    return np.asarray(a, dtype=np.float16).astype(np.float64)


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64 (exact).

    A bfloat16 is the upper half of an IEEE binary32, so the bits shifted
    left by 16 are the binary32 encoding of the same value.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def decode_fp8_e4m3(bits: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 bit patterns (uint8) -> float64 (exact).

    Sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is
    subnormal (m / 8 * 2^-6); there is no infinity, and the two patterns
    with every exponent and mantissa bit set (0x7f, 0xff) are NaN.  The
    largest finite magnitude is 1.75 * 2^8 = 448.
    """
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return decode_f16(a)
    if dtype == "bf16":
        return decode_bf16(a)
    if dtype == "fp8":
        return decode_fp8_e4m3(a)
    raise ValueError(f"unknown dtype {dtype!r}")


def scale_value(scale: float | None, D: int) -> float:
    """The softmax scale as the float32 the kernel is given, in float64."""
    s = 1.0 / math.sqrt(D) if scale is None else float(scale)
    return float(np.float32(s))


# ---------------------------------------------------------------------------
# The definition.
# ---------------------------------------------------------------------------


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
              causal: bool, rows: np.ndarray | None = None,
              row_group: int = 256,
              causal_offset: int = 0,
              bias: np.ndarray | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Exact softmax attention in float64.

    q: [B, Hq, Nq, D], k: [B, Hkv, Nkv, D], v: [B, Hkv, Nkv, Dv], float64.
    rows: None (all Nq rows) or int array [Hq, R] or [R] of query rows.
    causal_offset: with ``causal``, row i sees keys j <= i + causal_offset.
    bias: None or float64 broadcastable to [B, Hq, Nq, Nkv], added to the
    scaled scores (-inf removes a key).
    Returns (o [B, Hq, R, Dv], lse [B, Hq, R]) in float64, natural log.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Nq, D = q.shape
    Bk, Hkv, Nkv, Dk = k.shape
    Dv = v.shape[3]
    if v.shape[:3] != k.shape[:3] or Bk != B or Dk != D:
        raise ValueError("shape mismatch between q, k and v")
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if rows is None:
        rows_h = np.tile(np.arange(Nq, dtype=np.int64), (Hq, 1))
    else:
        rows = np.asarray(rows, dtype=np.int64)
        rows_h = np.tile(rows, (Hq, 1)) if rows.ndim == 1 else rows
    R = rows_h.shape[1]
    o = np.empty((B, Hq, R, Dv), dtype=np.float64)
    lse = np.empty((B, Hq, R), dtype=np.float64)
    key_idx = np.arange(Nkv, dtype=np.int64)
    if bias is not None:
        bias = np.broadcast_to(np.asarray(bias, dtype=np.float64), (B, Hq, Nq, Nkv))
    for b in range(B):
        for hq in range(Hq):
            hk = hq // G                      # consecutive query heads share a KV head
            kk = k[b, hk]
            vv = v[b, hk]
            for r0 in range(0, R, row_group):
                ri = rows_h[hq, r0:r0 + row_group]
                s = scale * (q[b, hq, ri] @ kk.T)            # [r, Nkv]
                if bias is not None:
                    s = s + bias[b, hq, ri]
                if causal:
                    s = np.where(key_idx[None, :] <= ri[:, None] + causal_offset, s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                empty = ~np.isfinite(m)                        # rows with no allowed key
                m = np.where(empty, 0.0, m)
                e = np.exp(s - m)
                denom = np.where(empty, 1.0, e.sum(axis=1, keepdims=True))
                o[b, hq, r0:r0 + len(ri)] = (e @ vv) / denom
                lse[b, hq, r0:r0 + len(ri)] = np.where(empty, -np.inf, (m + np.log(denom)))[:, 0]
    return o, lse


def attention_two_pass(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                       causal: bool, rows: np.ndarray | None = None,
                       row_block: int = 256, key_block: int = 4096,
                       causal_offset: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """The same definition as :func:`attention`, streamed over key blocks in
    two passes so that no row's full score vector is held: for each block
    of query rows, pass 1 walks the key blocks for the exact row maximum
    m_i; pass 2 walks them again accumulating l_i = sum_j exp(s_ij - m_i)
    and sum_j exp(s_ij - m_i) v_j with m_i fixed; then o_i is the second
    sum over l_i and lse_i = m_i + ln l_i.  This is the plain
    max-subtraction of the definition done block by block (the ai-manual.ru
    article's chunked snippet, section 3, subtracts the maximum the same
    way), deliberately not the running-max rescaling the kernels use.
    Memory is O(row_block * key_block + row_block * Dv); the scores are
    computed twice.  Arguments and results as for :func:`attention`
    (no bias).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    Dv = v.shape[3]
    if v.shape[:3] != k.shape[:3] or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("shape mismatch between q, k and v")
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if rows is None:
        rows_h = np.tile(np.arange(Nq, dtype=np.int64), (Hq, 1))
    else:
        rows = np.asarray(rows, dtype=np.int64)
        rows_h = np.tile(rows, (Hq, 1)) if rows.ndim == 1 else rows
    R = rows_h.shape[1]
    o = np.empty((B, Hq, R, Dv))
    lse = np.empty((B, Hq, R))

    def scores(qr, kk, ri, j0):
        s = scale * (qr @ kk[j0:j0 + key_block].T)
        if causal:
            j = np.arange(j0, j0 + s.shape[1], dtype=np.int64)
            s = np.where(j[None, :] <= ri[:, None] + causal_offset, s, -np.inf)
        return s

    for b in range(B):
        for hq in range(Hq):
            kk = k[b, hq // G]
            vv = v[b, hq // G]
            for r0 in range(0, R, row_block):
                ri = rows_h[hq, r0:r0 + row_block]
                qr = q[b, hq, ri]
                m = np.full(len(ri), -np.inf)
                for j0 in range(0, Nkv, key_block):          # pass 1: the row maxima
                    m = np.maximum(m, scores(qr, kk, ri, j0).max(axis=1))
                empty = ~np.isfinite(m)                        # rows with no allowed key
                mz = np.where(empty, 0.0, m)
                l_sum = np.zeros(len(ri))
                acc = np.zeros((len(ri), Dv))
                for j0 in range(0, Nkv, key_block):          # pass 2: sums against m
                    e = np.exp(scores(qr, kk, ri, j0) - mz[:, None])
                    l_sum += e.sum(axis=1)
                    acc += e @ vv[j0:j0 + key_block]
                den = np.where(empty, 1.0, l_sum)
                o[b, hq, r0:r0 + len(ri)] = acc / den[:, None]
                lse[b, hq, r0:r0 + len(ri)] = np.where(empty, -np.inf, mz + np.log(den))
    return o, lse


def attention_from_storage(q, k, v, dtype: str, scale: float | None,
                           causal: bool, rows=None):
    """Decode 16-bit storage arrays, then evaluate :func:`attention`."""
    D = q.shape[-1]
    return attention(decode(q, dtype), decode(k, dtype), decode(v, dtype),
                     scale_value(scale, D), causal, rows=rows)


def attention_fp8(q8, k8, v8, q_descale: float, k_descale: float, v_descale: float,
                  scale: float, causal: bool, rows=None, causal_offset: int = 0):
    """Attention of FP8 (E4M3) inputs with per-tensor scale factors.

    Reading (the pages are silent on 8-bit inputs): each tensor holds
    x / x_descale rounded to E4M3, so its values are decode(x8) * x_descale;
    the result is :func:`attention` of those values (float64), with the
    softmax scale applied as usual.
    """
    return attention(decode_fp8_e4m3(q8) * q_descale, decode_fp8_e4m3(k8) * k_descale,
                     decode_fp8_e4m3(v8) * v_descale, scale, causal, rows=rows,
                     causal_offset=causal_offset)


# ---------------------------------------------------------------------------
# The gradients.
# ---------------------------------------------------------------------------


def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                       do: np.ndarray, scale: float, causal: bool,
                       row_group: int = 256, causal_offset: int = 0,
                       bias: np.ndarray | None = None):
    """Gradients of softmax attention in float64: (dq, dk, dv).

    For a loss whose gradient with respect to the output is ``do``
    ([B, Hq, Nq, Dv], V's width), the chain rule through the definition above, row by
    row: with P_ij = exp(s_ij - lse_i) over the allowed keys,

        dv_j  += sum_i P_ij do_i                  (dO flows through the sum)
        dP_ij  = <do_i, v_j>
        dS_ij  = P_ij (dP_ij - sum_l P_il dP_il)  (the softmax Jacobian)
        dq_i   = scale * sum_j dS_ij k_j
        dk_j  += scale * sum_i dS_ij q_i

    K/V gradients of a KV head sum over the query heads that read it (the
    GQA grouping of the forward).  Masked keys have P = 0 and get nothing
    from that row; a row with no allowed key (see ``attention``) has o = 0
    whatever the inputs, so all its gradients are 0.  ``bias`` is the
    forward's additive mask (not differentiated).  The post's first tier keeps autograd through its tiled
    forward (section "The DIY approach"); these are the gradients it yields.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Hq, Nq, D = q.shape
    Bk, Hkv, Nkv, Dk = k.shape
    Dv = v.shape[3]
    if (v.shape[:3] != k.shape[:3] or Bk != B or Dk != D
            or do.shape != (B, Hq, Nq, Dv)):
        raise ValueError("shape mismatch between q, k, v and do")
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    key_idx = np.arange(Nkv, dtype=np.int64)
    if bias is not None:
        bias = np.broadcast_to(np.asarray(bias, dtype=np.float64), (B, Hq, Nq, Nkv))
    for b in range(B):
        for hq in range(Hq):
            hk = hq // G
            kk = k[b, hk]
            vv = v[b, hk]
            for r0 in range(0, Nq, row_group):
                ri = np.arange(r0, min(Nq, r0 + row_group), dtype=np.int64)
                s = scale * (q[b, hq, ri] @ kk.T)
                if bias is not None:
                    s = s + bias[b, hq, ri]
                if causal:
                    s = np.where(key_idx[None, :] <= ri[:, None] + causal_offset, s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                m = np.where(np.isfinite(m), m, 0.0)             # rows with no allowed key
                e = np.exp(s - m)
                p = e / np.maximum(e.sum(axis=1, keepdims=True), 1e-300)   # softmax rows
                g = do[b, hq, ri]                                  # dL/dO rows
                dv[b, hk] += p.T @ g
                dp = g @ vv.T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[b, hq, ri] = scale * (ds @ kk)
                dk[b, hk] += scale * (ds.T @ q[b, hq, ri])
    return dq, dk, dv
