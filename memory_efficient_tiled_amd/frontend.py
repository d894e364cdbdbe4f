"""PyTorch scaled_dot_product_attention front end for the HIP attention forward.

The English noflash-attention post (section "From gfx906 to a broader
release") ships its method as a replacement for PyTorch's SDPA call: calls
it can serve go to the memory-efficient path, the rest to PyTorch.  Here:

* ``sdpa(query, key, value, ...)`` has SDPA's signature and semantics for
  what this library computes (head dim 64, 80, 96, 128 or 256; no dropout;
  top-left causal through ``is_causal``; PyTorch's causal biases
  ``causal_upper_left`` / ``causal_lower_right`` as ``attn_mask`` (the
  latter is bottom-right alignment, rows that see no key give 0); GQA via
  ``enable_gqa``, default scale 1/sqrt(E)) and raises ``NotImplementedError``
  for anything else (other masks included); inputs may be strided views such as [B, N, H, E]
  storage transposed to [B, H, N, E] (no copy is made).
* ``patch()`` installs it as ``torch.nn.functional.scaled_dot_product_attention``.
  Calls it cannot serve are handed to the original PyTorch function only
  with ``fallback=True`` (the default raises); ``unpatch()`` restores the
  original; ``stats()`` counts the calls each way.
* With autograd on and an input that requires grad, ``sdpa`` keeps the
  forward's log-sum-exp and its backward is the library's gradient kernels
  (``binding.attn_bwd``), which need contiguous tensors: strided inputs are
  copied once, in the backward only.

Only argument checks and marshalling happen here; the computation is the
HIP library's (``binding.attn_fwd`` / ``binding.attn_bwd``), which raises if
it is not built.
"""
from __future__ import annotations

import math

from . import binding

_original = None
_fallback = False
_counts = {"native": 0, "fallback": 0}


def _causal_bias_mode(attn_mask):
    """"top_left" / "bottom_right" for PyTorch's causal bias objects, else None."""
    try:
        from torch.nn.attention.bias import CausalBias, CausalVariant
    except ImportError:
        return None
    if not isinstance(attn_mask, CausalBias):
        return None
    return ("bottom_right" if attn_mask.variant == CausalVariant.LOWER_RIGHT
            else "top_left")


def causal_mode(attn_mask, is_causal):
    """The library's causal mode for an SDPA call it serves."""
    mode = _causal_bias_mode(attn_mask)
    if mode is not None:
        return mode
    return "top_left" if is_causal else False


def unsupported_reason(query, key, value, attn_mask=None, dropout_p=0.0,
                       is_causal=False, scale=None, enable_gqa=False):
    """Why this library cannot serve an SDPA call, or None if it can."""
    import torch
    ts = (query, key, value)
    if not all(isinstance(t, torch.Tensor) for t in ts):
        return "query, key and value must be tensors"
    if attn_mask is not None:
        if _causal_bias_mode(attn_mask) is None:
            return "attn_mask is not supported (only PyTorch's causal biases)"
        if is_causal:
            return "is_causal together with a causal bias"
        if (attn_mask.seq_len_q, attn_mask.seq_len_kv) != (query.shape[-2], key.shape[-2]):
            return "the causal bias's lengths differ from the inputs'"
    if dropout_p != 0.0:
        return "dropout is not supported"
    if not (query.dim() == key.dim() == value.dim()) or query.dim() not in (3, 4):
        return "inputs must all be 3-D [H, N, E] or 4-D [B, H, N, E]"
    if not (query.dtype == key.dtype == value.dtype) or query.dtype not in (
            torch.float16, torch.bfloat16):
        return "dtype must be float16 or bfloat16 for all inputs"
    E = query.shape[-1]
    if E not in (64, 80, 96, 128, 256) or key.shape[-1] != E or value.shape[-1] != E:
        return "head dimension must be 64, 80, 96, 128 or 256 for query, key and value"
    if E not in (64, 128) and torch.is_grad_enabled() and any(t.requires_grad for t in ts):
        return "gradients are built for head dimensions 64 and 128 only"
    if key.shape != value.shape:
        return "key and value must have one shape"
    if query.shape[:-3] != key.shape[:-3]:
        return "batch dimensions differ"
    Hq, Hkv = query.shape[-3], key.shape[-3]
    if Hq != Hkv and (not enable_gqa or Hq % Hkv != 0):
        return "query heads must equal key heads, or be a multiple with enable_gqa"
    if any(t.stride(-1) != 1 for t in ts):
        return "the last dimension must be contiguous"
    if any(s % 8 for t in ts for s in t.stride()[:-1]) or any(
            t.data_ptr() % 16 for t in ts):
        return "strides must be multiples of 8 elements and data 16-byte aligned"
    if any(t.stride(-2) < E or t.stride(-2) > (1 << 24) for t in ts):
        return "sequence strides must lie in [E, 2^24]"
    if query.shape[-2] == 0 or key.shape[-2] == 0 or Hq == 0 or (
            query.dim() == 4 and query.shape[0] == 0):
        return "empty inputs"
    if scale is not None and not math.isfinite(scale):
        return "scale must be finite"
    if any(t.device.type != "cuda" for t in ts) or not (
            query.device == key.device == value.device):
        return "inputs must be on one HIP device"
    return None


def sdpa(query, key, value, attn_mask=None, dropout_p=0.0, is_causal=False,
         scale=None, enable_gqa=False):
    """SDPA on the HIP library: softmax(scale * Q K^T [causal]) V.

    Same arguments as torch.nn.functional.scaled_dot_product_attention;
    returns a new contiguous tensor of the query's shape.  Raises
    NotImplementedError for calls the library cannot serve.
    """
    reason = unsupported_reason(query, key, value, attn_mask, dropout_p,
                                is_causal, scale, enable_gqa)
    if reason is not None:
        raise NotImplementedError(f"memory_efficient_tiled_amd.sdpa: {reason}")
    import torch
    squeeze = query.dim() == 3
    q, k, v = ((t.unsqueeze(0) for t in (query, key, value)) if squeeze
               else (query, key, value))
    mode = causal_mode(attn_mask, is_causal)
    if torch.is_grad_enabled() and any(t.requires_grad for t in (q, k, v)):
        out = _attention_fn().apply(q, k, v, mode, scale)
    else:
        out = binding.attn_fwd(q, k, v, causal=mode, scale=scale, return_lse=False)
    return out.squeeze(0) if squeeze else out


_fn = None


def _attention_fn():
    """torch.autograd.Function over the library's forward and gradients
    (defined on first use so that importing this module needs no torch)."""
    global _fn
    if _fn is not None:
        return _fn
    import torch

    class _Attention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, causal, scale):
            out, lse = binding.attn_fwd(q, k, v, causal=causal, scale=scale)
            ctx.save_for_backward(q, k, v, out, lse)
            ctx.causal, ctx.scale = causal, scale
            return out

        @staticmethod
        def backward(ctx, dout):
            q, k, v, out, lse = ctx.saved_tensors
            q, k, v, dout = (t.contiguous() for t in (q, k, v, dout))
            dq, dk, dv = binding.attn_bwd(q, k, v, out, lse, dout, causal=ctx.causal,
                                          scale=ctx.scale)
            return dq, dk, dv, None, None

    _fn = _Attention
    return _fn


def _patched(query, key, value, attn_mask=None, dropout_p=0.0, is_causal=False,
             scale=None, enable_gqa=False):
    reason = unsupported_reason(query, key, value, attn_mask, dropout_p,
                                is_causal, scale, enable_gqa)
    if reason is None:
        _counts["native"] += 1
        return sdpa(query, key, value, attn_mask, 0.0, is_causal, scale, enable_gqa)
    if not _fallback:
        raise NotImplementedError(f"memory_efficient_tiled_amd.sdpa: {reason}")
    _counts["fallback"] += 1
    kw = {"enable_gqa": enable_gqa} if enable_gqa else {}
    return _original(query, key, value, attn_mask=attn_mask, dropout_p=dropout_p,
                     is_causal=is_causal, scale=scale, **kw)


def patch(fallback: bool = False):
    """Route torch.nn.functional.scaled_dot_product_attention through sdpa().

    The library is loaded first, so a missing build raises here rather than
    silently leaving PyTorch's kernel in place.  With ``fallback`` the calls
    sdpa() cannot serve go to PyTorch's original function; otherwise they
    raise NotImplementedError.
    """
    import torch.nn.functional as F
    global _original, _fallback
    binding.load_library()
    if _original is None:
        _original = F.scaled_dot_product_attention
    _fallback = bool(fallback)
    F.scaled_dot_product_attention = _patched


def unpatch():
    """Restore PyTorch's own scaled_dot_product_attention."""
    import torch.nn.functional as F
    global _original
    if _original is not None:
        F.scaled_dot_product_attention = _original
        _original = None


def stats() -> dict:
    """Calls served by the library ("native") and handed to PyTorch
    ("fallback") since the module was loaded."""
    return dict(_counts)
