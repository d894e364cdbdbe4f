"""PyTorch scaled_dot_product_attention front end for the HIP attention forward.

The English noflash-attention post (section "From gfx906 to a broader
release") ships its method as a replacement for PyTorch's SDPA call: calls
it can serve go to the memory-efficient path, the rest to PyTorch.  Here:

* ``sdpa(query, key, value, ...)`` has SDPA's signature and semantics for
  what this library computes (head dim 64, 80, 96, 128 or 256, or query and
  key head dim 192 with value head dim 128; no dropout;
  top-left causal through ``is_causal``; PyTorch's causal biases
  ``causal_upper_left`` / ``causal_lower_right`` as ``attn_mask`` (the
  latter is bottom-right alignment, rows that see no key give 0); boolean
  or additive ``attn_mask`` tensors broadcastable to [B, H, L, S] (the mask
  itself gets no gradient); GQA via ``enable_gqa``, default scale
  1/sqrt(E)) and raises ``NotImplementedError`` for anything else; inputs may be strided views such as [B, N, H, E]
  storage transposed to [B, H, N, E] (no copy is made).
* ``patch()`` installs it as ``torch.nn.functional.scaled_dot_product_attention``.
  Calls it cannot serve are handed to the original PyTorch function only
  with ``fallback=True`` (the default raises); ``unpatch()`` restores the
  original; ``stats()`` counts the calls each way.
* ``sdpa`` runs through two torch custom ops (``torch_ops()``):
  ``memory_efficient_tiled_amd::attention`` (O and the log-sum-exp) and
  ``memory_efficient_tiled_amd::attention_backward``, registered with fake
  (shape-only) implementations and autograd, so torch.compile traces the
  call without a graph break and autograd uses the library's gradient
  kernels (``binding.attn_bwd``), which need contiguous tensors: strided
  inputs are copied once, in the backward only.
* ``available()``: the library is built and the device is a gfx950; calls on
  other devices are reported as unsupported.
* ``auto_patch()`` is the start-up rule of the same post's section "From
  gfx906 to a broader release": probe whether PyTorch itself has a fused
  SDPA kernel (flash or memory-efficient) for the device
  (``efficient_backend_available``); if it has, stay out of the way,
  otherwise patch.

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
                       is_causal=False, scale=None, enable_gqa=False, tracing=False):
    """Why this library cannot serve an SDPA call, or None if it can.

    With ``tracing`` (under torch.compile) the checks that need the data
    pointers or the device's properties are left to the library, which
    repeats them when the op runs and raises.
    """
    import torch
    ts = (query, key, value)
    if not all(isinstance(t, torch.Tensor) for t in ts):
        return "query, key and value must be tensors"
    if attn_mask is not None:
        if is_causal:
            return "is_causal together with an attn_mask"
        if _causal_bias_mode(attn_mask) is not None:
            if (attn_mask.seq_len_q, attn_mask.seq_len_kv) != (query.shape[-2], key.shape[-2]):
                return "the causal bias's lengths differ from the inputs'"
        elif isinstance(attn_mask, torch.Tensor):
            if attn_mask.dtype != torch.bool and attn_mask.dtype != query.dtype:
                return "attn_mask must be bool or have the inputs' dtype"
            if attn_mask.dim() > 4:
                return "attn_mask must have at most 4 dimensions"
            full = tuple(query.shape[:-1]) + (key.shape[-2],)
            for have, want in zip(reversed(attn_mask.shape), reversed(full)):
                if have not in (1, want):
                    return "attn_mask does not broadcast to the scores' shape"
            if attn_mask.device != query.device:
                return "attn_mask must be on the inputs' device"
        else:
            return "attn_mask must be a tensor or one of PyTorch's causal biases"
    if dropout_p != 0.0:
        return "dropout is not supported"
    if not (query.dim() == key.dim() == value.dim()) or query.dim() not in (3, 4):
        return "inputs must all be 3-D [H, N, E] or 4-D [B, H, N, E]"
    if not (query.dtype == key.dtype == value.dtype) or query.dtype not in (
            torch.float16, torch.bfloat16):
        return "dtype must be float16 or bfloat16 for all inputs"
    E, Ev = query.shape[-1], value.shape[-1]
    if key.shape[-1] != E or not (
            (Ev == E and E in (64, 80, 96, 128, 256)) or (E, Ev) == (192, 128)):
        return ("head dimension must be 64, 80, 96, 128 or 256 for query, key and value, "
                "or 192 for query and key with 128 for value")
    if key.shape[:-1] != value.shape[:-1]:
        return "key and value must have one shape apart from the head dimension"
    if query.shape[:-3] != key.shape[:-3]:
        return "batch dimensions differ"
    Hq, Hkv = query.shape[-3], key.shape[-3]
    if Hq != Hkv and (not enable_gqa or Hq % Hkv != 0):
        return "query heads must equal key heads, or be a multiple with enable_gqa"
    if any(t.stride(-1) != 1 for t in ts):
        return "the last dimension must be contiguous"
    if any(s % 8 for t in ts for s in t.stride()[:-1]) or (
            not tracing and any(t.data_ptr() % 16 for t in ts)):
        return "strides must be multiples of 8 elements and data 16-byte aligned"
    if any(t.stride(-2) < t.shape[-1] or t.stride(-2) > (1 << 24) for t in ts):
        return "sequence strides must lie in [head dimension, 2^24]"
    if query.shape[-2] == 0 or key.shape[-2] == 0 or Hq == 0 or (
            query.dim() == 4 and query.shape[0] == 0):
        return "empty inputs"
    if scale is not None and not math.isfinite(scale):
        return "scale must be finite"
    if any(t.device.type != "cuda" for t in ts) or not (
            query.device == key.device == value.device):
        return "inputs must be on one HIP device"
    if not tracing and not _device_ok(query.device):
        return "the device is not a gfx950 (MI355X)"
    return None


_arch = {}


def _device_ok(device) -> bool:
    import torch
    idx = device.index if device.index is not None else torch.cuda.current_device()
    if idx not in _arch:
        name = getattr(torch.cuda.get_device_properties(idx), "gcnArchName", "")
        _arch[idx] = name.split(":")[0] == "gfx950"
    return _arch[idx]


def available(device=None) -> bool:
    """True when the HIP library is built and loads and ``device`` (default:
    the current one) is a gfx950 GPU."""
    import torch
    try:
        binding.load_library()
    except Exception:
        return False
    if not torch.cuda.is_available():
        return False
    return _device_ok(torch.device("cuda", device) if isinstance(device, int)
                      else torch.device(device or "cuda"))


def sdpa(query, key, value, attn_mask=None, dropout_p=0.0, is_causal=False,
         scale=None, enable_gqa=False):
    """SDPA on the HIP library: softmax(scale * Q K^T [causal]) V.

    Same arguments as torch.nn.functional.scaled_dot_product_attention;
    returns a new contiguous tensor of the query's shape with the value's
    head dimension.  Raises
    NotImplementedError for calls the library cannot serve.
    """
    import torch
    reason = unsupported_reason(query, key, value, attn_mask, dropout_p, is_causal, scale,
                                enable_gqa, tracing=torch.compiler.is_compiling())
    if reason is not None:
        raise NotImplementedError(f"memory_efficient_tiled_amd.sdpa: {reason}")
    squeeze = query.dim() == 3
    q, k, v = ((t.unsqueeze(0) for t in (query, key, value)) if squeeze
               else (query, key, value))
    code = binding.causal_code(causal_mode(attn_mask, is_causal))
    sc = float(scale) if scale is not None else 1.0 / math.sqrt(q.shape[-1])
    # PyTorch's causal biases are tensor subclasses: they select a causal mode
    mask = (attn_mask if isinstance(attn_mask, torch.Tensor)
            and _causal_bias_mode(attn_mask) is None else None)
    out, _ = torch_ops()[0](q, k, v, mask, code, sc)
    return out.squeeze(0) if squeeze else out


_ops = None


def torch_ops():
    """Register (once) and return the torch custom ops behind ``sdpa``:

    * ``memory_efficient_tiled_amd::attention(q, k, v, mask, causal, scale) -> (out, lse)``
      (``mask`` None or an SDPA attn_mask tensor; ``causal`` the C ABI's
      code: 0 none, 1 top-left, 2 bottom-right);
    * ``memory_efficient_tiled_amd::attention_backward(dout, q, k, v, out, lse,
      mask, causal, scale) -> (dq, dk, dv)``, the first op's autograd formula
      (the log-sum-exp output and the mask are not differentiated).

    Both have fake implementations (output shapes only) for tracing.
    """
    global _ops
    if _ops is not None:
        return _ops
    import torch

    @torch.library.custom_op(
        "memory_efficient_tiled_amd::attention", mutates_args=(),
        schema="(Tensor q, Tensor k, Tensor v, Tensor? mask, int causal, float scale) "
               "-> (Tensor, Tensor)")
    def attention(q, k, v, mask, causal, scale):
        return binding.attn_fwd(q, k, v, causal=causal, scale=scale, mask=mask)

    @attention.register_fake
    def _(q, k, v, mask, causal, scale):
        B, Hq, Nq, _ = q.shape
        return (q.new_empty((B, Hq, Nq, v.shape[-1])),
                q.new_empty((B, Hq, Nq), dtype=torch.float32))

    @torch.library.custom_op(
        "memory_efficient_tiled_amd::attention_backward", mutates_args=(),
        schema="(Tensor dout, Tensor q, Tensor k, Tensor v, Tensor out, Tensor lse, "
               "Tensor? mask, int causal, float scale) -> (Tensor, Tensor, Tensor)")
    def attention_backward(dout, q, k, v, out, lse, mask, causal, scale):
        q, k, v, dout = (t.contiguous() for t in (q, k, v, dout))
        return binding.attn_bwd(q, k, v, out.contiguous(), lse, dout, causal=causal,
                                scale=scale, mask=mask)

    @attention_backward.register_fake
    def _(dout, q, k, v, out, lse, mask, causal, scale):
        return tuple(torch.empty_like(t, memory_format=torch.contiguous_format)
                     for t in (q, k, v))

    def setup_context(ctx, inputs, output):
        q, k, v, mask, causal, scale = inputs
        out, lse = output
        ctx.save_for_backward(q, k, v, out, lse, mask)
        ctx.mark_non_differentiable(lse)
        ctx.causal, ctx.scale = causal, scale

    def backward(ctx, dout, _dlse):
        q, k, v, out, lse, mask = ctx.saved_tensors
        dq, dk, dv = attention_backward(dout, q, k, v, out, lse, mask, ctx.causal, ctx.scale)
        return dq, dk, dv, None, None, None

    attention.register_autograd(backward, setup_context=setup_context)
    _ops = (attention, attention_backward)
    return _ops


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


def efficient_backend_available(device=None) -> bool:
    """Whether PyTorch has a fused SDPA kernel (flash or memory-efficient)
    for ``device`` (default: the current GPU): one small fp16 call to
    PyTorch's own function, restricted to those two backends, which raises
    when neither can run it.  PyTorch's global switches
    (``torch.backends.cuda.enable_flash_sdp`` / ``enable_mem_efficient_sdp``)
    are honoured, so a backend switched off counts as absent."""
    import torch
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    if not torch.cuda.is_available():
        return False
    dev = torch.device("cuda", device) if isinstance(device, int) else \
        torch.device(device or "cuda")
    # sdpa_kernel() enables what it lists, so list only what is switched on
    backends = ([SDPBackend.FLASH_ATTENTION] if torch.backends.cuda.flash_sdp_enabled()
                else []) + ([SDPBackend.EFFICIENT_ATTENTION]
                            if torch.backends.cuda.mem_efficient_sdp_enabled() else [])
    if not backends:
        return False
    fn = _original if _original is not None else F.scaled_dot_product_attention
    q = torch.zeros((1, 2, 16, 64), dtype=torch.float16, device=dev)
    try:
        with sdpa_kernel(backends):
            fn(q, q, q)
    except RuntimeError:
        return False
    return True


def auto_patch(fallback: bool = True, device=None) -> bool:
    """Patch only where PyTorch lacks a fused SDPA kernel.

    At start-up: when PyTorch has a flash or memory-efficient kernel for the
    device, SDPA is left alone; when it has not (only the math path, which
    builds the full score matrix) and this library can run there (a
    gfx950), ``patch(fallback)`` is applied.  Returns whether SDPA is now
    patched.  A missing build raises, as in ``patch``.
    """
    binding.load_library()
    if not available(device):
        return False
    if efficient_backend_available(device):
        return False
    patch(fallback=fallback)
    return True


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
