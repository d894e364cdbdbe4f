"""ctypes binding to libattn.so -- argument marshalling only.

Every step of the attention forward and of its gradients runs in the HIP
library; this module
checks tensor metadata, allocates the outputs with torch (device memory is
torch's), passes raw device pointers and torch's current HIP stream, and turns
non-zero return codes into exceptions.  There is no fallback: if the library
is missing or fails, the call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libattn.so"

ATTN_F16 = 0
ATTN_BF16 = 1

ATTN_MASK_NONE = 0
ATTN_MASK_BOOL = 1
ATTN_MASK_ADD = 2

ATTN_CAUSAL_NONE = 0
ATTN_CAUSAL_TOP_LEFT = 1
ATTN_CAUSAL_BOTTOM_RIGHT = 2

ATTN_OK = 0
ATTN_EINVAL = -1
ATTN_EUNSUPPORTED = -2
ATTN_ENOMEM = -3
ATTN_EHIP = -4
ATTN_ESCRATCH = -5

# bytes of the per-device scratch array of attn_fwd_noalloc
ATTN_NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None


class AttnPlan(ctypes.Structure):
    """struct attn_plan: how the library covers a shape (see attn_fwd_plan)."""
    _fields_ = [("tile_rows", ctypes.c_int),
                ("num_splits", ctypes.c_int),
                ("split_rows", ctypes.c_longlong),
                ("workspace_bytes", ctypes.c_size_t)]


class AttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"attn error {code}: {msg}")
        self.code = code


def lib_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


_INT = ctypes.c_int
_VP = ctypes.c_void_p
_FP = ctypes.POINTER(ctypes.c_float)


def load_library():
    """Load libattn.so (built in-tree next to this file); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    shape_args = [_INT] * 6                    # B, Hq, Hkv, Nq, Nkv, D
    lib.attn_fwd.argtypes = [_VP, _VP, _VP, _VP, _VP] + shape_args + \
        [ctypes.c_float, _INT, _INT, _VP]
    lib.attn_fwd.restype = _INT
    lib.attn_fwd_split.argtypes = [_VP, _VP, _VP, _VP, _VP] + shape_args + \
        [ctypes.c_float, _INT, _INT, _INT, _VP]
    lib.attn_fwd_split.restype = _INT
    lib.attn_fwd_noalloc.argtypes = [_VP, _VP, _VP, _VP, _VP] + shape_args + \
        [ctypes.c_float, _INT, _INT, _INT, _VP]
    lib.attn_fwd_noalloc.restype = _INT
    lib.attn_fwd_check.argtypes = [_VP, _VP, _VP, _VP, _VP] + shape_args + \
        [ctypes.c_float, _INT, _INT]
    lib.attn_fwd_check.restype = _INT
    _LLP = ctypes.POINTER(ctypes.c_longlong)
    lib.attn_fwd_strided.argtypes = [_VP, _VP, _VP, _VP, _VP] + shape_args + \
        [_LLP] * 4 + [ctypes.c_float, _INT, _INT, _INT, _VP]
    lib.attn_fwd_strided.restype = _INT
    lib.attn_fwd_strided_check.argtypes = [_VP, _VP, _VP, _VP, _VP] + shape_args + \
        [_LLP] * 4 + [ctypes.c_float, _INT, _INT]
    lib.attn_fwd_strided_check.restype = _INT
    lib.attn_fwd_masked.argtypes = [_VP, _VP, _VP, _VP, _VP] + shape_args + \
        [_LLP] * 4 + [_VP, _INT, _LLP, ctypes.c_float, _INT, _INT, _INT, _VP]
    lib.attn_fwd_masked.restype = _INT
    lib.attn_fwd_masked_check.argtypes = [_VP, _VP, _VP, _VP, _VP] + shape_args + \
        [_LLP] * 4 + [_VP, _INT, _LLP, ctypes.c_float, _INT, _INT]
    lib.attn_fwd_masked_check.restype = _INT
    shape_dv = shape_args + [_INT]             # ..., D, Dv
    lib.attn_fwd_dv.argtypes = [_VP, _VP, _VP, _VP, _VP] + shape_dv + \
        [_LLP] * 4 + [_VP, _INT, _LLP, ctypes.c_float, _INT, _INT, _INT, _VP]
    lib.attn_fwd_dv.restype = _INT
    lib.attn_fwd_dv_check.argtypes = [_VP, _VP, _VP, _VP, _VP] + shape_dv + \
        [_LLP] * 4 + [_VP, _INT, _LLP, ctypes.c_float, _INT, _INT]
    lib.attn_fwd_dv_check.restype = _INT
    _F = ctypes.c_float
    lib.attn_fwd_fp8.argtypes = [_VP] * 5 + shape_args + [_F, _F, _F, _F, _INT, _INT, _INT, _VP]
    lib.attn_fwd_fp8.restype = _INT
    lib.attn_fwd_fp8_check.argtypes = [_VP] * 5 + shape_args + [_F, _F, _F, _F, _INT, _INT]
    lib.attn_fwd_fp8_check.restype = _INT
    lib.attn_bwd_dv.argtypes = [_VP] * 9 + shape_dv + [_VP, _INT, _LLP, ctypes.c_float,
                                                       _INT, _INT, _VP]
    lib.attn_bwd_dv.restype = _INT
    lib.attn_bwd_dv_check.argtypes = [_VP] * 9 + shape_dv + [_VP, _INT, _LLP,
                                                             ctypes.c_float, _INT, _INT]
    lib.attn_bwd_dv_check.restype = _INT
    lib.attn_fwd_plan.argtypes = shape_args + [_INT, _INT, _INT, _INT,
                                               ctypes.POINTER(AttnPlan)]
    lib.attn_fwd_plan.restype = _INT
    lib.attn_fwd_num_splits.argtypes = shape_args + [_INT, _INT, _INT]
    lib.attn_fwd_num_splits.restype = _INT
    lib.attn_fwd_workspace_bytes.argtypes = [_INT, _INT, _INT, _INT, _INT, _INT]
    lib.attn_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_bwd.argtypes = [_VP] * 9 + shape_args + [ctypes.c_float, _INT, _INT, _VP]
    lib.attn_bwd.restype = _INT
    lib.attn_bwd_check.argtypes = [_VP] * 9 + shape_args + [ctypes.c_float, _INT, _INT]
    lib.attn_bwd_check.restype = _INT
    lib.attn_bwd_masked.argtypes = [_VP] * 9 + shape_args + [_VP, _INT, _LLP, ctypes.c_float,
                                                             _INT, _INT, _VP]
    lib.attn_bwd_masked.restype = _INT
    lib.attn_bwd_masked_check.argtypes = [_VP] * 9 + shape_args + [_VP, _INT, _LLP,
                                                                   ctypes.c_float, _INT, _INT]
    lib.attn_bwd_masked_check.restype = _INT
    lib.ffn_chunked.argtypes = [_VP] * 6 + [_INT] * 6 + [_VP]
    lib.ffn_chunked.restype = _INT
    lib.ffn_chunked_check.argtypes = [_VP] * 6 + [_INT] * 6
    lib.ffn_chunked_check.restype = _INT
    lib.ffn_workspace_bytes.argtypes = [_INT] * 4
    lib.ffn_workspace_bytes.restype = ctypes.c_size_t
    _FP = ctypes.POINTER(ctypes.c_float)
    lib.ffn_verify.argtypes = [_VP] * 5 + [_INT] * 6 + [_FP, _FP, _VP]
    lib.ffn_verify.restype = _INT
    lib.attn_strerror.argtypes = [_INT]
    lib.attn_strerror.restype = ctypes.c_char_p
    lib.attn_last_hip_error.argtypes = []
    lib.attn_last_hip_error.restype = _INT
    lib.attn_workspace_pool.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.attn_workspace_pool.restype = _INT
    _lib = lib
    return lib


def workspace_pool() -> int:
    """attn_workspace_pool: the current device's hipMemPool_t (as an int)
    that serves the library's stream-ordered workspace.  Owned by the
    library; read its attributes or trim it, never destroy it."""
    lib = load_library()
    pool = ctypes.c_void_p()
    rc = lib.attn_workspace_pool(ctypes.byref(pool))
    if rc != ATTN_OK:
        _raise(rc)
    return int(pool.value)


def _raise(code: int):
    lib = load_library()
    msg = lib.attn_strerror(code).decode()
    if code == ATTN_EHIP:
        msg += f" (hipError {lib.attn_last_hip_error()})"
    raise AttnError(code, msg)


def causal_code(causal) -> int:
    """The C ABI's causal mode: False/None -> none, True or "top_left" ->
    keys j <= i, "bottom_right" -> keys j <= i + Nkv - Nq; ints pass through."""
    if causal is None or causal is False:
        return ATTN_CAUSAL_NONE
    if causal is True or causal == "top_left":
        return ATTN_CAUSAL_TOP_LEFT
    if causal == "bottom_right":
        return ATTN_CAUSAL_BOTTOM_RIGHT
    if isinstance(causal, int):
        return causal
    raise ValueError(f"causal must be a bool, 'top_left' or 'bottom_right', got {causal!r}")


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return ATTN_F16
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float16 or bfloat16")


def attn_fwd_check(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, B, Hq, Hkv, Nq, Nkv,
                   D, scale, causal, dtype_code) -> int:
    """Host-only argument validation (no HIP call); returns the error code."""
    return load_library().attn_fwd_check(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr,
                                         B, Hq, Hkv, Nq, Nkv, D, scale,
                                         causal_code(causal), dtype_code)


def attn_fwd_num_splits(B, Hq, Hkv, Nq, Nkv, D, causal, dtype_code,
                        num_cus=256) -> int:
    """The split-KV count the library picks for this shape (host-only)."""
    return load_library().attn_fwd_num_splits(B, Hq, Hkv, Nq, Nkv, D,
                                              causal_code(causal), dtype_code, num_cus)


def attn_fwd_plan(B, Hq, Hkv, Nq, Nkv, D, causal, dtype_code, num_splits=0,
                  num_cus=256) -> AttnPlan:
    """How the library covers this shape: rows per tile, split count, the
    rows merged from split pieces and the workspace bytes (host-only)."""
    plan = AttnPlan()
    rc = load_library().attn_fwd_plan(B, Hq, Hkv, Nq, Nkv, D, causal_code(causal),
                                      dtype_code, num_splits, num_cus,
                                      ctypes.byref(plan))
    if rc != ATTN_OK:
        _raise(rc)
    return plan


def attn_fwd_workspace_bytes(B, Hq, Nq, Nkv, D, causal=False) -> int:
    """Device bytes attn_fwd allocates for this shape on an MI355X (0 when
    nothing is split)."""
    return load_library().attn_fwd_workspace_bytes(B, Hq, Nq, Nkv, D, causal_code(causal))


def strides3(t):
    """ctypes array of the (batch, head, sequence) element strides of a 4-D
    tensor whose last dimension is contiguous."""
    if t.stride(3) != 1:
        raise ValueError("the head dimension (last) must be contiguous")
    return (ctypes.c_longlong * 3)(t.stride(0), t.stride(1), t.stride(2))


def mask_view(mask, B, Hq, Nq, Nkv, dtype):
    """(tensor, mask_type, strides) for attn_fwd_masked: ``mask`` (bool, or
    the inputs' dtype for an additive mask) broadcast to [B, Hq, Nq, Nkv]
    with zero strides where it broadcasts.  Keys must be contiguous with row
    strides a multiple of 4 elements; a mask that is not is copied once
    (its own shape, keys padded to a multiple of 4)."""
    import torch
    if mask.dtype == torch.bool:
        mtype, m = ATTN_MASK_BOOL, mask
    elif mask.dtype == dtype:
        mtype, m = ATTN_MASK_ADD, mask
    else:
        raise TypeError(f"mask dtype {mask.dtype}: expected bool or {dtype}")
    if m.dim() > 4:
        raise ValueError("mask must have at most 4 dimensions")
    while m.dim() < 4:
        m = m.unsqueeze(0)
    if m.shape[-1] == 1:
        m = m.expand(*m.shape[:-1], Nkv)
    for have, want in zip(m.shape, (B, Hq, Nq, Nkv)):
        if have not in (1, want):
            raise ValueError(f"mask of shape {tuple(mask.shape)} does not broadcast to "
                             f"{(B, Hq, Nq, Nkv)}")
    ok = (m.stride(3) == 1 and all(st % 4 == 0 for st in m.stride()[:3])
          and m.data_ptr() % 8 == 0)
    if not ok:
        pad = (Nkv + 3) // 4 * 4
        buf = torch.zeros(*m.shape[:3], pad, dtype=m.dtype, device=m.device)
        buf[..., :Nkv] = m
        m = buf[..., :Nkv]
    m = m.expand(B, Hq, Nq, Nkv)
    if mtype == ATTN_MASK_BOOL:
        m = m.view(torch.uint8)
    strides = (ctypes.c_longlong * 3)(m.stride(0), m.stride(1), m.stride(2))
    return m, mtype, strides


def attn_fwd(q, k, v, causal=False, scale: float | None = None,
             out=None, lse=None, return_lse: bool = True, num_splits: int = 0,
             mask=None):
    """O = softmax(scale * Q K^T [+ mask] [causal mask]) V on the GPU.

    ``causal``: False, True (= "top_left", keys j <= i) or "bottom_right"
    (keys j <= i + Nkv - Nq; rows that see no key give 0 and LSE -inf).
    ``mask``: None, or PyTorch SDPA's attn_mask (bool: True keeps a key;
    the inputs' dtype: added to the scaled scores), broadcastable to
    [B, Hq, Nq, Nkv].

    q: [B, Hq, Nq, D]; k: [B, Hkv, Nkv, D]; v: [B, Hkv, Nkv, Dv] with Dv = D,
    or (D, Dv) = (192, 128); same dtype (float16 or bfloat16), on one HIP
    device, any strides with the last dimension contiguous (e.g. [B, N, H, D]
    storage viewed as [B, H, N, D]).  Returns
    (out, lse) with out [B, Hq, Nq, Dv] (new tensors are contiguous; a given
    ``out`` may be strided) and lse float32 [B, Hq, Nq] (natural log), or
    just out when ``return_lse`` is False.  ``num_splits`` = 0 lets the
    library choose the split-KV count; a positive value forces it.  Runs on
    torch's current stream; no host synchronisation.
    """
    import torch
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a HIP device, got {t.device}")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, H, N, D]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on one device")
    B, Hq, Nq, D = q.shape
    Bk, Hkv, Nkv, Dk = k.shape
    Dv = v.shape[3]
    if tuple(v.shape[:3]) != tuple(k.shape[:3]) or Bk != B or Dk != D:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} "
                         f"v{tuple(v.shape)}")
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, Nq, Dv), dtype=q.dtype, device=q.device)
    elif tuple(out.shape) != (B, Hq, Nq, Dv) or out.dtype != q.dtype or out.device != q.device:
        raise ValueError("out must be [B, Hq, Nq, Dv] with the dtype and device of q")
    if return_lse:
        if lse is None:
            lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
        elif (tuple(lse.shape) != (B, Hq, Nq) or lse.dtype != torch.float32
              or not lse.is_contiguous() or lse.device != q.device):
            raise ValueError("lse must be a contiguous float32 [B, Hq, Nq] tensor on q's device")
    lse_ptr = lse.data_ptr() if return_lse else None
    qs, ks, vs, os_ = strides3(q), strides3(k), strides3(v), strides3(out)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if Dv != D:
            m, mtype, ms = None, ATTN_MASK_NONE, None
            if mask is not None:
                if mask.device != q.device:
                    raise ValueError("mask must be on q's device")
                m, mtype, ms = mask_view(mask, B, Hq, Nq, Nkv, q.dtype)
            rc = lib.attn_fwd_dv(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                 out.data_ptr(), lse_ptr, B, Hq, Hkv, Nq, Nkv, D, Dv,
                                 qs, ks, vs, os_, None if m is None else m.data_ptr(),
                                 mtype, ms, float(scale), causal_code(causal), dt,
                                 int(num_splits), stream)
        elif mask is None:
            rc = lib.attn_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                      out.data_ptr(), lse_ptr, B, Hq, Hkv, Nq, Nkv, D,
                                      qs, ks, vs, os_, float(scale), causal_code(causal), dt,
                                      int(num_splits), stream)
        else:
            if mask.device != q.device:
                raise ValueError("mask must be on q's device")
            m, mtype, ms = mask_view(mask, B, Hq, Nq, Nkv, q.dtype)
            rc = lib.attn_fwd_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                     out.data_ptr(), lse_ptr, B, Hq, Hkv, Nq, Nkv, D,
                                     qs, ks, vs, os_, m.data_ptr(), mtype, ms, float(scale),
                                     causal_code(causal), dt, int(num_splits), stream)
    if rc != ATTN_OK:
        _raise(rc)
    return (out, lse) if return_lse else out


def attn_fwd_noalloc(q, k, v, out, lse=None, causal=False, scale: float | None = None,
                     num_splits: int = 0):
    """attn_fwd on contiguous [B, H, N, D] tensors into the caller's ``out``
    (and ``lse`` float32 [B, Hq, Nq], or None) without any device
    allocation: the library's split-KV partials live in its per-device
    scratch array (ATTN_NOALLOC_SCRATCH_BYTES); a plan that needs more
    raises AttnError with code ATTN_ESCRATCH before anything runs.  Calls
    that may overlap on one GPU race on that array.  Runs on torch's
    current stream.
    """
    import torch
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dim() != 4:
            raise ValueError(f"{name} must be a 4-D tensor on a HIP device")
        if not t.is_contiguous() or t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must be contiguous, with q's dtype and device")
    B, Hq, Nq, D = q.shape
    _, Hkv, Nkv, _ = k.shape
    if tuple(k.shape) != (B, Hkv, Nkv, D) or tuple(v.shape) != tuple(k.shape) or \
            tuple(out.shape) != tuple(q.shape):
        raise ValueError("shapes must be q, out [B, Hq, Nq, D] and k, v [B, Hkv, Nkv, D]")
    if lse is not None and (tuple(lse.shape) != (B, Hq, Nq) or lse.dtype != torch.float32
                            or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [B, Hq, Nq] tensor on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = lib.attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  None if lse is None else lse.data_ptr(), B, Hq, Hkv, Nq,
                                  Nkv, D, float(scale), causal_code(causal), _dtype_code(q),
                                  int(num_splits), stream)
    if rc != ATTN_OK:
        _raise(rc)
    return out


def attn_fwd_fp8(q, k, v, q_descale=1.0, k_descale=1.0, v_descale=1.0, causal=False,
                 scale: float | None = None, out_dtype=None, out=None, lse=None,
                 return_lse: bool = True, num_splits: int = 0):
    """O = softmax(scale * Q K^T [causal]) V on 8-bit inputs.

    q, k, v: contiguous torch.float8_e4m3fn (or uint8 holding E4M3 bytes)
    tensors [B, Hq, Nq, 128] and [B, Hkv, Nkv, 128] on one HIP device, whose
    values are the stored numbers times q_descale, k_descale, v_descale.
    Returns (out, lse): out [B, Hq, Nq, 128] in ``out_dtype`` (torch.bfloat16
    by default, or torch.float16), lse float32 [B, Hq, Nq].  ``causal`` and
    ``num_splits`` as for attn_fwd.  Runs on torch's current stream.
    """
    import torch
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype not in (torch.float8_e4m3fn, torch.uint8):
            raise TypeError(f"{name} must be float8_e4m3fn (or uint8 E4M3 bytes)")
        if t.device.type != "cuda" or t.device != q.device:
            raise ValueError(f"{name} must be on q's HIP device")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D [B, H, N, D] tensor")
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Nkv, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} "
                         f"v{tuple(v.shape)}")
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    codes = {torch.bfloat16: ATTN_BF16, torch.float16: ATTN_F16}
    if out_dtype not in codes:
        raise TypeError("out_dtype must be torch.bfloat16 or torch.float16")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, Nq, D), dtype=out_dtype, device=q.device)
    elif (tuple(out.shape) != (B, Hq, Nq, D) or out.dtype != out_dtype
          or not out.is_contiguous() or out.device != q.device):
        raise ValueError("out must be a contiguous [B, Hq, Nq, D] tensor of out_dtype")
    if return_lse:
        if lse is None:
            lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
        elif (tuple(lse.shape) != (B, Hq, Nq) or lse.dtype != torch.float32
              or not lse.is_contiguous() or lse.device != q.device):
            raise ValueError("lse must be a contiguous float32 [B, Hq, Nq] tensor on q's device")
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = lib.attn_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              lse.data_ptr() if return_lse else None, B, Hq, Hkv, Nq, Nkv, D,
                              float(q_descale), float(k_descale), float(v_descale),
                              float(scale), causal_code(causal), codes[out_dtype],
                              int(num_splits), stream)
    if rc != ATTN_OK:
        _raise(rc)
    return (out, lse) if return_lse else out


def attn_bwd_check(q_ptr, k_ptr, v_ptr, out_ptr, dout_ptr, lse_ptr, dq_ptr, dk_ptr,
                   dv_ptr, B, Hq, Hkv, Nq, Nkv, D, scale, causal, dtype_code) -> int:
    """Host-only validation of attn_bwd's arguments; returns the error code."""
    return load_library().attn_bwd_check(q_ptr, k_ptr, v_ptr, out_ptr, dout_ptr, lse_ptr,
                                         dq_ptr, dk_ptr, dv_ptr, B, Hq, Hkv, Nq, Nkv, D,
                                         scale, causal_code(causal), dtype_code)


def attn_bwd(q, k, v, out, lse, dout, causal=False, scale: float | None = None,
             dq=None, dk=None, dv=None, mask=None):
    """(dq, dk, dv): gradients of attn_fwd's output with respect to q, k, v.

    q, k, v, out, lse are the forward's inputs and outputs (same scale and
    causal flag, and ``mask`` if it had one), dout the gradient at out.  Every tensor must be contiguous
    ([B, H, N, D]; v, out, dout and dv with V's head dimension Dv, which is
    D or, for D = 192, 128; lse float32 [B, Hq, Nq]) and on one HIP device;
    dq, dk, dv are allocated unless given.  Runs on torch's current stream.
    """
    import torch
    lib = load_library()
    named = (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout), ("lse", lse))
    for name, t in named:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device != q.device or t.device.type != "cuda":
            raise ValueError(f"{name} must be on q's HIP device")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dim() != 4:
        raise ValueError("q must be 4-D [B, H, N, D]")
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    Dv = v.shape[3] if v.dim() == 4 else -1
    if tuple(k.shape) != (B, Hkv, Nkv, D) or tuple(v.shape) != (B, Hkv, Nkv, Dv):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} "
                         f"v{tuple(v.shape)}")
    for name, t in (("out", out), ("dout", dout)):
        if tuple(t.shape) != (B, Hq, Nq, Dv) or t.dtype != q.dtype:
            raise ValueError(f"{name} must be [B, Hq, Nq, Dv] with q's dtype")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    if tuple(lse.shape) != (B, Hq, Nq) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, Hq, Nq]")
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    grads = []
    for name, g, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if g is None:
            g = torch.empty_like(like, memory_format=torch.contiguous_format)
        elif (tuple(g.shape) != tuple(like.shape) or g.dtype != like.dtype
              or g.device != like.device or not g.is_contiguous()):
            raise ValueError(f"{name} must be contiguous with the shape and dtype of "
                             f"its input")
        grads.append(g)
    dq, dk, dv = grads
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if Dv != D:
            m, mtype, ms = None, ATTN_MASK_NONE, None
            if mask is not None:
                if mask.device != q.device:
                    raise ValueError("mask must be on q's device")
                m, mtype, ms = mask_view(mask, B, Hq, Nq, Nkv, q.dtype)
            rc = lib.attn_bwd_dv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                 dv.data_ptr(), B, Hq, Hkv, Nq, Nkv, D, Dv,
                                 None if m is None else m.data_ptr(), mtype, ms, float(scale),
                                 causal_code(causal), dt, stream)
        elif mask is None:
            rc = lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                              dv.data_ptr(), B, Hq, Hkv, Nq, Nkv, D, float(scale),
                              causal_code(causal), dt, stream)
        else:
            if mask.device != q.device:
                raise ValueError("mask must be on q's device")
            m, mtype, ms = mask_view(mask, B, Hq, Nq, Nkv, q.dtype)
            rc = lib.attn_bwd_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                     dout.data_ptr(), lse.data_ptr(), dq.data_ptr(),
                                     dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Nq, Nkv, D,
                                     m.data_ptr(), mtype, ms, float(scale), causal_code(causal),
                                     dt, stream)
    if rc != ATTN_OK:
        _raise(rc)
    return dq, dk, dv


FFN_GELU_TANH = 0


def ffn_chunked(x, w1, b1, w2, b2, chunk_rows: int = 0, out=None, verify: bool = False):
    """y = W2 gelu(W1 x + b1) + b2 (GELU, tanh approximation) over chunks of
    ``chunk_rows`` token rows (0 = the library's choice), on the GPU.

    x [..., Dm], w1 [F, Dm], b1 [F] or None, w2 [Dm, F], b2 [Dm] or None:
    contiguous float16 or bfloat16 tensors of one dtype on one HIP device,
    Dm and F multiples of 8.  Returns y of x's shape (or fills ``out``).
    With ``verify`` the library first runs its chunking check (ffn_verify)
    and this raises if the chunked rows differ from the single-chunk rows by
    more than 2^-6 of the largest output (rounding of the products moves
    them far less), or if either evaluation holds a NaN or infinity.  Runs on torch's current stream.
    """
    import torch
    lib = load_library()
    for name, t in (("x", x), ("w1", w1), ("w2", w2), ("b1", b1), ("b2", b2)):
        if t is None and name in ("b1", "b2"):
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda" or t.device != x.device or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor on x's HIP device")
        if t.dtype != x.dtype:
            raise TypeError(f"{name} must have x's dtype")
    Dm = x.shape[-1]
    N = x.numel() // Dm if Dm else 0
    F = w1.shape[0]
    if tuple(w1.shape) != (F, Dm) or tuple(w2.shape) != (Dm, F):
        raise ValueError(f"weights must be w1 [F, Dm], w2 [Dm, F]; got {tuple(w1.shape)}, "
                         f"{tuple(w2.shape)}")
    if (b1 is not None and tuple(b1.shape) != (F,)) or (b2 is not None and
                                                        tuple(b2.shape) != (Dm,)):
        raise ValueError("biases must be b1 [F], b2 [Dm]")
    dt = _dtype_code(x)
    if out is None:
        out = torch.empty_like(x)
    elif tuple(out.shape) != tuple(x.shape) or out.dtype != x.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of x's shape and dtype")
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        if verify:
            d, r = ctypes.c_float(), ctypes.c_float()
            rc = lib.ffn_verify(x.data_ptr(), w1.data_ptr(), ptr(b1), w2.data_ptr(), ptr(b2),
                                N, Dm, F, FFN_GELU_TANH, int(chunk_rows), dt,
                                ctypes.byref(d), ctypes.byref(r), stream)
            if rc != ATTN_OK:
                _raise(rc)
            # non-finite outputs come back as +inf and fail here
            if not (math.isfinite(d.value) and math.isfinite(r.value)
                    and d.value <= 2.0 ** -6 * max(r.value, 1e-30)):
                raise RuntimeError(f"ffn chunking check failed: chunked rows differ by "
                                   f"{d.value} (largest output {r.value})")
        rc = lib.ffn_chunked(x.data_ptr(), w1.data_ptr(), ptr(b1), w2.data_ptr(), ptr(b2),
                             out.data_ptr(), N, Dm, F, FFN_GELU_TANH, int(chunk_rows), dt, stream)
    if rc != ATTN_OK:
        _raise(rc)
    return out
