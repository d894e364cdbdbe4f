"""MI355X-native memory-efficient (tiled, online-softmax) attention: forward
and gradients.

The compute path is the HIP library ``libattn.so`` (built from ``csrc/``);
this package only marshals arguments to its C entry points.
"""
from .binding import (attn_bwd, attn_bwd_check, attn_fwd, attn_fwd_check, attn_fwd_fp8,
                      attn_fwd_noalloc, attn_fwd_num_splits, ffn_chunked,
                      attn_fwd_plan, attn_fwd_workspace_bytes, lib_path, workspace_pool,
                      load_library, AttnError, AttnPlan)
from .frontend import (auto_patch, available, efficient_backend_available, patch, sdpa,
                       stats as sdpa_stats, torch_ops, unpatch, unsupported_reason)

__all__ = ["attn_bwd", "attn_bwd_check", "attn_fwd", "attn_fwd_check", "attn_fwd_fp8",
           "attn_fwd_noalloc", "attn_fwd_num_splits", "ffn_chunked",
           "attn_fwd_plan", "attn_fwd_workspace_bytes", "lib_path", "workspace_pool",
           "load_library", "AttnError", "AttnPlan", "sdpa", "patch", "unpatch",
           "sdpa_stats", "unsupported_reason", "available", "torch_ops", "auto_patch",
           "efficient_backend_available"]
