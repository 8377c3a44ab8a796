"""MI355X-native Kimi Delta Attention (KDA): chunkwise prefill and fused decode.

The compute path is the C-ABI library ``libkda.so`` (hand-written HIP kernels
for gfx950, declared in ``include/kda.h``).  This package is a thin ctypes
binding over it: torch supplies device memory and streams, every arithmetic
step runs in the library.  There is no CPU fallback; calling into the binding
without a built library or without a GPU raises.
"""
from .kda import (KDAError, ShortConv, abi_version, checkpoint_rows, conv_norm, conv_norm_varlen,
                  decode_step, decode_step_conv, library_path, prefill, prefill_bwd,
                  prefill_bwd_workspace_size, prefill_conv,
                  prefill_conv_workspace_size, prefill_split_workspace_size, prefill_varlen,
                  prefill_workspace_size)

__all__ = ["KDAError", "ShortConv", "abi_version", "checkpoint_rows", "conv_norm",
           "conv_norm_varlen",
           "decode_step", "decode_step_conv", "library_path", "prefill", "prefill_bwd",
           "prefill_bwd_workspace_size", "prefill_conv",
           "prefill_conv_workspace_size", "prefill_split_workspace_size", "prefill_varlen",
           "prefill_workspace_size"]
