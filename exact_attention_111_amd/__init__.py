"""exact_attention_111_amd — exact scaled-dot-product attention for AMD MI355X (gfx950).

FlashAttention-style prefill (``fwd``), its gradients (``bwd``) and split-K decode (``decode``) run in
hand-written HIP kernels behind the C ABI of ``libfa.so`` (``include/fa.h``); this
package only marshals arguments to it.
"""
from .binding import (FaError, bwd, bwd_workspace_bytes, decode, decode_workspace_bytes, fwd, lib,  # noqa: F401
                      status_string)

__all__ = ["fwd", "bwd", "bwd_workspace_bytes", "decode", "decode_workspace_bytes", "FaError", "lib", "status_string"]
