"""exact_attention_111_amd — exact scaled-dot-product attention for AMD MI355X (gfx950).

FlashAttention-style prefill (``fwd``), its gradients (``bwd``) and split-K decode (``decode``, and
``decode_paged`` for a paged KV cache) run in
hand-written HIP kernels behind the C ABI of ``libfa.so`` (``include/fa.h``); this
package only marshals arguments to it.
"""
from .binding import (FaError, bwd, bwd_workspace_bytes, decode, decode_noalloc, decode_paged,  # noqa: F401
                      decode_workspace_bytes,
                      fwd, fwd_fp8, lib, status_string)

__all__ = ["fwd", "fwd_fp8", "bwd", "bwd_workspace_bytes", "decode", "decode_noalloc", "decode_paged", "decode_workspace_bytes", "FaError", "lib",
           "status_string"]
