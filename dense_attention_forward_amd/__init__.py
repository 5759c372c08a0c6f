"""MI355X (gfx950) dense attention forward: bf16, head_dim 128, non-causal.

``forward(q, k, v, scale=None) -> (o, lse)`` runs the hand-written HIP
kernel through the C ABI of ``include/attn_fwd.h``.
"""
from ._lib import (AttnError, HEAD_DIM, LIB_PATH, attn_fwd_raw, check, default_scale, forward,
                   lib, status_str)

__all__ = ["AttnError", "HEAD_DIM", "LIB_PATH", "attn_fwd_raw", "check", "default_scale",
           "forward", "lib", "status_str"]
