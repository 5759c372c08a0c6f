"""MI355X (gfx950) dense attention forward: bf16, head_dim 128, non-causal.

``forward(q, k, v, scale=None) -> (o, lse)`` runs the hand-written HIP
kernel through the C ABI of ``include/attn_fwd.h``.
"""
from ._lib import (VARIANT_AUTO, VARIANT_PAIR128, VARIANT_PAIR256, VARIANT_PAIR256_EXP2EMU, VARIANT_TILE128, AttnError, HEAD_DIM, LIB_PATH,
                   attn_fwd_raw, check, default_scale, forward, lib, mfma_rate, pick, status_str)

__all__ = ["VARIANT_AUTO", "VARIANT_PAIR128", "VARIANT_PAIR256", "VARIANT_PAIR256_EXP2EMU", "VARIANT_TILE128", "AttnError", "HEAD_DIM",
           "LIB_PATH", "attn_fwd_raw", "check", "default_scale", "forward", "lib", "mfma_rate",
           "pick", "status_str"]
