"""ctypes binding of the C ABI declared in include/attn_fwd.h.

Argument marshalling only: torch supplies device buffers and the current
stream; every step of the attention forward runs in the HIP library. If
the library is missing the calls raise; there is no other code path.
"""
from __future__ import annotations

import ctypes
import math
import threading
from pathlib import Path

PKG = Path(__file__).resolve().parent
LIB_PATH = PKG / "libattn_fwd.so"

ATTN_OK = 0
STATUS_NAMES = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_ALIGN",
    4: "ATTN_ERR_SCALE", 5: "ATTN_ERR_OVERLAP", 6: "ATTN_ERR_LAUNCH", 7: "ATTN_ERR_VARIANT",
}
VARIANT_AUTO, VARIANT_TILE128, VARIANT_PAIR256, VARIANT_PAIR256_EXP2EMU, VARIANT_PAIR128 = 0, 1, 2, 3, 4
HEAD_DIM = 128

_lock = threading.Lock()
_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libattn_fwd.so (built by dense_attention_forward_amd.build)."""
    global _lib
    with _lock:
        if _lib is None:
            if not LIB_PATH.exists():
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m dense_attention_forward_amd.build`")
            l = ctypes.CDLL(str(LIB_PATH))
            vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
            l.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, vp]
            l.attn_fwd.restype = i
            l.attn_fwd_variant.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
            l.attn_fwd_variant.restype = i
            l.attn_fwd_pick.argtypes = [i, i, i]
            l.attn_fwd_pick.restype = i
            l.attn_fwd_check.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f]
            l.attn_fwd_check.restype = i
            l.attn_status_str.argtypes = [i]
            l.attn_status_str.restype = ctypes.c_char_p
            l.attn_mfma_rate.argtypes = [vp, vp, i, i, vp]
            l.attn_mfma_rate.restype = i
            _lib = l
        return _lib


def status_str(status: int) -> str:
    return lib().attn_status_str(int(status)).decode()


def check(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int,
          B: int, H: int, S: int, D: int, scale: float) -> int:
    """Host-only argument validation (no device access)."""
    return lib().attn_fwd_check(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, S, D, scale)


def attn_fwd_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int,
                 B: int, H: int, S: int, D: int, scale: float, stream: int,
                 variant: int = VARIANT_AUTO) -> int:
    """Direct call of the C entry point with raw device pointers; returns the status."""
    if variant == VARIANT_AUTO:
        return lib().attn_fwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, S, D, scale, stream)
    return lib().attn_fwd_variant(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, S, D, scale, variant,
                                  stream)


def pick(B: int, H: int, S: int) -> int:
    """The kernel variant attn_fwd uses for this shape (host only)."""
    return lib().attn_fwd_pick(B, H, S)


def default_scale(D: int = HEAD_DIM) -> float:
    return 1.0 / math.sqrt(D)


def forward(q, k, v, scale: float | None = None, out=None, lse=None, variant: int = VARIANT_AUTO):
    """Attention forward on [B, H, S, 128] bf16 CUDA/HIP tensors -> (o bf16, lse fp32 [B, H, S]).

    Enqueued on torch's current stream; does not synchronise."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16, got {t.dtype}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, S, D]")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"q, k, v shapes differ: {tuple(q.shape)} {tuple(k.shape)} {tuple(v.shape)}")
    if k.device != q.device or v.device != q.device:
        raise ValueError(f"q, k, v are on different devices: {q.device} {k.device} {v.device}")
    B, H, S, D = q.shape
    if scale is None:
        scale = default_scale(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if out.dtype != torch.bfloat16 or out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 tensor shaped like q")
    if lse.dtype != torch.float32 or lse.shape != (B, H, S) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, S] tensor")
    # the kernel writes through these pointers: they must be device memory of q's GPU
    if out.device != q.device or lse.device != q.device:
        raise ValueError(f"out and lse must be on {q.device}, got {out.device} and {lse.device}")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = attn_fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                      B, H, S, D, float(scale), stream, variant)
    if st != ATTN_OK:
        raise AttnError(st, status_str(st))
    return out, lse


MFMA_RATE_FLOPS_PER_WG_ITER = 4 * 32 * 16384  # 4 waves x 32 MFMAs x 2*16*16*32


def mfma_rate(operands, sink, workgroups: int, iters: int) -> int:
    """Enqueue the MFMA-rate stream (include/attn_mfma_rate.h) on torch's current
    stream: `operands` a device tensor of at least workgroups*256*128 bytes,
    `sink` a float32 device tensor of at least workgroups*256 elements.
    Returns the FLOPs the launch performs; raises AttnError on a bad status."""
    import torch

    if not (operands.is_cuda and sink.is_cuda and sink.dtype == torch.float32):
        raise ValueError("operands and a float32 sink must be device tensors")
    if not (operands.is_contiguous() and sink.is_contiguous()):
        raise ValueError("operands and sink must be contiguous")
    if operands.numel() * operands.element_size() < workgroups * 256 * 128 or sink.numel() < workgroups * 256:
        raise ValueError("operands or sink too small for this many workgroups")
    stream = torch.cuda.current_stream(operands.device).cuda_stream
    st = lib().attn_mfma_rate(operands.data_ptr(), sink.data_ptr(), int(workgroups), int(iters), stream)
    if st != ATTN_OK:
        raise AttnError(st, status_str(st))
    return workgroups * iters * MFMA_RATE_FLOPS_PER_WG_ITER
