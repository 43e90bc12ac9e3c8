"""Tensor-level wrapper over the C ABI (argument marshalling only).

attention() checks the tensors, takes their device pointers and the current
HIP stream, and calls attn_fwd / attn_fwd_f32.  It never computes attention
itself: a missing library raises at import, a failed call raises
AttentionError.
"""
from __future__ import annotations

import math

import torch

from . import _lib


class AttentionError(RuntimeError):
    def __init__(self, status: int):
        msg = _lib.attn_status_str(status)
        if status == _lib.ERR_HIP:
            msg += f" (hipError_t {_lib.attn_last_hip_error()})"
        super().__init__(f"attn status {status}: {msg}")
        self.status = status


def default_scale(d_k: int) -> float:
    """1/sqrt(d_k) rounded once to fp32 (the value the library receives)."""
    return float(torch.tensor(1.0 / math.sqrt(d_k), dtype=torch.float32))


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float | None = None,
              causal: bool = False, key_lens: torch.Tensor | None = None,
              out: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """softmax(scale * q k^T) v for [B, h, T, d] device tensors (bf16 or fp32).

    key_lens: optional int32 [B] device tensor (key padding); causal: j <= i.
    The kernel is enqueued on `stream` (default: the current stream).
    """
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, h, T, d]")
    B, h, Tq, dk = q.shape
    Tk = k.shape[2]
    dv = v.shape[3]
    if k.shape != (B, h, Tk, dk) or v.shape[:3] != (B, h, Tk):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q, k, v must all be bfloat16 or all float32")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if out is None:
        out = torch.empty((B, h, Tq, dv), dtype=q.dtype, device=q.device)
    elif out.shape != (B, h, Tq, dv) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, h, Tq, d_v] tensor of the input dtype")
    mask = _lib.MASK_CAUSAL if causal else _lib.MASK_NONE
    kl_ptr = None
    if key_lens is not None:
        if key_lens.dtype != torch.int32 or not key_lens.is_cuda or key_lens.shape != (B,):
            raise ValueError("key_lens must be an int32 [B] device tensor")
        mask |= _lib.MASK_KEYPAD
        kl_ptr = key_lens.data_ptr()
    if scale is None:
        scale = default_scale(dk)
    st = (stream if stream is not None else torch.cuda.current_stream(q.device)).cuda_stream
    fn = _lib.attn_fwd if q.dtype == torch.bfloat16 else _lib.attn_fwd_f32
    status = fn(q.data_ptr() or None, k.data_ptr() or None, v.data_ptr() or None,
                out.data_ptr() or None, B, h, Tq, Tk, dk, dv, float(scale), mask, kl_ptr, st)
    if status != _lib.OK:
        raise AttentionError(status)
    return out
