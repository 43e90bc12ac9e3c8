"""Tensor-level wrapper over the C ABI (argument marshalling only).

attention() checks the tensors, takes their device pointers and the current
HIP stream, and calls attn_fwd / attn_fwd_f32; attention_lse() and
attention_backward() do the same for attn_fwd_lse and attn_bwd, and
AttentionFunction ties the two into torch.autograd.  Nothing here computes
attention itself: a missing library raises on first use, a failed call
raises AttentionError.
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


def _check_qkv(q, k, v, dtypes):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, h, T, d]")
    B, h, Tq, dk = q.shape
    Tk = k.shape[2]
    dv = v.shape[3]
    if k.shape != (B, h, Tk, dk) or v.shape[:3] != (B, h, Tk):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in dtypes:
        raise TypeError("q, k, v must share one dtype out of " + ", ".join(str(d) for d in dtypes))
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or t.device != q.device:
            raise ValueError(f"{name} must be a device tensor on q's device")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    return B, h, Tq, Tk, dk, dv


def _on_device(t, device) -> bool:
    """True when t lives in the memory of the GPU `device` (a CPU tensor's address
    would pass every check of the C ABI and then be written by a kernel)."""
    return t.is_cuda and t.device == torch.device(device)


def _mask_args(B, causal, key_lens, device):
    mask = _lib.MASK_CAUSAL if causal else _lib.MASK_NONE
    kl_ptr = None
    if key_lens is not None:
        if (key_lens.dtype != torch.int32 or tuple(key_lens.shape) != (B,) or not key_lens.is_contiguous()
                or not _on_device(key_lens, device)):
            raise ValueError("key_lens must be a contiguous int32 [B] tensor on the inputs' device")
        mask |= _lib.MASK_KEYPAD
        kl_ptr = key_lens.data_ptr()
    return mask, kl_ptr


def _out_like(t, shape, dtype, device, name):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or not _on_device(t, device):
        raise ValueError(f"{name} must be a contiguous {tuple(shape)} {dtype} tensor on {device}")
    return t


def _ptr(t):
    return None if t is None else (t.data_ptr() or None)


def _stream_handle(stream, device):
    """The HIP stream handle to enqueue on: `stream`, or the current stream of
    `device`.  A stream of another GPU is refused: its kernel would run there on
    pointers into this device's memory."""
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if torch.device(stream.device) != torch.device(device):
        raise ValueError(f"stream is on {stream.device}, the tensors on {device}")
    return stream.cuda_stream


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float | None = None,
              causal: bool = False, key_lens: torch.Tensor | None = None,
              out: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """softmax(scale * q k^T) v for [B, h, T, d] device tensors (bf16 or fp32).

    key_lens: optional int32 [B] device tensor (key padding); causal: j <= i.
    The kernel is enqueued on `stream` (default: the current stream).
    """
    B, h, Tq, Tk, dk, dv = _check_qkv(q, k, v, (torch.bfloat16, torch.float32))
    out = _out_like(out, (B, h, Tq, dv), q.dtype, q.device, "out")
    mask, kl_ptr = _mask_args(B, causal, key_lens, q.device)
    if scale is None:
        scale = default_scale(dk)
    st = _stream_handle(stream, q.device)
    fn = _lib.attn_fwd if q.dtype == torch.bfloat16 else _lib.attn_fwd_f32
    status = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, h, Tq, Tk, dk, dv, float(scale), mask, kl_ptr, st)
    if status != _lib.OK:
        raise AttentionError(status)
    return out

def attention_lse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float | None = None,
                  causal: bool = False, key_lens: torch.Tensor | None = None,
                  out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                  stream: torch.cuda.Stream | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """bf16 forward that also returns the fp32 row log-sum-exp [B, h, Tq] (attn_fwd_lse)."""
    B, h, Tq, Tk, dk, dv = _check_qkv(q, k, v, (torch.bfloat16,))
    out = _out_like(out, (B, h, Tq, dv), q.dtype, q.device, "out")
    lse = _out_like(lse, (B, h, Tq), torch.float32, q.device, "lse")
    mask, kl_ptr = _mask_args(B, causal, key_lens, q.device)
    if scale is None:
        scale = default_scale(dk)
    st = _stream_handle(stream, q.device)
    status = _lib.attn_fwd_lse(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, h, Tq, Tk, dk, dv,
                               float(scale), mask, kl_ptr, st)
    if status != _lib.OK:
        raise AttentionError(status)
    return out, lse


def attention_weights(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float | None = None,
                      causal: bool = False, key_lens: torch.Tensor | None = None,
                      out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                      weights: torch.Tensor | None = None,
                      stream: torch.cuda.Stream | None = None):
    """bf16 forward returning (out, weights, lse); weights fp32 [B, h, Tq, Tk] (attn_fwd_weights)."""
    B, h, Tq, Tk, dk, dv = _check_qkv(q, k, v, (torch.bfloat16,))
    out = _out_like(out, (B, h, Tq, dv), q.dtype, q.device, "out")
    lse = _out_like(lse, (B, h, Tq), torch.float32, q.device, "lse")
    weights = _out_like(weights, (B, h, Tq, Tk), torch.float32, q.device, "weights")
    mask, kl_ptr = _mask_args(B, causal, key_lens, q.device)
    if scale is None:
        scale = default_scale(dk)
    st = _stream_handle(stream, q.device)
    status = _lib.attn_fwd_weights(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(weights), B, h, Tq, Tk,
                                   dk, dv, float(scale), mask, kl_ptr, st)
    if status != _lib.OK:
        raise AttentionError(status)
    return out, weights, lse


def attention_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                       dout: torch.Tensor, lse: torch.Tensor, scale: float | None = None,
                       causal: bool = False, key_lens: torch.Tensor | None = None,
                       dq: torch.Tensor | None = None, dk: torch.Tensor | None = None,
                       dv: torch.Tensor | None = None, delta: torch.Tensor | None = None,
                       stream: torch.cuda.Stream | None = None):
    """Gradients (dq, dk, dv) of attention for bf16 tensors (attn_bwd).

    out and lse are what attention_lse returned for these inputs; dout is the
    gradient of the loss with respect to out.  delta (fp32 [2, B, h, Tq]) is
    the kernels' workspace, allocated here when not given.
    """
    B, h, Tq, Tk, d_k, d_v = _check_qkv(q, k, v, (torch.bfloat16,))
    for name, t, shape in (("out", out, (B, h, Tq, d_v)), ("dout", dout, (B, h, Tq, d_v))):
        if (tuple(t.shape) != shape or t.dtype != torch.bfloat16 or not t.is_contiguous()
                or not _on_device(t, q.device)):
            raise ValueError(f"{name} must be a contiguous bf16 tensor of shape {shape} on q's device")
    if (tuple(lse.shape) != (B, h, Tq) or lse.dtype != torch.float32 or not lse.is_contiguous()
            or not _on_device(lse, q.device)):
        raise ValueError("lse must be a contiguous fp32 [B, h, Tq] tensor on q's device")
    dq = _out_like(dq, q.shape, q.dtype, q.device, "dq")
    dk = _out_like(dk, k.shape, k.dtype, k.device, "dk")
    dv = _out_like(dv, v.shape, v.dtype, v.device, "dv")
    delta = _out_like(delta, (2, B, h, Tq), torch.float32, q.device, "delta")
    mask, kl_ptr = _mask_args(B, causal, key_lens, q.device)
    if scale is None:
        scale = default_scale(d_k)
    st = _stream_handle(stream, q.device)
    status = _lib.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(delta),
                           _ptr(dq), _ptr(dk), _ptr(dv), B, h, Tq, Tk, d_k, d_v, float(scale), mask, kl_ptr, st)
    if status != _lib.OK:
        raise AttentionError(status)
    return dq, dk, dv


class AttentionFunction(torch.autograd.Function):
    """softmax(scale q k^T) v with gradients: forward attn_fwd_lse, backward attn_bwd (bf16)."""

    @staticmethod
    def forward(ctx, q, k, v, scale=None, causal=False, key_lens=None):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        out, lse = attention_lse(q, k, v, scale=scale, causal=causal, key_lens=key_lens)
        ctx.save_for_backward(q, k, v, out, lse, key_lens)
        ctx.scale, ctx.causal = scale, causal
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, lse, key_lens = ctx.saved_tensors
        dq, dk, dv = attention_backward(q, k, v, out, dout.contiguous(), lse, scale=ctx.scale,
                                        causal=ctx.causal, key_lens=key_lens)
        return dq, dk, dv, None, None, None


def decode_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float | None = None,
                     key_lens: torch.Tensor | None = None, out: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None,
                     stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """One query row per (b, head) against a bf16 K/V cache (attn_decode).

    q: [B, h, 1, d]; k, v: [B, h, Tk, d]; key_lens: optional int32 [B] device
    tensor of valid cache lengths.  workspace: optional uint8 device tensor of
    at least attn_decode_workspace_bytes(B, h, Tk, d) bytes (allocated here
    when not given; calls sharing one must not overlap in time).
    """
    B, h, Tq, Tk, dk, dv = _check_qkv(q, k, v, (torch.bfloat16,))
    if Tq != 1:
        raise ValueError("decode_attention takes one query row per (b, head): q must be [B, h, 1, d]")
    out = _out_like(out, (B, h, 1, dv), q.dtype, q.device, "out")
    mask, kl_ptr = _mask_args(B, False, key_lens, q.device)
    need = _lib.attn_decode_workspace_bytes(B, h, Tk, dk) if B > 0 and h > 0 else 0
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.dtype != torch.uint8 or not workspace.is_contiguous() or not _on_device(workspace, q.device):
        raise ValueError("workspace must be a contiguous uint8 tensor on q's device")
    if scale is None:
        scale = default_scale(dk)
    st = _stream_handle(stream, q.device)
    status = _lib.attn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, h, Tk, dk, dv, float(scale), mask, kl_ptr,
                              _ptr(workspace), workspace.numel(), st)
    if status != _lib.OK:
        raise AttentionError(status)
    return out


def multi_head_attention(xq: torch.Tensor, wq: torch.Tensor, wk: torch.Tensor, wv: torch.Tensor,
                         wo: torch.Tensor, heads: int, xk: torch.Tensor | None = None,
                         xv: torch.Tensor | None = None, scale: float | None = None, causal: bool = False,
                         key_lens: torch.Tensor | None = None, out: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None,
                         stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """Concat(head_1..head_h) W^O with head_i = Attention(xq W_i^Q, xk W_i^K, xv W_i^V) (attn_mha_fwd).

    xq: [B, Tq, d_model]; xk, xv: [B, Tk, d_model] (default: xq, i.e. self-attention);
    wq, wk, wv, wo: [d_model, d_model]; all bf16 device tensors.  scale defaults
    to 1/sqrt(d_model / heads).  workspace: optional uint8 device tensor of at
    least attn_mha_workspace_bytes(B, Tq, Tk, d_model) bytes.
    """
    xk = xq if xk is None else xk
    xv = xk if xv is None else xv
    ts = (("xq", xq), ("xk", xk), ("xv", xv), ("wq", wq), ("wk", wk), ("wv", wv), ("wo", wo))
    for name, t in ts:
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or not _on_device(t, xq.device):
            raise ValueError(f"{name} must be a contiguous bf16 tensor on xq's device")
    if xq.dim() != 3 or xk.dim() != 3 or xv.shape != xk.shape:
        raise ValueError("xq must be [B, Tq, d_model] and xk, xv [B, Tk, d_model]")
    B, Tq, dm = xq.shape
    Tk = xk.shape[1]
    if xk.shape[0] != B or xk.shape[2] != dm:
        raise ValueError("xk, xv must be [B, Tk, d_model] with the batch and width of xq")
    for name, w in (("wq", wq), ("wk", wk), ("wv", wv), ("wo", wo)):
        if tuple(w.shape) != (dm, dm):
            raise ValueError(f"{name} must be [d_model, d_model]")
    out = _out_like(out, (B, Tq, dm), torch.bfloat16, xq.device, "out")
    mask, kl_ptr = _mask_args(B, causal, key_lens, xq.device)
    need = _lib.attn_mha_workspace_bytes(B, Tq, Tk, dm)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=xq.device)
    elif workspace.dtype != torch.uint8 or not workspace.is_contiguous() or not _on_device(workspace, xq.device):
        raise ValueError("workspace must be a contiguous uint8 tensor on xq's device")
    if scale is None:
        scale = default_scale(dm // heads) if heads > 0 and dm % heads == 0 else 1.0
    st = _stream_handle(stream, xq.device)
    status = _lib.attn_mha_fwd(_ptr(xq), _ptr(xk), _ptr(xv), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo), _ptr(out),
                               B, Tq, Tk, dm, heads, float(scale), mask, kl_ptr, _ptr(workspace),
                               workspace.numel(), st)
    if status != _lib.OK:
        raise AttentionError(status)
    return out
