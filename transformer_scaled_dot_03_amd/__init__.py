"""Scaled dot-product attention on MI355X (gfx950), HIP kernels behind a C ABI.

Low level (same names and parameters as include/attn.h):
    attn_fwd, attn_fwd_f32, attn_fwd_lse, attn_fwd_weights, attn_bwd, attn_decode,
    attn_decode_workspace_bytes, attn_mha_fwd, attn_mha_workspace_bytes, attn_status_str,
    attn_last_hip_error, attn_version

Tensor level:
    attention(q, k, v, scale=None, causal=False, key_lens=None, out=None, stream=None)
    attention_lse(q, k, v, ...) -> (out, lse)
    attention_weights(q, k, v, ...) -> (out, weights, lse)
    attention_backward(q, k, v, out, dout, lse, ...) -> (dq, dk, dv)
    AttentionFunction.apply(q, k, v, scale, causal, key_lens)   (torch.autograd)
    decode_attention(q, k_cache, v_cache, scale=None, key_lens=None, ...) -> out [B, h, 1, d]
    multi_head_attention(xq, wq, wk, wv, wo, heads, xk=None, xv=None, ...) -> y [B, Tq, d_model]

PyTorch only supplies device memory and the stream handle; the work is done
by libattn.so.
"""
from ._lib import (  # noqa: F401
    ERR_ALIAS, ERR_ALIGN, ERR_HEADDIM, ERR_HIP, ERR_MASK, ERR_NULL, ERR_SCALE, ERR_SHAPE,
    ERR_TOO_LARGE, ERR_WORKSPACE, LIB_PATH, MASK_CAUSAL, MASK_KEYPAD, MASK_NONE, OK, LibraryMissing,
    attn_bwd, attn_decode, attn_decode_workspace_bytes, attn_fwd, attn_fwd_f32, attn_fwd_lse, attn_fwd_weights, attn_last_hip_error, attn_mha_fwd, attn_mha_workspace_bytes, attn_status_str, attn_version, raw_library,
)
from .ops import (AttentionError, AttentionFunction, attention, attention_backward, attention_lse,  # noqa: F401
                  attention_weights, decode_attention, multi_head_attention)

__version__ = "0.1.0"
