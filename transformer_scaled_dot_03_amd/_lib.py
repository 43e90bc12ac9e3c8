"""ctypes binding of libattn.so: argument marshalling only.

Every function here forwards to the C ABI declared in include/attn.h with the
same name and parameter list; all computation happens in the HIP kernels.
If the library has not been built the import fails loudly: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_KEYPAD = 2

OK = 0
ERR_NULL = -1
ERR_SHAPE = -2
ERR_HEADDIM = -3
ERR_MASK = -4
ERR_ALIAS = -5
ERR_ALIGN = -6
ERR_SCALE = -7
ERR_TOO_LARGE = -8
ERR_WORKSPACE = -9
ERR_HIP = -100

# names and C signatures of every exported entry point (kept in step with attn.h)
_P = ctypes.c_void_p
_I = ctypes.c_int
_FWD_ARGS = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I, _P, _P]
_FWD_LSE_ARGS = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I, _P, _P]
_BWD_ARGS = [_P] * 10 + [_I] * 6 + [ctypes.c_float, _I, _P, _P]
SIGNATURES = {
    "attn_fwd": (_I, _FWD_ARGS),
    "attn_fwd_f32": (_I, _FWD_ARGS),
    "attn_fwd_lse": (_I, _FWD_LSE_ARGS),
    "attn_bwd": (_I, _BWD_ARGS),
    "attn_mha_fwd": (_I, [_P] * 8 + [_I] * 5 + [ctypes.c_float, _I, _P, _P, ctypes.c_size_t, _P]),
    "attn_mha_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "attn_fwd_weights": (_I, [_P] * 6 + [_I] * 6 + [ctypes.c_float, _I, _P, _P]),
    "attn_decode": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_float, _I, _P, _P, ctypes.c_size_t, _P]),
    "attn_decode_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "attn_decode_static": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_float, _I, _P, _P]),
    "attn_status_str": (ctypes.c_char_p, [_I]),
    "attn_last_hip_error": (_I, []),
    "attn_version": (ctypes.c_char_p, []),
}


class LibraryMissing(ImportError):
    pass


def _load():
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing(
            f"{LIB_PATH} is not built: run `python -m transformer_scaled_dot_03_amd.build` "
            "(or __graft_entry__.build()); there is no non-HIP fallback")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = None


def raw_library():
    """The loaded ctypes.CDLL; loaded on first use, raises LibraryMissing if unbuilt."""
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def attn_fwd(q, k, v, out, B, h, Tq, Tk, d_k, d_v, scale, mask_kind, key_lens, stream) -> int:
    """bf16 attention forward (attn.h `attn_fwd`); pointers are ints (device addresses)."""
    return raw_library().attn_fwd(q, k, v, out, B, h, Tq, Tk, d_k, d_v, scale, mask_kind, key_lens, stream)


def attn_fwd_f32(q, k, v, out, B, h, Tq, Tk, d_k, d_v, scale, mask_kind, key_lens, stream) -> int:
    """fp32 attention forward (attn.h `attn_fwd_f32`)."""
    return raw_library().attn_fwd_f32(q, k, v, out, B, h, Tq, Tk, d_k, d_v, scale, mask_kind, key_lens,
                                      stream)


def attn_fwd_lse(q, k, v, out, lse, B, h, Tq, Tk, d_k, d_v, scale, mask_kind, key_lens, stream) -> int:
    """bf16 attention forward that also writes the fp32 row log-sum-exp (attn.h `attn_fwd_lse`)."""
    return raw_library().attn_fwd_lse(q, k, v, out, lse, B, h, Tq, Tk, d_k, d_v, scale, mask_kind, key_lens,
                                      stream)


def attn_bwd(q, k, v, out, dout, lse, delta, dq, dk, dv, B, h, Tq, Tk, d_k, d_v, scale, mask_kind, key_lens,
             stream) -> int:
    """bf16 attention backward: dq, dk, dv (and delta) from out, dout and lse (attn.h `attn_bwd`)."""
    return raw_library().attn_bwd(q, k, v, out, dout, lse, delta, dq, dk, dv, B, h, Tq, Tk, d_k, d_v, scale,
                                  mask_kind, key_lens, stream)


def attn_fwd_weights(q, k, v, out, lse, weights, B, h, Tq, Tk, d_k, d_v, scale, mask_kind, key_lens,
                     stream) -> int:
    """bf16 forward plus fp32 log-sum-exp and fp32 attention weights (attn.h `attn_fwd_weights`)."""
    return raw_library().attn_fwd_weights(q, k, v, out, lse, weights, B, h, Tq, Tk, d_k, d_v, scale, mask_kind,
                                          key_lens, stream)


def attn_mha_fwd(xq, xk, xv, wq, wk, wv, wo, y, B, Tq, Tk, d_model, h, scale, mask_kind, key_lens, workspace,
                 workspace_bytes, stream) -> int:
    """bf16 multi-head attention forward (attn.h `attn_mha_fwd`)."""
    return raw_library().attn_mha_fwd(xq, xk, xv, wq, wk, wv, wo, y, B, Tq, Tk, d_model, h, scale, mask_kind,
                                      key_lens, workspace, workspace_bytes, stream)


def attn_mha_workspace_bytes(B, Tq, Tk, d_model) -> int:
    """Workspace bytes attn_mha_fwd needs (attn.h `attn_mha_workspace_bytes`)."""
    return raw_library().attn_mha_workspace_bytes(B, Tq, Tk, d_model)


def attn_decode(q, k, v, out, B, h, Tk, d_k, d_v, scale, mask_kind, key_lens, workspace, workspace_bytes,
                stream) -> int:
    """bf16 single-row decode attention over a K/V cache (attn.h `attn_decode`)."""
    return raw_library().attn_decode(q, k, v, out, B, h, Tk, d_k, d_v, scale, mask_kind, key_lens, workspace,
                                     workspace_bytes, stream)


def attn_decode_static(q, k, v, out, B, h, Tk, d_k, d_v, scale, mask_kind, key_lens, stream) -> int:
    """attn_decode with the partials in the library's static device array (attn.h `attn_decode_static`)."""
    return raw_library().attn_decode_static(q, k, v, out, B, h, Tk, d_k, d_v, scale, mask_kind, key_lens, stream)


# bytes of the static device array behind attn_decode_static (attn.h ATTN_DECODE_STATIC_SCRATCH_BYTES)
DECODE_STATIC_SCRATCH_BYTES = 16 << 20


def attn_decode_workspace_bytes(B, h, Tk, d) -> int:
    """Workspace bytes attn_decode needs (attn.h `attn_decode_workspace_bytes`)."""
    return raw_library().attn_decode_workspace_bytes(B, h, Tk, d)


def attn_status_str(status: int) -> str:
    return raw_library().attn_status_str(status).decode()


def attn_last_hip_error() -> int:
    return raw_library().attn_last_hip_error()


def attn_version() -> str:
    return raw_library().attn_version().decode()
