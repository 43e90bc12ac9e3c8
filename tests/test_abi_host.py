"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every entry point include/attn.h declares, and
reject bad arguments with the documented status before any HIP call (the
pointers below are never dereferenced; these calls make no HIP call at all).

The calls pass made-up device addresses.  Where a GPU is visible, a
regressed check would launch a kernel on them, so there the tests of this
file run only in a child process that sees no GPU (test_abi_isolated.py
starts it with HIP_VISIBLE_DEVICES empty): a launch then fails with
ATTN_ERR_HIP instead of touching memory.  The same child mode runs them
against a build of the library whose host code is instrumented with
AddressSanitizer and UndefinedBehaviorSanitizer (ATTN_ABI_TEST_LIB).
"""
from __future__ import annotations

import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

# set by test_abi_isolated.py in the child processes it starts
CHILD = os.environ.get("ATTN_ABI_HOST_CHILD") == "1"
GPU_NODE = os.path.exists("/dev/kfd")

pytestmark = pytest.mark.skipif(
    GPU_NODE and not CHILD,
    reason="a GPU is visible: these fake-address calls run in a GPU-less child (test_abi_isolated.py)")


def _visible_gpus() -> int:
    """Devices the HIP runtime reports in this process (0 if it reports an error)."""
    hip = ctypes.CDLL("libamdhip64.so")
    n = ctypes.c_int(0)
    return n.value if hip.hipGetDeviceCount(ctypes.byref(n)) == 0 else 0


@pytest.fixture(scope="module", autouse=True)
def no_gpu_in_child():
    """In the child on a GPU host, refuse to run if the runtime still sees a device."""
    if CHILD and GPU_NODE and _visible_gpus() != 0:
        pytest.exit("HIP_VISIBLE_DEVICES did not hide the GPU: not running fake-address calls", returncode=3)


@pytest.fixture(scope="module")
def L():
    from transformer_scaled_dot_03_amd import _lib
    other = os.environ.get("ATTN_ABI_TEST_LIB")
    if other:
        # a differently built copy of the library (the sanitizer build)
        _lib.LIB_PATH = other
        _lib._lib = None
    elif not os.path.exists(_lib.LIB_PATH):
        from transformer_scaled_dot_03_amd import build
        build.build()
    return _lib


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", src)))


def _declared_enum():
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return {k: int(v) for k, v in re.findall(r"\b(ATTN_\w+)\s*=\s*(-?\d+)", src)}


def test_header_declares_expected_entry_points():
    assert _declared_functions() == sorted(
        ["attn_fwd", "attn_fwd_f32", "attn_fwd_lse", "attn_fwd_weights", "attn_bwd", "attn_decode",
         "attn_decode_static", "attn_decode_workspace_bytes", "attn_mha_fwd", "attn_mha_workspace_bytes",
         "attn_status_str", "attn_last_hip_error", "attn_version"])


def test_library_exports_every_declared_symbol(L):
    lib = L.raw_library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    # and the binding covers exactly the declared set
    assert sorted(L.SIGNATURES) == _declared_functions()


def test_status_constants_match_header(L):
    enum = _declared_enum()
    assert enum["ATTN_OK"] == L.OK
    for name in ("NULL", "SHAPE", "HEADDIM", "MASK", "ALIAS", "ALIGN", "SCALE", "TOO_LARGE", "WORKSPACE", "HIP"):
        assert enum["ATTN_ERR_" + name] == getattr(L, "ERR_" + name)
    for name in ("NONE", "CAUSAL", "KEYPAD"):
        assert enum["ATTN_MASK_" + name] == getattr(L, "MASK_" + name)


def test_status_strings_and_version(L):
    for code in (L.OK, L.ERR_NULL, L.ERR_SHAPE, L.ERR_HEADDIM, L.ERR_MASK, L.ERR_ALIAS,
                 L.ERR_ALIGN, L.ERR_SCALE, L.ERR_TOO_LARGE, L.ERR_WORKSPACE, L.ERR_HIP):
        s = L.attn_status_str(code)
        assert s and s != "unknown status"
    assert L.attn_status_str(12345) == "unknown status"
    assert "gfx950" in L.attn_version()
    assert L.attn_last_hip_error() == 0


# fake, well-aligned, non-overlapping device addresses: never dereferenced
Q, K, V, O, KL = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000
GOOD = dict(q=Q, k=K, v=V, out=O, B=2, h=3, Tq=70, Tk=90, d_k=64, d_v=64, scale=0.125,
            mask_kind=0, key_lens=None, stream=None)


def _call(L, f32=False, **over):
    a = dict(GOOD)
    a.update(over)
    fn = L.attn_fwd_f32 if f32 else L.attn_fwd
    return fn(a["q"], a["k"], a["v"], a["out"], a["B"], a["h"], a["Tq"], a["Tk"], a["d_k"],
              a["d_v"], a["scale"], a["mask_kind"], a["key_lens"], a["stream"])


@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("over,code", [
    (dict(B=-1), "ERR_SHAPE"),
    (dict(h=-2), "ERR_SHAPE"),
    (dict(Tq=-1), "ERR_SHAPE"),
    (dict(Tk=-1), "ERR_SHAPE"),
    (dict(d_v=128), "ERR_SHAPE"),
    (dict(d_k=32, d_v=32), "ERR_HEADDIM"),
    (dict(d_k=256, d_v=256), "ERR_HEADDIM"),
    (dict(d_k=0, d_v=0), "ERR_HEADDIM"),
    (dict(mask_kind=4), "ERR_MASK"),
    (dict(mask_kind=-1), "ERR_MASK"),
    (dict(mask_kind=2), "ERR_MASK"),            # key padding without key_lens
    (dict(mask_kind=3), "ERR_MASK"),
    (dict(scale=float("nan")), "ERR_SCALE"),
    (dict(scale=float("inf")), "ERR_SCALE"),
    (dict(scale=-math.inf), "ERR_SCALE"),
    (dict(q=None), "ERR_NULL"),
    (dict(out=None), "ERR_NULL"),
    (dict(k=None), "ERR_NULL"),
    (dict(v=None), "ERR_NULL"),
    (dict(q=Q + 8), "ERR_ALIGN"),
    (dict(k=K + 2), "ERR_ALIGN"),
    (dict(v=V + 4), "ERR_ALIGN"),
    (dict(out=O + 12), "ERR_ALIGN"),
    (dict(mask_kind=2, key_lens=KL + 2), "ERR_ALIGN"),
    (dict(mask_kind=2, key_lens=O + 64), "ERR_ALIAS"),   # out overlaps key_lens
    (dict(out=Q), "ERR_ALIAS"),
    (dict(out=K + 4096), "ERR_ALIAS"),
    (dict(out=V - 16), "ERR_ALIAS"),
    (dict(B=1 << 30, h=1 << 10, Tq=1 << 20), "ERR_TOO_LARGE"),
    (dict(B=1, h=1, Tk=1 << 25, d_k=128, d_v=128), "ERR_TOO_LARGE"),   # one head's K: 8 GiB
])
def test_bad_arguments_rejected_before_any_launch(L, f32, over, code):
    assert _call(L, f32=f32, **over) == getattr(L, code)
    assert L.attn_last_hip_error() == 0


@pytest.mark.parametrize("over", [dict(B=0), dict(h=0), dict(Tq=0), dict(B=0, q=None, out=None),
                                  dict(Tq=0, q=None, k=None, v=None, out=None)])
def test_empty_problem_is_a_no_op(L, over):
    assert _call(L, **over) == L.OK


def test_keypad_needs_key_lens_even_when_empty(L):
    assert _call(L, B=0, mask_kind=L.MASK_KEYPAD) == L.ERR_MASK


LSE = 0x60000000


def _call_lse(L, **over):
    a = dict(GOOD, lse=LSE)
    a.update(over)
    return L.attn_fwd_lse(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["h"], a["Tq"], a["Tk"],
                          a["d_k"], a["d_v"], a["scale"], a["mask_kind"], a["key_lens"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(lse=None), "ERR_NULL"),
    (dict(lse=LSE + 2), "ERR_ALIGN"),
    (dict(lse=O + 64), "ERR_ALIAS"),
    (dict(lse=Q), "ERR_ALIAS"),
    (dict(mask_kind=2, key_lens=LSE + 8), "ERR_ALIAS"),   # lse overlaps key_lens
    (dict(d_k=32, d_v=32), "ERR_HEADDIM"),
    (dict(mask_kind=2), "ERR_MASK"),
    (dict(scale=float("nan")), "ERR_SCALE"),
    (dict(out=K), "ERR_ALIAS"),
])
def test_fwd_lse_bad_arguments(L, over, code):
    assert _call_lse(L, **over) == getattr(L, code)
    assert L.attn_last_hip_error() == 0


def test_fwd_lse_empty_is_a_no_op(L):
    assert _call_lse(L, Tq=0, lse=None) == L.OK
    assert _call_lse(L, B=0, lse=None, q=None, out=None) == L.OK


WTS = 0x70000000


def _call_wts(L, **over):
    a = dict(GOOD, lse=LSE, weights=WTS)
    a.update(over)
    return L.attn_fwd_weights(a["q"], a["k"], a["v"], a["out"], a["lse"], a["weights"], a["B"], a["h"], a["Tq"],
                              a["Tk"], a["d_k"], a["d_v"], a["scale"], a["mask_kind"], a["key_lens"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(weights=None), "ERR_NULL"),
    (dict(lse=None), "ERR_NULL"),
    (dict(weights=WTS + 8), "ERR_ALIGN"),
    (dict(weights=Q + 1024), "ERR_ALIAS"),
    (dict(weights=LSE - 64), "ERR_ALIAS"),       # its first bytes run into lse
    (dict(weights=O), "ERR_ALIAS"),
    (dict(mask_kind=2, key_lens=WTS + 1024), "ERR_ALIAS"),   # weights overlap key_lens
    (dict(d_k=32, d_v=32, weights=None), "ERR_HEADDIM"),   # the forward's checks come first
    (dict(mask_kind=5), "ERR_MASK"),
    (dict(scale=float("inf")), "ERR_SCALE"),
    (dict(Tq=-1), "ERR_SHAPE"),
])
def test_fwd_weights_bad_arguments(L, over, code):
    assert _call_wts(L, **over) == getattr(L, code)
    assert L.attn_last_hip_error() == 0


def test_fwd_weights_empty_is_a_no_op(L):
    assert _call_wts(L, Tq=0, lse=None, weights=None) == L.OK
    assert _call_wts(L, B=0, q=None, out=None, lse=None, weights=None) == L.OK


# backward: fake addresses 256 MiB apart, never dereferenced
BW = dict(q=0x10000000, k=0x20000000, v=0x30000000, out=0x40000000, dout=0x50000000, lse=0x60000000,
          delta=0x70000000, dq=0x80000000, dk=0x90000000, dv=0xA0000000, B=2, h=3, Tq=70, Tk=90, d_k=64,
          d_v=64, scale=0.125, mask_kind=0, key_lens=None, stream=None)


def _call_bwd(L, **over):
    a = dict(BW)
    a.update(over)
    return L.attn_bwd(a["q"], a["k"], a["v"], a["out"], a["dout"], a["lse"], a["delta"], a["dq"], a["dk"],
                      a["dv"], a["B"], a["h"], a["Tq"], a["Tk"], a["d_k"], a["d_v"], a["scale"],
                      a["mask_kind"], a["key_lens"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(B=-1), "ERR_SHAPE"),
    (dict(Tk=-3), "ERR_SHAPE"),
    (dict(d_v=128), "ERR_SHAPE"),
    (dict(d_k=96, d_v=96), "ERR_HEADDIM"),
    (dict(mask_kind=8), "ERR_MASK"),
    (dict(mask_kind=2), "ERR_MASK"),
    (dict(scale=float("inf")), "ERR_SCALE"),
    (dict(q=None), "ERR_NULL"),
    (dict(out=None), "ERR_NULL"),
    (dict(dout=None), "ERR_NULL"),
    (dict(lse=None), "ERR_NULL"),
    (dict(delta=None), "ERR_NULL"),
    (dict(dq=None), "ERR_NULL"),
    (dict(k=None), "ERR_NULL"),
    (dict(v=None), "ERR_NULL"),
    (dict(dk=None), "ERR_NULL"),
    (dict(dv=None), "ERR_NULL"),
    (dict(Tq=0, dk=None), "ERR_NULL"),          # the dK/dV kernel still runs
    (dict(Tk=0, dq=None), "ERR_NULL"),          # the dQ kernel still runs
    (dict(dout=0x50000008), "ERR_ALIGN"),
    (dict(dq=0x80000004), "ERR_ALIGN"),
    (dict(dk=0x90000002), "ERR_ALIGN"),
    (dict(dv=0xA0000008), "ERR_ALIGN"),
    (dict(lse=0x60000002), "ERR_ALIGN"),
    (dict(delta=0x70000001), "ERR_ALIGN"),
    (dict(mask_kind=2, key_lens=0xB0000002), "ERR_ALIGN"),
    (dict(dq=0x10000000 + 4096), "ERR_ALIAS"),  # dq inside q
    (dict(dk=0x80000000 + 64), "ERR_ALIAS"),    # dk inside dq
    (dict(delta=0x60000000 + 16), "ERR_ALIAS"), # delta inside lse
    (dict(dv=0x50000000), "ERR_ALIAS"),         # dv on dout
    (dict(delta=0xA0000000 + 128), "ERR_ALIAS"),
    (dict(mask_kind=2, key_lens=0x80000000 + 4), "ERR_ALIAS"),   # dq overlaps key_lens
    (dict(B=1 << 30, h=1 << 10, Tq=1 << 20), "ERR_TOO_LARGE"),
    (dict(B=1, h=1, Tq=1 << 24, d_k=128, d_v=128), "ERR_TOO_LARGE"),   # one head's Q: 4 GiB
])
def test_bwd_bad_arguments_rejected_before_any_launch(L, over, code):
    assert _call_bwd(L, **over) == getattr(L, code)
    assert L.attn_last_hip_error() == 0


@pytest.mark.parametrize("over", [dict(B=0), dict(h=0), dict(Tq=0, Tk=0),
                                  dict(B=0, **{n: None for n in ("q", "k", "v", "out", "dout", "lse", "delta",
                                                                 "dq", "dk", "dv")})])
def test_bwd_empty_problem_is_a_no_op(L, over):
    assert _call_bwd(L, **over) == L.OK


# decode: fake addresses, never dereferenced
DEC = dict(q=0x10000000, k=0x20000000, v=0x30000000, out=0x40000000, B=4, h=8, Tk=5000, d_k=128, d_v=128,
           scale=0.088, mask_kind=0, key_lens=None, ws=0x50000000, ws_bytes=1 << 26, stream=None)


def _call_dec(L, **over):
    a = dict(DEC)
    a.update(over)
    return L.attn_decode(a["q"], a["k"], a["v"], a["out"], a["B"], a["h"], a["Tk"], a["d_k"], a["d_v"],
                         a["scale"], a["mask_kind"], a["key_lens"], a["ws"], a["ws_bytes"], a["stream"])


def test_decode_workspace_size(L):
    assert L.attn_decode_workspace_bytes(0, 8, 100, 64) == 0
    assert L.attn_decode_workspace_bytes(2, 8, 100, 96) == 0
    assert L.attn_decode_workspace_bytes(2, 8, -1, 64) == 0
    small = L.attn_decode_workspace_bytes(1, 1, 10, 64)
    assert small > 0 and small % 256 == 0
    # grows with the cache length (more splits) and with d
    assert L.attn_decode_workspace_bytes(1, 1, 100000, 64) > small
    assert L.attn_decode_workspace_bytes(1, 1, 10, 128) > small
    # at least one partial (max, sum, d outputs) per (b, head)
    assert L.attn_decode_workspace_bytes(3, 5, 0, 64) >= 3 * 5 * (64 + 2) * 4


@pytest.mark.parametrize("over,code", [
    (dict(B=-1), "ERR_SHAPE"),
    (dict(d_v=64), "ERR_SHAPE"),
    (dict(d_k=80, d_v=80), "ERR_HEADDIM"),
    (dict(mask_kind=1), "ERR_MASK"),            # causal is not a decode mask
    (dict(mask_kind=3), "ERR_MASK"),
    (dict(mask_kind=2), "ERR_MASK"),            # key padding without key_lens
    (dict(scale=float("nan")), "ERR_SCALE"),
    (dict(q=None), "ERR_NULL"),
    (dict(k=None), "ERR_NULL"),
    (dict(out=None), "ERR_NULL"),
    (dict(ws=None), "ERR_WORKSPACE"),
    (dict(ws_bytes=1024), "ERR_WORKSPACE"),
    (dict(ws=0x50000008), "ERR_ALIGN"),
    (dict(out=0x40000004), "ERR_ALIGN"),
    (dict(ws=0x20000000 + 4096), "ERR_ALIAS"),  # workspace inside k
    (dict(out=0x10000000), "ERR_ALIAS"),
    (dict(mask_kind=2, key_lens=0x50000000 + 64), "ERR_ALIAS"),   # the workspace overlaps key_lens
    (dict(Tk=1 << 25), "ERR_TOO_LARGE"),
])
def test_decode_bad_arguments_rejected_before_any_launch(L, over, code):
    assert _call_dec(L, **over) == getattr(L, code)
    assert L.attn_last_hip_error() == 0


def test_decode_empty_is_a_no_op(L):
    assert _call_dec(L, B=0, q=None, out=None, ws=None) == L.OK
    assert _call_dec(L, h=0) == L.OK


def _call_dec_static(L, **over):
    a = dict(DEC)
    a.update(over)
    return L.attn_decode_static(a["q"], a["k"], a["v"], a["out"], a["B"], a["h"], a["Tk"], a["d_k"], a["d_v"],
                                a["scale"], a["mask_kind"], a["key_lens"], a["stream"])


def test_decode_static_scratch_size_matches_header(L):
    m = re.search(r"#define ATTN_DECODE_STATIC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == L.DECODE_STATIC_SCRATCH_BYTES


@pytest.mark.parametrize("over,code", [
    (dict(B=-1), "ERR_SHAPE"),
    (dict(d_v=64), "ERR_SHAPE"),
    (dict(d_k=80, d_v=80), "ERR_HEADDIM"),
    (dict(mask_kind=1), "ERR_MASK"),
    (dict(mask_kind=2), "ERR_MASK"),
    (dict(scale=float("inf")), "ERR_SCALE"),
    (dict(q=None), "ERR_NULL"),
    (dict(v=None), "ERR_NULL"),
    (dict(out=0x40000004), "ERR_ALIGN"),
    (dict(out=0x20000000 + 256), "ERR_ALIAS"),   # out inside k
    (dict(mask_kind=2, key_lens=0x40000000), "ERR_ALIAS"),   # out on key_lens
    (dict(Tk=1 << 25), "ERR_TOO_LARGE"),
    # more partials than the static array holds: one per (b, head) already exceeds 16 MiB
    (dict(B=1024, h=64, Tk=1, d_k=64, d_v=64), "ERR_WORKSPACE"),
])
def test_decode_static_bad_arguments_rejected_before_any_hip_call(L, over, code):
    assert _call_dec_static(L, **over) == getattr(L, code)
    assert L.attn_last_hip_error() == 0


def test_decode_static_limit_is_the_workspace_size(L):
    # the largest problems it takes are exactly those whose attn_decode workspace fits the array
    assert L.attn_decode_workspace_bytes(8, 16, 16384, 128) <= L.DECODE_STATIC_SCRATCH_BYTES
    assert L.attn_decode_workspace_bytes(1024, 64, 1, 64) > L.DECODE_STATIC_SCRATCH_BYTES


def test_decode_static_empty_is_a_no_op(L):
    assert _call_dec_static(L, B=0, q=None, out=None) == L.OK
    assert _call_dec_static(L, h=0) == L.OK


# multi-head: fake addresses 256 MiB apart, never dereferenced
MHA = dict(xq=0x10000000, xk=0x10000000, xv=0x10000000, wq=0x20000000, wk=0x30000000, wv=0x40000000,
           wo=0x50000000, y=0x60000000, B=2, Tq=100, Tk=100, dm=512, h=8, scale=0.125, mask_kind=0,
           key_lens=None, ws=0x80000000, ws_bytes=1 << 28, stream=None)


def _call_mha(L, **over):
    a = dict(MHA)
    a.update(over)
    return L.attn_mha_fwd(a["xq"], a["xk"], a["xv"], a["wq"], a["wk"], a["wv"], a["wo"], a["y"], a["B"], a["Tq"],
                          a["Tk"], a["dm"], a["h"], a["scale"], a["mask_kind"], a["key_lens"], a["ws"],
                          a["ws_bytes"], a["stream"])


def test_mha_workspace_size(L):
    assert L.attn_mha_workspace_bytes(-1, 10, 10, 512) == 0
    assert L.attn_mha_workspace_bytes(1, 10, 10, 0) == 0
    n = L.attn_mha_workspace_bytes(2, 100, 100, 512)
    # the four transposed weights, the projected q, k, v rows and the attention output (bf16)
    assert n == 4 * 512 * 512 * 2 + 2 * (100 + 2 * 100) * 512 * 2 + 2 * 100 * 512 * 2
    assert L.attn_mha_workspace_bytes(2, 100, 300, 512) > n


@pytest.mark.parametrize("over,code", [
    (dict(B=-1), "ERR_SHAPE"),
    (dict(h=0), "ERR_SHAPE"),
    (dict(h=3), "ERR_SHAPE"),                 # 512 % 3 != 0
    (dict(h=16), "ERR_HEADDIM"),              # d = 32
    (dict(dm=96, h=1), "ERR_HEADDIM"),
    (dict(mask_kind=4), "ERR_MASK"),
    (dict(mask_kind=2), "ERR_MASK"),
    (dict(scale=float("nan")), "ERR_SCALE"),
    (dict(wq=None), "ERR_NULL"),
    (dict(y=None), "ERR_NULL"),
    (dict(xk=None), "ERR_NULL"),
    (dict(ws=None), "ERR_WORKSPACE"),
    (dict(ws_bytes=4096), "ERR_WORKSPACE"),
    (dict(ws=0x80000010), "ERR_ALIGN"),       # the workspace needs 256 bytes
    (dict(wo=0x50000008), "ERR_ALIGN"),
    (dict(y=0x10000000 + 512), "ERR_ALIAS"),  # y inside xq
    (dict(ws=0x30000000), "ERR_ALIAS"),       # workspace on wk
    (dict(y=0x80000000 + 4096), "ERR_ALIAS"), # y inside the workspace
    (dict(mask_kind=2, key_lens=0x60000000 + 16), "ERR_ALIAS"),   # y overlaps key_lens
    (dict(mask_kind=2, key_lens=0x80000000 + 16), "ERR_ALIAS"),   # the workspace overlaps key_lens
    (dict(B=70000, Tq=40000, Tk=40000), "ERR_TOO_LARGE"),   # B T rows past 2^31 - 1
    (dict(Tq=1 << 21, Tk=1 << 21), "ERR_TOO_LARGE"),        # one head's projected rows past 4 GiB
])
def test_mha_bad_arguments_rejected_before_any_launch(L, over, code):
    assert _call_mha(L, **over) == getattr(L, code)
    assert L.attn_last_hip_error() == 0


def test_mha_empty_is_a_no_op(L):
    assert _call_mha(L, B=0, xq=None, y=None, ws=None) == L.OK
    assert _call_mha(L, Tq=0) == L.OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from transformer_scaled_dot_03_amd import _lib
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(_lib.LibraryMissing):
        _lib.attn_version()


def test_mfma_probe_library_exports_and_rejects_bad_arguments():
    """The benchmark's pure-MFMA probe library loads and validates before launching."""
    from transformer_scaled_dot_03_amd import build
    if not os.path.exists(build.PROBE_LIB_PATH):
        build.build()
    lib = ctypes.CDLL(build.PROBE_LIB_PATH)
    header = open(os.path.join(ROOT, "include", "mfma_probe.h")).read()
    header = re.sub(r"/\*.*?\*/", "", header, flags=re.S)
    for name in set(re.findall(r"\b(mfma_probe_\w+)\s*\(", header)):
        assert hasattr(lib, name), name
    fn = lib.mfma_probe_launch
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    assert fn(None, 0x1000, 4, 4, None) == -1
    assert fn(0x1000, None, 4, 4, None) == -1
    assert fn(0x1000, 0x2000, 0, 4, None) == -1
    assert fn(0x1000, 0x2000, 4, 0, None) == -1
