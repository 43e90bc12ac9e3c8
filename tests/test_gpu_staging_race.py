"""Race check of the direct-to-LDS staging of every pipelined kernel (GPU).

The shipped kernels overlap the direct-to-LDS loads of later tiles with the
reads of the current ones (double buffering, one barrier per step): the bf16
forward (K/V tiles), the backward's dQ kernel (K/V tiles) and dK/dV kernel
(Q/dO tiles with their lse and D), the weights kernel (K tiles) and the
projection GEMM of the multi-head call (A and B^T tiles).
libattn_serial_test.so is the same source built with the loads of every step
waited for before the step reads LDS, so no load is ever in flight while a
tile is read: it cannot race.  If a pipelined kernel read a tile before its
load landed, or a load overwrote a tile still being read, its output would
differ from the serial build's; both must agree bit for bit.  Shapes are
ragged (partial key tiles, a partial last query tile, key padding, causal
diagonals, GEMM row blocks and column tiles past the matrix edge, an odd
number of 64-wide k steps) so every pipeline edge runs.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import pytest
import torch

from transformer_scaled_dot_03_amd.workloads import random_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SERIAL = os.path.join(ROOT, "transformer_scaled_dot_03_amd", "libattn_serial_test.so")


@pytest.fixture(scope="module")
def libs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from transformer_scaled_dot_03_amd import _lib
    if not os.path.exists(SERIAL):
        pytest.fail("libattn_serial_test.so is not built (python -m transformer_scaled_dot_03_amd.build)")
    serial = ctypes.CDLL(SERIAL)
    for name in ("attn_fwd", "attn_fwd_lse", "attn_bwd", "attn_fwd_weights", "attn_mha_fwd",
                 "attn_mha_workspace_bytes"):
        res, args = _lib.SIGNATURES[name]
        fn = getattr(serial, name)
        fn.restype, fn.argtypes = res, args
    return _lib.raw_library(), serial


CASES = [
    # (B, h, Tq, Tk, d, causal, key_lens)
    (1, 2, 300, 333, 64, False, None),
    (1, 2, 333, 300, 128, False, None),
    (2, 3, 257, 1000, 64, False, [1000, 77]),
    (2, 2, 513, 513, 128, True, None),
    (2, 3, 300, 300, 64, True, [300, 130]),
    (1, 1, 1, 4097, 128, False, None),
    (3, 2, 129, 65, 64, True, None),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}h{}q{}k{}d{}-c{}-kl{}".format(*c))
def test_pipelined_forward_equals_serial_staging(libs, case):
    fast, serial = libs
    B, h, Tq, Tk, d, causal, key_lens = case
    print(f"[staging race] {case}", flush=True)
    q, k, v = (t.to(DEV) for t in random_inputs(B, h, Tq, Tk, d, seed=Tq + Tk + d))
    kl = None if key_lens is None else torch.tensor(key_lens, dtype=torch.int32, device=DEV)
    mask = (1 if causal else 0) | (2 if kl is not None else 0)
    st = torch.cuda.current_stream().cuda_stream
    outs, lses = [], []
    for lib in (fast, serial):
        out = torch.full_like(q, float("nan"))
        lse = torch.full((B, h, Tq), float("nan"), dtype=torch.float32, device=DEV)
        rc = lib.attn_fwd_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, h, Tq,
                              Tk, d, d, float(np.float32(d ** -0.5)), mask,
                              None if kl is None else kl.data_ptr(), st)
        assert rc == 0
        outs.append(out)
        lses.append(lse)
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), "output differs from serial staging"
    assert torch.equal(lses[0].view(torch.int32), lses[1].view(torch.int32)), "lse differs from serial staging"


BWD_CASES = [
    # (B, h, Tq, Tk, d, causal, key_lens)
    (1, 2, 300, 333, 64, False, None),
    (1, 2, 333, 300, 128, False, None),
    (2, 2, 257, 700, 128, False, [700, 77]),
    (2, 2, 513, 513, 128, True, None),
    (2, 3, 300, 300, 64, True, [300, 130]),
    (1, 2, 129, 65, 128, True, None),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "B{}h{}q{}k{}d{}-c{}-kl{}".format(*c))
def test_pipelined_backward_equals_serial_staging(libs, case):
    from transformer_scaled_dot_03_amd.workloads import grad_output
    fast, serial = libs
    B, h, Tq, Tk, d, causal, key_lens = case
    print(f"[staging race, backward] {case}", flush=True)
    q, k, v = (t.to(DEV) for t in random_inputs(B, h, Tq, Tk, d, seed=Tq + Tk + d + 1))
    dout = grad_output(B, h, Tq, d, seed=Tq).to(DEV)
    kl = None if key_lens is None else torch.tensor(key_lens, dtype=torch.int32, device=DEV)
    klp = None if kl is None else kl.data_ptr()
    mask = (1 if causal else 0) | (2 if kl is not None else 0)
    scale = float(np.float32(d ** -0.5))
    st = torch.cuda.current_stream().cuda_stream
    out = torch.empty_like(q)
    lse = torch.empty((B, h, Tq), dtype=torch.float32, device=DEV)
    assert fast.attn_fwd_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, h, Tq, Tk,
                             d, d, scale, mask, klp, st) == 0
    results = []
    for lib in (fast, serial):
        delta = torch.full((2, B, h, Tq), float("nan"), dtype=torch.float32, device=DEV)
        dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
        rc = lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                          delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, h, Tq, Tk, d, d, scale,
                          mask, klp, st)
        assert rc == 0
        results.append((dq, dk, dv, delta))
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), results[0][:3], results[1][:3]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name} differs from serial staging"
    assert torch.equal(results[0][3].view(torch.int32), results[1][3].view(torch.int32)), "delta differs"


WEIGHT_CASES = [
    (1, 2, 200, 333, 64, False, None),
    (2, 2, 257, 300, 128, True, None),
    (2, 2, 130, 200, 64, False, [200, 61]),
]


@pytest.mark.parametrize("case", WEIGHT_CASES, ids=lambda c: "B{}h{}q{}k{}d{}-c{}-kl{}".format(*c))
def test_pipelined_weights_equal_serial_staging(libs, case):
    fast, serial = libs
    B, h, Tq, Tk, d, causal, key_lens = case
    print(f"[staging race, weights] {case}", flush=True)
    q, k, v = (t.to(DEV) for t in random_inputs(B, h, Tq, Tk, d, seed=Tq + Tk + d + 2))
    kl = None if key_lens is None else torch.tensor(key_lens, dtype=torch.int32, device=DEV)
    mask = (1 if causal else 0) | (2 if kl is not None else 0)
    st = torch.cuda.current_stream().cuda_stream
    ws = []
    for lib in (fast, serial):
        out = torch.empty_like(q)
        lse = torch.empty((B, h, Tq), dtype=torch.float32, device=DEV)
        w = torch.full((B, h, Tq, Tk), float("nan"), dtype=torch.float32, device=DEV)
        rc = lib.attn_fwd_weights(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                  w.data_ptr(), B, h, Tq, Tk, d, d, float(np.float32(d ** -0.5)), mask,
                                  None if kl is None else kl.data_ptr(), st)
        assert rc == 0
        ws.append(w)
    torch.cuda.synchronize()
    assert torch.equal(ws[0].view(torch.int32), ws[1].view(torch.int32)), "weights differ from serial staging"


MHA_CASES = [
    # (B, Tq, Tk, d_model, heads, cross): the GEMM's last row block and column tile partly past the matrix,
    # an odd number of 64-wide k steps (d_model 320, 192), more tiles than CUs (B 16, T 1024: 384 QKV tiles)
    (2, 130, 130, 320, 5, False),
    (2, 77, 200, 192, 3, True),
    (16, 1024, 1024, 512, 8, False),
    (3, 300, 300, 256, 2, False),
]


@pytest.mark.parametrize("case", MHA_CASES, ids=lambda c: "B{}q{}k{}dm{}h{}-x{}".format(*c))
def test_pipelined_gemm_equals_serial_staging(libs, case):
    from transformer_scaled_dot_03_amd.workloads import mha_inputs
    fast, serial = libs
    B, Tq, Tk, dm, heads, cross = case
    print(f"[staging race, multi-head GEMM] {case}", flush=True)
    xq, xk, xv, wq, wk, wv, wo = (t.to(DEV) for t in mha_inputs(B, Tq, Tk, dm, seed=5, cross=cross))
    st = torch.cuda.current_stream().cuda_stream
    nbytes = fast.attn_mha_workspace_bytes(B, Tq, Tk, dm)
    assert nbytes > 0
    ys = []
    for lib in (fast, serial):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        y = torch.full((B, Tq, dm), float("nan"), dtype=torch.bfloat16, device=DEV)
        rc = lib.attn_mha_fwd(xq.data_ptr(), xk.data_ptr(), xv.data_ptr(), wq.data_ptr(), wk.data_ptr(),
                              wv.data_ptr(), wo.data_ptr(), y.data_ptr(), B, Tq, Tk, dm, heads,
                              float(np.float32((dm // heads) ** -0.5)), 0, None, ws.data_ptr(), nbytes, st)
        assert rc == 0
        ys.append(y)
    torch.cuda.synchronize()
    assert torch.equal(ys[0].view(torch.int16), ys[1].view(torch.int16)), "multi-head output differs from serial staging"
