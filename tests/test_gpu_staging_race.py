"""Race check of the forward's K/V staging (GPU).

The shipped bf16 forward overlaps the direct-to-LDS loads of later K/V tiles
with the reads of the current ones (double buffering, one barrier per step).
libattn_serial_test.so is the same source built with the loads of every step
waited for before the step reads LDS, so no load is ever in flight while a
tile is read: it cannot race.  If the pipelined kernel read a tile before its
load landed, or a load overwrote a tile still being read, its output would
differ from the serial build's; both must agree bit for bit.  Shapes are
ragged (partial key tiles, a partial last query tile, key padding, causal
diagonals) so every pipeline edge runs.
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
    for name in ("attn_fwd", "attn_fwd_lse"):
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
