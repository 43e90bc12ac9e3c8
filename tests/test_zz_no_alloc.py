"""GPU check of attn_decode_static, the decode entry point that allocates nothing.

attn_decode_static runs the kernels of attn_decode with the per-split partials
in the library's static device array instead of a caller workspace.  Through
the C ABI, each call is compared with attn_decode on the same inputs (the same
kernels and split sizes: bitwise equal) and with the fp64 oracle at the bf16
decode tolerance (tests/parity.py).  Two calls run back to back, the second
on a smaller problem, so the second must not see anything the first left in
the shared array; then the first problem runs again.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import attention_fp64
from tests.parity import assert_parity
from transformer_scaled_dot_03_amd.workloads import random_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from transformer_scaled_dot_03_amd import _lib
    _lib.raw_library()   # fail loudly if the HIP library is missing
    return _lib


def _case(B, h, Tk, d, key_lens, seed):
    q, k, v = random_inputs(B, h, 1, Tk, d, seed=seed)
    kl = None if key_lens is None else torch.tensor(key_lens, dtype=torch.int32)
    return q, k, v, kl


def _run_both(L, q, k, v, kl, scale):
    """(static result, workspace result), both through the C ABI on the current stream."""
    B, h, _, d = q.shape
    Tk = k.shape[2]
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    kld = None if kl is None else kl.to(DEV)
    mask = L.MASK_KEYPAD if kl is not None else L.MASK_NONE
    klp = None if kld is None else kld.data_ptr()
    st = torch.cuda.current_stream().cuda_stream
    out_s = torch.full_like(qd, float("nan"))
    out_w = torch.full_like(qd, float("nan"))
    nb = L.attn_decode_workspace_bytes(B, h, Tk, d)
    assert 0 < nb <= L.DECODE_STATIC_SCRATCH_BYTES
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    print(f"[no-alloc decode] B{B} h{h} Tk{Tk} d{d} keypad={kl is not None}", flush=True)
    rc = L.attn_decode_static(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out_s.data_ptr(), B, h, Tk, d, d,
                              scale, mask, klp, st)
    assert rc == L.OK, L.attn_status_str(rc)
    rc = L.attn_decode(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out_w.data_ptr(), B, h, Tk, d, d, scale, mask,
                       klp, ws.data_ptr(), nb, st)
    assert rc == L.OK, L.attn_status_str(rc)
    torch.cuda.synchronize()
    return out_s.float().cpu().numpy(), out_w.float().cpu().numpy()


def _check(L, B, h, Tk, d, key_lens, seed):
    q, k, v, kl = _case(B, h, Tk, d, key_lens, seed)
    scale = float(np.float32(d ** -0.5))
    got_s, got_w = _run_both(L, q, k, v, kl, scale)
    assert np.array_equal(got_s, got_w), "static-scratch decode differs from the workspace decode"
    want = attention_fp64(q.float().numpy(), k.float().numpy(), v.float().numpy(), scale,
                          key_lens=None if kl is None else kl.numpy())
    assert_parity(got_s, want, "bf16", f"static decode B{B} h{h} Tk{Tk} d{d}")


def test_decode_static_two_calls_second_smaller(L):
    # a large problem (many splits per head, ragged key padding), then a smaller one
    _check(L, 4, 8, 9000, 128, [9000, 5000, 1, 8999], seed=11)
    _check(L, 2, 3, 300, 64, None, seed=12)
    # and the large one again after the small one
    _check(L, 4, 8, 9000, 128, [9000, 5000, 1, 8999], seed=13)


def test_decode_static_at_the_size_limit(L):
    """A problem whose partials fill most of the static array (8 x 16 heads, 16384 keys, d 128)."""
    assert L.attn_decode_workspace_bytes(8, 16, 16384, 128) > L.DECODE_STATIC_SCRATCH_BYTES // 4
    _check(L, 8, 16, 16384, 128, None, seed=14)


def test_decode_static_rejects_over_the_limit_without_launching(L):
    B, h, Tk, d = 1024, 64, 1, 64
    assert L.attn_decode_workspace_bytes(B, h, Tk, d) > L.DECODE_STATIC_SCRATCH_BYTES
    q = torch.zeros((B, h, 1, d), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((B, h, Tk, d), dtype=torch.bfloat16, device=DEV)
    out = torch.zeros_like(q)
    rc = L.attn_decode_static(q.data_ptr(), kv.data_ptr(), kv.data_ptr(), out.data_ptr(), B, h, Tk, d, d, 0.125,
                              L.MASK_NONE, None, torch.cuda.current_stream().cuda_stream)
    assert rc == L.ERR_WORKSPACE
