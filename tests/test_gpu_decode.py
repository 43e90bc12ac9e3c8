"""GPU parity of single-row decode attention (attn_decode) against the fp64 oracle.

The oracle is attention_fp64 with Tq = 1 (the plain definition; no causal
mask: the newest position sees the whole valid cache).  Tolerances are the
bf16 ones of the forward (tests/parity.py): max |Δ| <= 2e-2 and per-row
||Δ||/||ref|| <= 1e-2; the decode path keeps the weights in fp32, so its
errors are smaller than the forward's.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import attention_fp64
from tests.parity import assert_parity
from transformer_scaled_dot_03_amd.workloads import WORKLOADS, make_inputs, random_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def tsd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_scaled_dot_03_amd as m
    m.raw_library()  # fail loudly if the HIP library is missing
    return m


def _f32(t):
    return t.float().cpu().numpy()


def _decode(tsd, q, k, v, scale, key_lens=None, workspace=None):
    kl = None if key_lens is None else torch.as_tensor(key_lens, dtype=torch.int32).to(DEV)
    out = tsd.decode_attention(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale, key_lens=kl, workspace=workspace)
    torch.cuda.synchronize()
    return out


def _check(tsd, q, k, v, scale, key_lens, what):
    out = _decode(tsd, q, k, v, scale, key_lens)
    kl = None if key_lens is None else np.asarray(key_lens)
    want = attention_fp64(_f32(q), _f32(k), _f32(v), scale, key_lens=kl)
    err = assert_parity(_f32(out), want, "bf16", what)
    print(f"[decode parity] {what}: max abs {err[0]:.3e}, max row rel {err[1]:.3e}", flush=True)
    return out


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Tk", [1, 63, 64, 255, 256, 257, 1000, 4097])
@pytest.mark.parametrize("keypad", [False, True])
def test_decode_cache_lengths(tsd, d, Tk, keypad):
    q, k, v = random_inputs(2, 3, 1, Tk, d, seed=Tk + d)
    key_lens = [max(Tk // 3, 1), Tk + 7] if keypad else None   # one clamped above Tk
    _check(tsd, q, k, v, float(np.float32(d ** -0.5)), key_lens, f"decode d{d} Tk{Tk} keypad={keypad}")


@pytest.mark.parametrize("d", [64, 128])
def test_decode_empty_caches_give_zeros(tsd, d):
    q, k, v = random_inputs(4, 2, 1, 300, d, seed=3)
    out = _check(tsd, q, k, v, 0.1, [0, 300, 1, 0], f"decode lengths d{d}")
    assert not out[0].any() and not out[3].any()
    q, k, v = random_inputs(2, 2, 1, 0, d, seed=4)
    assert not _decode(tsd, q, k, v, 0.1).any()


def test_decode_many_splits(tsd):
    """A 200000-entry cache: hundreds of split work-groups merged per head."""
    q, k, v = random_inputs(1, 2, 1, 200000, 64, seed=5)
    _check(tsd, q, k, v, 0.125, None, "decode Tk200000")
    _check(tsd, q, k, v, 0.125, [123457], "decode Tk200000 L123457")


@pytest.mark.parametrize("scale", [-0.3, 0.0, 2.0])
def test_decode_scale_sign_zero_and_peaked(tsd, scale):
    q, k, v = random_inputs(2, 2, 1, 777, 128, seed=6, qk_mul=3.0)
    _check(tsd, q, k, v, scale, None, f"decode scale {scale}")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["decode_bf16_b8h16k16384d128", "decode_keypad_bf16_b64h8k4096d64"])
def test_decode_workload_full(tsd, name):
    w = WORKLOADS[name]
    print(f"[decode parity] start {name}", flush=True)
    q, k, v, kl = make_inputs(w, seed=0)
    _check(tsd, q, k, v, w.scale, None if kl is None else kl.numpy(), name)


def test_decode_workspace_reuse_and_guards(tsd):
    """One workspace serves calls of different sizes; nothing is written outside out and it."""
    need = max(tsd.attn_decode_workspace_bytes(3, 4, 5000, 128), tsd.attn_decode_workspace_bytes(1, 2, 70, 64))
    pad = 4096
    ws_buf = torch.full((need + 2 * pad,), 0x5A, dtype=torch.uint8, device=DEV)
    ws = ws_buf[pad:pad + need]
    for (B, H, Tk, d) in ((3, 4, 5000, 128), (1, 2, 70, 64)):
        q, k, v = random_inputs(B, H, 1, Tk, d, seed=B * Tk)
        ob = torch.full((B * H * d + 2 * pad,), 3.0, dtype=torch.bfloat16, device=DEV)
        out = ob[pad:pad + B * H * d].view(B, H, 1, d)
        tsd.decode_attention(q.to(DEV), k.to(DEV), v.to(DEV), scale=0.1, out=out, workspace=ws)
        torch.cuda.synchronize()
        want = attention_fp64(_f32(q), _f32(k), _f32(v), 0.1)
        assert_parity(_f32(out), want, "bf16", f"decode reuse B{B} Tk{Tk}")
        assert torch.all(ob[:pad] == 3.0) and torch.all(ob[-pad:] == 3.0)
        assert torch.all(ws_buf[:pad] == 0x5A) and torch.all(ws_buf[-pad:] == 0x5A)


def test_decode_deterministic_and_rejects_small_workspace(tsd):
    q, k, v = (t.to(DEV) for t in random_inputs(2, 4, 1, 3000, 128, seed=7))
    a = tsd.decode_attention(q, k, v, scale=0.1)
    b = tsd.decode_attention(q, k, v, scale=0.1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    small = torch.empty(64, dtype=torch.uint8, device=DEV)
    with pytest.raises(tsd.AttentionError) as e:
        tsd.decode_attention(q, k, v, scale=0.1, workspace=small)
    assert e.value.status == tsd.ERR_WORKSPACE
