"""The library's calls under HIP graph capture.

Every entry point only enqueues kernels on the caller's stream (no allocation,
no memset, no host synchronisation), so a caller can capture a sequence of
calls into a graph and replay it.  Each test captures one call into a
torch.cuda.CUDAGraph (inputs and outputs allocated before the capture), then
replays it several times with unrelated eager work and synchronisations in
between, and checks every replay bitwise against the eager result of the same
call on the same inputs.
"""
from __future__ import annotations

import pytest
import torch

from transformer_scaled_dot_03_amd.workloads import grad_output, mha_inputs, random_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REPLAYS = 4


@pytest.fixture(scope="module")
def tsd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_scaled_dot_03_amd as m
    m.raw_library()  # fail loudly if the HIP library is missing
    return m


def _capture_and_replay(run, outs, eager):
    """run() writes into the tensors `outs`; eager: their expected values."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on the capturing stream, outside the graph
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    scratch = torch.empty(1 << 20, device=DEV)
    for i in range(REPLAYS):
        for o in outs:
            o.fill_(float("nan"))   # a replay that writes nothing is caught
        scratch.normal_()            # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, want in zip(outs, eager):
            assert torch.equal(o, want), f"replay {i} differs from the eager result"
        print(f"[graph] replay {i} bitwise equal", flush=True)


def test_forward_graph(tsd):
    q, k, v = (t.to(DEV) for t in random_inputs(2, 4, 333, 290, 128, dtype="bf16", seed=21))
    kl = torch.tensor([290, 117], dtype=torch.int32, device=DEV)
    want = tsd.attention(q, k, v, causal=True, key_lens=kl)
    out = torch.empty_like(q)
    _capture_and_replay(lambda: tsd.attention(q, k, v, causal=True, key_lens=kl, out=out), [out], [want])


def test_backward_graph(tsd):
    q, k, v = (t.to(DEV) for t in random_inputs(2, 3, 200, 150, 64, dtype="bf16", seed=22))
    g = grad_output(2, 3, 200, 64, seed=22).to(DEV)
    o, lse = tsd.attention_lse(q, k, v, causal=True)
    want = tsd.attention_backward(q, k, v, o, g, lse, causal=True)
    dq, dk, dv = (torch.empty_like(t) for t in (q, k, v))
    delta = torch.empty((2, 2, 3, 200), dtype=torch.float32, device=DEV)
    _capture_and_replay(lambda: tsd.attention_backward(q, k, v, o, g, lse, causal=True, dq=dq, dk=dk, dv=dv,
                                                       delta=delta),
                        [dq, dk, dv], list(want))


def test_decode_graph(tsd):
    q, k, v = (t.to(DEV) for t in random_inputs(3, 4, 1, 5000, 128, dtype="bf16", seed=23))
    kl = torch.tensor([5000, 1, 2047], dtype=torch.int32, device=DEV)
    want = tsd.decode_attention(q, k, v, key_lens=kl)
    out = torch.empty_like(q)
    ws = torch.empty(tsd.attn_decode_workspace_bytes(3, 4, 5000, 128), dtype=torch.uint8, device=DEV)
    _capture_and_replay(lambda: tsd.decode_attention(q, k, v, key_lens=kl, out=out, workspace=ws), [out], [want])


def test_multi_head_graph(tsd):
    xq, xk, xv, wq, wk, wv, wo = (t.to(DEV) for t in mha_inputs(2, 300, 300, 512, seed=24))
    want = tsd.multi_head_attention(xq, wq, wk, wv, wo, 8)
    y = torch.empty_like(want)
    ws = torch.empty(tsd.attn_mha_workspace_bytes(2, 300, 300, 512), dtype=torch.uint8, device=DEV)
    _capture_and_replay(lambda: tsd.multi_head_attention(xq, wq, wk, wv, wo, 8, out=y, workspace=ws), [y], [want])
