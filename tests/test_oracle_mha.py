"""Pins for the oracle's multi-head attention (test infrastructure).

multi_head_attention_fp64 is pinned against PyTorch's own multi-head attention
routine (torch.nn.functional.multi_head_attention_forward, float64, no biases)
under every mask combination, against closed forms (one head with identity
projections is plain attention; a zero W^O gives zeros), against head
permutation invariance, and against a planted mistake (the heads' column
blocks taken in the wrong order of the reshape).
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import attention_fp64, multi_head_attention_fp64


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _weights(dm, h, d, seed):
    return (_rand((dm, h * d), seed, dm ** -0.5), _rand((dm, h * d), seed + 1, dm ** -0.5),
            _rand((dm, h * d), seed + 2, dm ** -0.5), _rand((h * d, dm), seed + 3, (h * d) ** -0.5))


@pytest.mark.parametrize("causal,key_lens", [(False, None), (True, None), (False, [5, 9]), (True, [9, 3])])
def test_matches_torch_multi_head_attention(causal, key_lens):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    B, T, dm, h = 2, 9, 12, 3
    d = dm // h
    x = _rand((B, T, dm), 1)
    wq, wk, wv, wo = _weights(dm, h, d, 2)
    y = multi_head_attention_fp64(x, x, x, wq, wk, wv, wo, h, 1.0 / np.sqrt(d), causal=causal, key_lens=key_lens)
    xt = torch.tensor(x).transpose(0, 1)                     # torch wants [T, B, E]
    in_w = torch.tensor(np.concatenate([wq.T, wk.T, wv.T]))  # torch computes x @ W^T
    attn_mask = torch.triu(torch.ones(T, T, dtype=torch.bool), 1) if causal else None
    kpm = None
    if key_lens is not None:
        kpm = torch.arange(T)[None, :] >= torch.tensor(key_lens)[:, None]   # True = ignore
    out, _ = F.multi_head_attention_forward(
        xt, xt, xt, dm, h, in_w, None, None, None, False, 0.0, torch.tensor(wo.T), None,
        training=False, key_padding_mask=kpm, need_weights=False, attn_mask=attn_mask)
    np.testing.assert_allclose(y, out.transpose(0, 1).numpy(), rtol=0, atol=1e-12)


def test_cross_attention_with_distinct_inputs_matches_torch():
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    B, Tq, Tk, dm, h = 2, 5, 7, 8, 2
    d = dm // h
    xq, xk, xv = _rand((B, Tq, dm), 3), _rand((B, Tk, dm), 4), _rand((B, Tk, dm), 5)
    wq, wk, wv, wo = _weights(dm, h, d, 6)
    y = multi_head_attention_fp64(xq, xk, xv, wq, wk, wv, wo, h, 1.0 / np.sqrt(d))
    out, _ = F.multi_head_attention_forward(
        torch.tensor(xq).transpose(0, 1), torch.tensor(xk).transpose(0, 1), torch.tensor(xv).transpose(0, 1),
        dm, h, None, None, None, None, False, 0.0, torch.tensor(wo.T), None, training=False,
        need_weights=False, use_separate_proj_weight=True, q_proj_weight=torch.tensor(wq.T),
        k_proj_weight=torch.tensor(wk.T), v_proj_weight=torch.tensor(wv.T))
    np.testing.assert_allclose(y, out.transpose(0, 1).numpy(), rtol=0, atol=1e-12)


def test_closed_forms():
    B, T, dm = 2, 6, 4
    x = _rand((B, T, dm), 7)
    eye = np.eye(dm)
    # one head, identity projections: plain attention of x with itself
    y = multi_head_attention_fp64(x, x, x, eye, eye, eye, eye, 1, 0.3, causal=True, key_lens=[6, 2])
    want = attention_fp64(x[:, None], x[:, None], x[:, None], 0.3, causal=True, key_lens=[6, 2])[:, 0]
    np.testing.assert_allclose(y, want, rtol=0, atol=1e-14)
    # zero output projection
    wq, wk, wv, _ = _weights(dm, 2, 2, 8)
    assert not multi_head_attention_fp64(x, x, x, wq, wk, wv, np.zeros((4, dm)), 2, 0.5).any()


def test_head_permutation_invariance_and_row_subset():
    B, T, dm, h = 1, 8, 12, 3
    d = dm // h
    x = _rand((B, T, dm), 9)
    wq, wk, wv, wo = _weights(dm, h, d, 10)
    y = multi_head_attention_fp64(x, x, x, wq, wk, wv, wo, h, 0.4)
    perm = [2, 0, 1]
    cols = np.concatenate([np.arange(p * d, p * d + d) for p in perm])
    y2 = multi_head_attention_fp64(x, x, x, wq[:, cols], wk[:, cols], wv[:, cols], wo[cols], h, 0.4)
    np.testing.assert_allclose(y, y2, rtol=0, atol=1e-12)
    rows = np.array([0, 3, 7])
    np.testing.assert_allclose(multi_head_attention_fp64(x, x, x, wq, wk, wv, wo, h, 0.4, rows=rows),
                               y[:, rows], rtol=0, atol=1e-14)


def test_planted_head_split_mistake_is_caught():
    """Splitting the projected row as (d, h) instead of (h, d) changes the result."""
    B, T, dm, h = 1, 5, 8, 2
    d = dm // h
    x = _rand((B, T, dm), 11)
    wq, wk, wv, wo = _weights(dm, h, d, 12)
    y = multi_head_attention_fp64(x, x, x, wq, wk, wv, wo, h, 0.5)
    # the mistake: head i takes columns i, i + h, i + 2h, ... (a (d, h) reshape)
    cols = np.concatenate([np.arange(i, dm, h) for i in range(h)])
    wrong = multi_head_attention_fp64(x, x, x, wq[:, cols], wk[:, cols], wv[:, cols], wo, h, 0.5)
    assert not np.allclose(y, wrong, atol=1e-6)
