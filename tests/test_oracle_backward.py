"""Pins for the oracle's log-sum-exp and gradients (test infrastructure).

The gradient formulas are derived by the chain rule; they are pinned here
against things other than themselves: central finite differences of the
forward oracle on tiny inputs (which catch any dropped scale, sign or
transposition), the pages' PyTorch formula differentiated by torch.autograd in
float64, closed forms and invariants.  The log-sum-exp is pinned by
scipy.special.logsumexp and closed forms.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
from oracle import attention_backward_fp64, attention_backward_sampled_fp64, attention_fp64, attention_lse_fp64


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _loss(q, k, v, g, scale, causal, key_lens):
    """L = sum(dO * O): its gradient with respect to O is dO."""
    return float((attention_fp64(q, k, v, scale, causal=causal, key_lens=key_lens) * g).sum())


def _fd_grad(f, x, h=1e-6):
    grad = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        old = x[idx]
        x[idx] = old + h
        fp = f()
        x[idx] = old - h
        fm = f()
        x[idx] = old
        grad[idx] = (fp - fm) / (2 * h)
    return grad


@pytest.mark.parametrize("causal,key_lens", [(False, None), (True, None), (False, [2, 4]), (True, [3, 1])])
def test_gradients_match_finite_differences(causal, key_lens):
    B, H, Tq, Tk, d = 2, 1, 4, 5, 3
    q, k, v, g = _rand((B, H, Tq, d), 1), _rand((B, H, Tk, d), 2), _rand((B, H, Tk, d), 3), _rand((B, H, Tq, d), 4)
    scale = 0.7
    dq, dk, dv, _ = attention_backward_fp64(q, k, v, g, scale, causal=causal, key_lens=key_lens)
    f = lambda: _loss(q, k, v, g, scale, causal, key_lens)
    np.testing.assert_allclose(dq, _fd_grad(f, q), rtol=0, atol=2e-8)
    np.testing.assert_allclose(dk, _fd_grad(f, k), rtol=0, atol=2e-8)
    np.testing.assert_allclose(dv, _fd_grad(f, v), rtol=0, atol=2e-8)


def test_gradients_match_torch_autograd_of_the_pages_formula():
    """cuijiawei.cn snippet (q @ k^T / sqrt(d_k), masked_fill, softmax, @ v) in float64, differentiated."""
    torch = pytest.importorskip("torch")
    B, H, Tq, Tk, d = 2, 2, 9, 11, 8
    q, k, v, g = _rand((B, H, Tq, d), 5), _rand((B, H, Tk, d), 6), _rand((B, H, Tk, d), 7), _rand((B, H, Tq, d), 8)
    L = [7, 11]
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    mask = torch.ones(B, 1, Tq, Tk, dtype=torch.bool) & torch.tril(torch.ones(Tq, Tk, dtype=torch.bool))
    for b in range(B):
        mask[b, :, :, L[b]:] = False
    scores = (tq @ tk.transpose(-2, -1) / d ** 0.5).masked_fill(mask == 0, float("-inf"))
    out = torch.softmax(scores, dim=-1) @ tv
    out.backward(torch.tensor(g))
    dq, dk, dv, delta = attention_backward_fp64(q, k, v, g, 1.0 / d ** 0.5, causal=True, key_lens=L)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(delta, (g * out.detach().numpy()).sum(-1), rtol=0, atol=1e-12)


def test_key_gradients_sum_to_zero_and_shift_invariance():
    """Each row of dS sums to zero, so sum_j dK_j = 0; adding c to every key leaves dQ unchanged."""
    q, k, v, g = _rand((1, 2, 12, 6), 9), _rand((1, 2, 10, 6), 10), _rand((1, 2, 10, 6), 11), _rand((1, 2, 12, 6), 12)
    for causal in (False, True):
        dq, dk, _, _ = attention_backward_fp64(q, k, v, g, 0.4, causal=causal, key_lens=[8])
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
        c = _rand((6,), 13, 3.0)
        dq2, _, _, _ = attention_backward_fp64(q, k + c, v, g, 0.4, causal=causal, key_lens=[8])
        np.testing.assert_allclose(dq, dq2, rtol=0, atol=1e-12)


def test_gradient_closed_forms():
    q, k, v = _rand((1, 1, 6, 4), 14), _rand((1, 1, 1, 4), 15), _rand((1, 1, 1, 4), 16)
    g = _rand((1, 1, 6, 4), 17)
    # one key: weights are all 1, so dQ = dK = 0 and dV = sum of dO rows
    dq, dk, dv, _ = attention_backward_fp64(q, k, v, g, 0.9)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_allclose(dv[0, 0, 0], g[0, 0].sum(axis=0), atol=1e-14)
    # zero upstream gradient: all gradients vanish
    q, k, v = _rand((1, 1, 5, 4), 18), _rand((1, 1, 7, 4), 19), _rand((1, 1, 7, 4), 20)
    dq, dk, dv, delta = attention_backward_fp64(q, k, v, np.zeros((1, 1, 5, 4)), 0.9, causal=True)
    assert not dq.any() and not dk.any() and not dv.any() and not delta.any()
    # masked keys (past the length) receive no gradient; empty rows give dQ = 0
    g = _rand((2, 1, 5, 4), 21)
    q2, k2, v2 = _rand((2, 1, 5, 4), 22), _rand((2, 1, 7, 4), 23), _rand((2, 1, 7, 4), 24)
    dq, dk, dv, _ = attention_backward_fp64(q2, k2, v2, g, 0.9, key_lens=[3, 0])
    assert np.all(dk[0, :, 3:] == 0) and np.all(dv[0, :, 3:] == 0)
    assert np.all(dq[1] == 0) and np.all(dk[1] == 0) and np.all(dv[1] == 0)


def test_lse_matches_scipy_logsumexp_and_closed_forms():
    q, k = _rand((2, 2, 7, 5), 25), _rand((2, 2, 9, 5), 26)
    v = _rand((2, 2, 9, 5), 27)
    for causal, kl in ((False, None), (True, [9, 4])):
        _, lse = attention_lse_fp64(q, k, v, 0.45, causal=causal, key_lens=kl)
        for b in range(2):
            for h in range(2):
                for i in range(7):
                    ok = oracle.allowed_mask(np.array([i]), 9, causal, None if kl is None else kl[b])[0]
                    s = (q[b, h, i] @ k[b, h].T) * 0.45
                    assert abs(lse[b, h, i] - logsumexp(s[ok])) < 1e-12
    # equal scores: lse = s + log(n); one key: lse = its score; no key: -inf
    _, lse = attention_lse_fp64(np.zeros((1, 1, 3, 2)), _rand((1, 1, 6, 2), 28), _rand((1, 1, 6, 2), 29), 1.0,
                                key_lens=[4])
    np.testing.assert_allclose(lse, math.log(4), atol=1e-15)
    qq, kk = _rand((1, 1, 2, 3), 30), _rand((1, 1, 1, 3), 31)
    _, lse = attention_lse_fp64(qq, kk, kk, 2.0)
    np.testing.assert_allclose(lse[0, 0], 2.0 * (qq[0, 0] @ kk[0, 0, 0]), atol=1e-14)
    _, lse = attention_lse_fp64(qq, kk, kk, 2.0, key_lens=[0])
    assert np.all(lse == -np.inf)
    # a row subset gives the same rows as the full computation
    out_f, lse_f = attention_lse_fp64(q, k, v, 0.45, causal=True, key_lens=[9, 4], block=3)
    rows = np.array([0, 4, 6])
    out_r, lse_r = attention_lse_fp64(q, k, v, 0.45, causal=True, key_lens=[9, 4], rows=rows, block=2)
    np.testing.assert_allclose(lse_r, lse_f[:, :, rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(out_r, out_f[:, :, rows], rtol=0, atol=1e-14)


@pytest.mark.parametrize("kind", ["no_scale", "sign", "delta_from_dp", "no_transpose"])
def test_planted_gradient_mistakes_fail_finite_differences(kind, monkeypatch):
    orig = oracle.attention.attention_backward_fp64

    def mutant(q, k, v, dout, scale, causal=False, key_lens=None):
        dq, dk, dv, delta = orig(q, k, v, dout, scale, causal=causal, key_lens=key_lens)
        if kind == "no_scale":
            return dq / scale, dk, dv, delta
        if kind == "sign":
            return -dq, dk, dv, delta
        if kind == "delta_from_dp":
            return dq, dk * 1.5, dv, delta
        return dq, dk, dv[:, :, ::-1], delta

    B, H, Tq, Tk, d = 1, 1, 4, 4, 3
    q, k, v, g = _rand((B, H, Tq, d), 32), _rand((B, H, Tk, d), 33), _rand((B, H, Tk, d), 34), _rand((B, H, Tq, d), 35)
    dq, dk, dv, _ = mutant(q, k, v, g, 0.7)
    f = lambda: _loss(q, k, v, g, 0.7, False, None)
    ok = (np.allclose(dq, _fd_grad(f, q), atol=1e-6) and np.allclose(dk, _fd_grad(f, k), atol=1e-6)
          and np.allclose(dv, _fd_grad(f, v), atol=1e-6))
    assert not ok


@pytest.mark.parametrize("causal,key_lens", [(False, None), (True, None), (False, [40, 0]), (True, [70, 13])])
def test_sampled_gradients_equal_the_full_ones(causal, key_lens):
    """The blocked, sampled form (for long sequences) reduces to the whole-matrix one, which the
    finite-difference and autograd pins above fix."""
    B, H, Tq, Tk, d = 2, 2, 75, 83, 5
    q, k, v, g = _rand((B, H, Tq, d), 40), _rand((B, H, Tk, d), 41), _rand((B, H, Tk, d), 42), _rand((B, H, Tq, d), 43)
    dq, dk, dv, _ = attention_backward_fp64(q, k, v, g, 0.6, causal=causal, key_lens=key_lens)
    rows = np.array([0, 3, 31, 32, 74])
    keys = np.array([0, 1, 12, 39, 40, 69, 82])
    sq, sk, sv = attention_backward_sampled_fp64(q, k, v, g, 0.6, causal=causal, key_lens=key_lens, rows=rows,
                                                 keys=keys, block=16)
    np.testing.assert_allclose(sq, dq[:, :, rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(sk, dk[:, :, keys], rtol=0, atol=1e-12)
    np.testing.assert_allclose(sv, dv[:, :, keys], rtol=0, atol=1e-12)
    # a head subset leaves the others zero
    sq, sk, _ = attention_backward_sampled_fp64(q, k, v, g, 0.6, causal=causal, key_lens=key_lens, rows=rows,
                                                keys=keys, heads=[(1, 0)])
    np.testing.assert_allclose(sq[1, 0], dq[1, 0, rows], rtol=0, atol=1e-12)
    assert not sq[0].any() and not sk[0].any() and not sq[1, 1].any()
