"""Pins for the fp64 oracle: checks against what the pages and the mathematics fix.

Every check here compares the oracle with something other than its own
formula: values the pages print for worked examples (fixtures under
tests/golden/), closed forms, special cases that reduce to a library routine
(scipy's softmax, NumPy's mean / cumulative sum), invariants the pages state
(rows sum to one, masked weights are zero, order-blindness), and a scalar
brute force on tiny inputs.  Each is chosen so that a plausible slip in the
oracle (dropped scale, wrong sign, transposed operand, off-by-one mask, softmax
over the wrong axis, no max subtraction) fails at least one of them; the
planted-mistake tests at the end show that they do.
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest
from scipy.special import softmax as scipy_softmax

import oracle
from oracle import allowed_mask, attention_fp64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_fixture(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            vals[key] = [float(x) for x in rest]
    return vals


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _attn_single(q, k, v, scale, **kw):
    """Oracle on one (b, head): q [Tq, d], k [Tk, d], v [Tk, dv]."""
    kl = kw.pop("key_len", None)
    out = attention_fp64(q[None, None], k[None, None], v[None, None], scale,
                         key_lens=None if kl is None else [kl], **kw)
    return out


# --------------------------------------------------------------------------
# worked examples printed on the pages
# --------------------------------------------------------------------------

def test_three_score_softmax_example():
    """muhitai.com, "Step 4: Apply Softmax": [2.0, 1.0, 0.5] -> ~[0.63, 0.23, 0.14].

    With d_k = 1, scale 1, query 1 and keys equal to the scores, the scores are
    exactly [2, 1, 0.5]; with V = I the output row is the weight vector.
    """
    fx = _read_fixture("softmax_three_scores.txt")
    scores = np.array(fx["scores"])
    q = np.ones((1, 1))
    k = scores[:, None]
    v = np.eye(3)
    o = _attn_single(q, k, v, 1.0)[0, 0, 0]
    np.testing.assert_array_equal(np.round(o, 2), np.array(fx["weights"]))


def test_two_word_example():
    """aiany.app Step 5: scaled scores 12 vs 10 -> weights ~0.88 / 0.12, = 1/(1+e^-2).

    Raw dot products 96 and 80 over d_k = 64, divided by 8 (= sqrt(64)) as the
    page does, give the printed scores; this pins the scale as a division by
    sqrt(d_k) (without it the weight would be 1/(1+e^-16)).
    """
    fx = _read_fixture("two_word_scores.txt")
    dk = int(fx["d_k"][0])
    s1, s2 = fx["scores"]
    scale = 1.0 / math.sqrt(dk)
    q = np.ones((1, dk))
    k = np.stack([np.full(dk, s1 / (dk * scale)), np.full(dk, s2 / (dk * scale))])
    assert (q @ k.T)[0].tolist() == [96.0, 80.0]
    o = _attn_single(q, k, np.eye(2), scale)[0, 0, 0]
    np.testing.assert_array_equal(np.round(o, 2), np.array(fx["weights"]))
    # the page's own closed form 1/(1+e^-2)
    assert abs(o[0] - 1.0 / (1.0 + math.exp(-2.0))) < 1e-15
    assert abs(o[0] - 0.8807970779778823) < 1e-15


def test_equal_scores_split_evenly_and_gap_of_four_dominates():
    """aiany.app Step 5 ("Drag the scores"): equal scores -> 50/50; gap of 4+ -> winner ~all."""
    fx = _read_fixture("two_word_scores.txt")
    e1, e2 = fx["equal_scores"]
    o = _attn_single(np.ones((1, 1)), np.array([[e1], [e2]]), np.eye(2), 1.0)[0, 0, 0]
    np.testing.assert_array_equal(o, np.array(fx["equal_weights"]))
    o4 = _attn_single(np.ones((1, 1)), np.array([[4.0], [0.0]]), np.eye(2), 1.0)[0, 0, 0]
    assert abs(o4[0] - 1.0 / (1.0 + math.exp(-4.0))) < 1e-15 and o4[0] > 0.98


# --------------------------------------------------------------------------
# special cases that reduce to a library routine
# --------------------------------------------------------------------------

@pytest.mark.parametrize("Tq,Tk,d", [(5, 7, 3), (9, 4, 16), (1, 6, 8), (33, 33, 64)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("key_len", [None, 3, 0])
def test_identity_values_give_scipy_softmax(Tq, Tk, d, causal, key_len):
    """With V = I (d_v = Tk) the output rows are the attention weights themselves.

    Compared with scipy.special.softmax of scale * Q K^T over the allowed keys
    (masked weights 0).  Tq != Tk and random Q, K catch a transposed product;
    asymmetric masks catch a mask on the wrong index.
    """
    q = _rand((Tq, d), 1)
    k = _rand((Tk, d), 2)
    scale = 1.0 / math.sqrt(d)
    o = _attn_single(q, k, np.eye(Tk), scale, causal=causal, key_len=key_len)[0, 0]
    s = (q @ k.T) * scale
    for i in range(Tq):
        ok = [j for j in range(Tk)
              if (not causal or j <= i) and (key_len is None or j < key_len)]
        want = np.zeros(Tk)
        if ok:
            want[ok] = scipy_softmax(s[i, ok])
        np.testing.assert_allclose(o[i], want, rtol=0, atol=1e-14)


def test_zero_query_gives_mean_of_allowed_values():
    """Equal scores (aiany.app Step 5) -> uniform weights -> the mean of the value rows.

    Unmasked: numpy mean; key padding L: mean of the first L rows; causal: the
    prefix mean cumsum / (i + 1).
    """
    Tq, Tk, d = 12, 12, 8
    q = np.zeros((Tq, d))
    k = _rand((Tk, d), 3)
    v = _rand((Tk, d), 4)
    o = _attn_single(q, k, v, 0.125)[0, 0]
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), (Tq, d)), atol=1e-14)
    o = _attn_single(q, k, v, 0.125, key_len=5)[0, 0]
    np.testing.assert_allclose(o, np.broadcast_to(v[:5].mean(axis=0), (Tq, d)), atol=1e-14)
    o = _attn_single(q, k, v, 0.125, causal=True)[0, 0]
    prefix = np.cumsum(v, axis=0) / np.arange(1, Tk + 1)[:, None]
    np.testing.assert_allclose(o, prefix, atol=1e-14)
    # scale 0 is the same special case for any Q
    o = _attn_single(_rand((Tq, d), 5), k, v, 0.0, causal=True)[0, 0]
    np.testing.assert_allclose(o, prefix, atol=1e-14)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def test_single_key_returns_its_value():
    """Tk = 1: the only weight is 1, so every output row is V[0]."""
    q = _rand((2, 3, 7, 16), 6)
    k = _rand((2, 3, 1, 16), 7)
    v = _rand((2, 3, 1, 16), 8)
    o = attention_fp64(q, k, v, 0.25)
    np.testing.assert_array_equal(o, np.broadcast_to(v, o.shape))


def test_identical_value_rows_return_that_row():
    """All value rows equal -> the weighted mean is that row (weights sum to 1)."""
    q = _rand((1, 2, 9, 8), 9)
    k = _rand((1, 2, 11, 8), 10)
    row = _rand((8,), 11)
    v = np.broadcast_to(row, (1, 2, 11, 8)).copy()
    for causal in (False, True):
        o = attention_fp64(q, k, v, 0.3, causal=causal, key_lens=[6])
        np.testing.assert_allclose(o, np.broadcast_to(row, o.shape), rtol=1e-14, atol=1e-14)


def test_causal_row_zero_is_first_value():
    """Causal rule j <= t (notebook chapter, "Masked Attention in the Decoder"): row 0 sees key 0 only."""
    q = _rand((2, 3, 10, 8), 12)
    k = _rand((2, 3, 10, 8), 13)
    v = _rand((2, 3, 10, 8), 14)
    o = attention_fp64(q, k, v, 0.5, causal=True)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])


def test_winner_takes_all_at_huge_scores():
    """Scores of order 1e3: the max-subtracted softmax stays finite and picks the best key.

    Without the row-max subtraction exp() overflows to inf and the output is NaN.
    """
    d = 4
    k = np.eye(d) * 1000.0
    q = np.array([[0.1, 0.9, 0.3, 0.2], [5.0, 1.0, 1.0, 1.0]])
    v = _rand((d, 6), 15)
    o = _attn_single(q, k, v, 1.0)[0, 0]
    assert np.all(np.isfinite(o))
    np.testing.assert_array_equal(o[0], v[1])
    np.testing.assert_array_equal(o[1], v[0])


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal,key_lens", [(False, None), (True, None), (False, [3, 9]), (True, [0, 7])])
def test_weights_rows_sum_to_one_and_masked_are_zero(causal, key_lens):
    """Each row of weights sums to 1 (overview page; aiany.app Step 6); masked weights are 0."""
    B, H, Tq, Tk, d = 2, 2, 9, 9, 5
    q, k, v = _rand((B, H, Tq, d), 16), _rand((B, H, Tk, d), 17), _rand((B, H, Tk, d), 18)
    _, w = attention_fp64(q, k, v, 0.7, causal=causal, key_lens=key_lens, return_weights=True)
    for b in range(B):
        L = None if key_lens is None else key_lens[b]
        ok = allowed_mask(np.arange(Tq), Tk, causal, L)
        assert np.all(w[b][:, ~ok] == 0.0)
        sums = w[b].sum(axis=-1)
        has = ok.any(axis=-1)
        np.testing.assert_allclose(sums[:, has], 1.0, atol=1e-12)
        assert np.all(sums[:, ~has] == 0.0)


def test_output_is_convex_combination_of_values():
    """Every output coordinate lies between the min and max of the allowed value rows."""
    q, k, v = _rand((1, 1, 16, 8), 19, 3.0), _rand((1, 1, 16, 8), 20, 3.0), _rand((1, 1, 16, 8), 21)
    o = attention_fp64(q, k, v, 0.125, causal=True)[0, 0]
    for i in range(16):
        lo = v[0, 0, :i + 1].min(axis=0)
        hi = v[0, 0, :i + 1].max(axis=0)
        assert np.all(o[i] >= lo - 1e-14) and np.all(o[i] <= hi + 1e-14)


def test_key_value_permutation_invariance():
    """Attention is order-blind (aiany.app Step 8; notebook "Positional Encoding"):
    permuting (K, V) jointly leaves the output unchanged; under key padding the
    permutation stays inside the valid prefix."""
    Tq, Tk, d = 7, 13, 8
    q, k, v = _rand((Tq, d), 22), _rand((Tk, d), 23), _rand((Tk, d), 24)
    perm = np.random.default_rng(25).permutation(Tk)
    o1 = _attn_single(q, k, v, 0.4)
    o2 = _attn_single(q, k[perm], v[perm], 0.4)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    L = 6
    pl = np.concatenate([np.random.default_rng(26).permutation(L), np.arange(L, Tk)])
    o1 = _attn_single(q, k, v, 0.4, key_len=L)
    o2 = _attn_single(q, k[pl], v[pl], 0.4, key_len=L)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)


def test_query_permutation_equivariance():
    """Permuting the query rows permutes the output rows (notebook: permutation-equivariant)."""
    Tq, Tk, d = 9, 6, 4
    q, k, v = _rand((Tq, d), 27), _rand((Tk, d), 28), _rand((Tk, d), 29)
    perm = np.random.default_rng(30).permutation(Tq)
    o1 = _attn_single(q, k, v, 0.9)[0, 0]
    o2 = _attn_single(q[perm], k, v, 0.9)[0, 0]
    np.testing.assert_allclose(o1[perm], o2, rtol=0, atol=1e-14)


def test_score_shift_invariance():
    """softmax(x + c) = softmax(x): adding a vector c to every key adds q.c to a whole row."""
    Tq, Tk, d = 8, 10, 6
    q, k, v = _rand((Tq, d), 31), _rand((Tk, d), 32), _rand((Tk, d), 33)
    c = _rand((d,), 34, 5.0)
    for causal in (False, True):
        o1 = _attn_single(q, k, v, 0.5, causal=causal)
        o2 = _attn_single(q, k + c[None, :], v, 0.5, causal=causal)
        np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# mask laws: masking is the same as dropping the masked keys
# --------------------------------------------------------------------------

def test_key_padding_equals_truncated_keys():
    """Key padding with length L equals unmasked attention over K[:L], V[:L]."""
    Tq, Tk, d = 11, 14, 8
    q, k, v = _rand((Tq, d), 35), _rand((Tk, d), 36), _rand((Tk, d), 37)
    for L in (1, 5, 13, 14):
        o1 = _attn_single(q, k, v, 0.35, key_len=L)
        o2 = _attn_single(q, k[:L], v[:L], 0.35)
        np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-14)


def test_causal_row_equals_prefix_attention():
    """Causal row i equals unmasked attention of that query over K[:i+1], V[:i+1]
    (notebook chapter e_tj cases; muhitai.com causal table); for Tq > Tk rows past
    the end see every key (literal j <= i reading)."""
    Tq, Tk, d = 12, 9, 8
    q, k, v = _rand((Tq, d), 38), _rand((Tk, d), 39), _rand((Tk, d), 40)
    o = _attn_single(q, k, v, 0.35, causal=True)[0, 0]
    for i in range(Tq):
        n = min(i + 1, Tk)
        want = _attn_single(q[i:i + 1], k[:n], v[:n], 0.35)[0, 0, 0]
        np.testing.assert_allclose(o[i], want, rtol=0, atol=1e-14)


def test_causal_and_padding_combine_as_intersection():
    Tq, Tk, d, L = 10, 10, 4, 6
    q, k, v = _rand((Tq, d), 41), _rand((Tk, d), 42), _rand((Tk, d), 43)
    o = _attn_single(q, k, v, 0.5, causal=True, key_len=L)[0, 0]
    for i in range(Tq):
        n = min(i + 1, L)
        want = _attn_single(q[i:i + 1], k[:n], v[:n], 0.5)[0, 0, 0]
        np.testing.assert_allclose(o[i], want, rtol=0, atol=1e-14)


def test_empty_rows_and_clamped_lengths():
    """Readings where the pages are silent: no allowed key -> zero row; lengths clamp to [0, Tk]."""
    Tq, Tk, d = 4, 6, 3
    q, k, v = _rand((Tq, d), 44), _rand((Tk, d), 45), _rand((Tk, d), 46)
    assert np.all(_attn_single(q, k, v, 1.0, key_len=0) == 0.0)
    assert np.all(_attn_single(q, k, v, 1.0, key_len=-5) == 0.0)
    np.testing.assert_array_equal(_attn_single(q, k, v, 1.0, key_len=99), _attn_single(q, k, v, 1.0))
    o = attention_fp64(q[None, None], k[None, None, :0], v[None, None, :0], 1.0)
    assert o.shape == (1, 1, Tq, d) and np.all(o == 0.0)


def test_row_subset_and_blocking_match_full():
    """Row-subset mode and the row blocking return exactly the full computation's rows."""
    q, k, v = _rand((1, 2, 37, 8), 47), _rand((1, 2, 37, 8), 48), _rand((1, 2, 37, 8), 49)
    full = attention_fp64(q, k, v, 0.2, causal=True)
    rows = np.array([0, 5, 17, 36])
    sub = attention_fp64(q, k, v, 0.2, causal=True, rows=rows, block=3)
    np.testing.assert_allclose(sub, full[:, :, rows], rtol=0, atol=1e-15)
    blk = attention_fp64(q, k, v, 0.2, causal=True, block=5)
    np.testing.assert_allclose(blk, full, rtol=0, atol=1e-15)


# --------------------------------------------------------------------------
# brute force on tiny inputs, and the pages' PyTorch formula in float64
# --------------------------------------------------------------------------

def _brute(q, k, v, scale, causal, L):
    Tq, Tk, dv = q.shape[0], k.shape[0], v.shape[1]
    out = [[0.0] * dv for _ in range(Tq)]
    for i in range(Tq):
        js = [j for j in range(Tk) if (not causal or j <= i) and (L is None or j < max(0, min(L, Tk)))]
        if not js:
            continue
        s = {j: scale * math.fsum(float(q[i, c]) * float(k[j, c]) for c in range(q.shape[1])) for j in js}
        top = max(s.values())
        e = {j: math.exp(s[j] - top) for j in js}
        z = math.fsum(e.values())
        for c in range(dv):
            out[i][c] = math.fsum(e[j] / z * float(v[j, c]) for j in js)
    return np.array(out)


@pytest.mark.parametrize("seed", range(6))
def test_scalar_brute_force_tiny(seed):
    rng = np.random.default_rng(100 + seed)
    Tq, Tk, d, dv = (int(x) for x in rng.integers(1, 7, size=4))
    q, k, v = rng.standard_normal((Tq, d)) * 2, rng.standard_normal((Tk, d)) * 2, rng.standard_normal((Tk, dv))
    causal = bool(seed % 2)
    L = None if seed < 2 else int(rng.integers(-1, Tk + 2))
    o = _attn_single(q, k, v, 0.6, causal=causal, key_len=L)[0, 0]
    np.testing.assert_allclose(o, _brute(q, k, v, 0.6, causal, L), rtol=0, atol=1e-12)


def test_pages_pytorch_formula_float64():
    """The cuijiawei.cn snippet's steps (q @ k^T / sqrt(d_k), masked_fill(mask == 0, -inf),
    softmax, @ v) run through torch in float64 on the CPU agree with the oracle."""
    torch = pytest.importorskip("torch")
    B, H, Tq, Tk, d = 2, 3, 17, 17, 16
    q, k, v = _rand((B, H, Tq, d), 50), _rand((B, H, Tk, d), 51), _rand((B, H, Tk, d), 52)
    L = [9, 17]
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    mask = torch.ones(B, 1, Tq, Tk, dtype=torch.bool)
    mask &= torch.tril(torch.ones(Tq, Tk, dtype=torch.bool))
    for b in range(B):
        mask[b, :, :, L[b]:] = False
    scores = tq @ tk.transpose(-2, -1) / d ** 0.5
    scores = scores.masked_fill(mask == 0, float("-inf"))
    want = torch.softmax(scores, dim=-1) @ tv
    got = attention_fp64(q, k, v, 1.0 / d ** 0.5, causal=True, key_lens=L)
    np.testing.assert_allclose(got, want.numpy(), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# planted mistakes: each plausible slip in the oracle fails at least one pin
# --------------------------------------------------------------------------

def _mutant(kind):
    def softmax_rows(scores, allowed):
        if kind == "no_max_sub":
            s = np.where(allowed, scores, -np.inf)
            e = np.exp(s)
            return e / e.sum(axis=-1, keepdims=True)
        if kind == "wrong_axis":
            s = np.where(allowed, scores, -np.inf)
            m = s.max(axis=0, keepdims=True)
            e = np.exp(s - m)
            return e / e.sum(axis=0, keepdims=True)
        raise ValueError(kind)

    def mask(rows, Tk, causal, key_len):
        rows = np.asarray(rows)
        j = np.arange(Tk)[None, :]
        ok = np.ones((rows.shape[0], Tk), dtype=bool)
        if causal:
            ok &= (j < rows[:, None]) if kind == "causal_strict" else (j <= rows[:, None])
        if key_len is not None:
            L = min(max(int(key_len), 0), Tk)
            ok &= (j <= L) if kind == "pad_off_by_one" else (j < L)
        return ok

    return softmax_rows, mask


def _run_pins():
    """Run a subset of the pins; return the number that fail."""
    pins = [
        test_three_score_softmax_example,
        test_two_word_example,
        lambda: test_identity_values_give_scipy_softmax(5, 7, 3, True, 3),
        test_causal_row_zero_is_first_value,
        test_winner_takes_all_at_huge_scores,
        test_key_padding_equals_truncated_keys,
        lambda: test_weights_rows_sum_to_one_and_masked_are_zero(True, [3, 9]),
    ]
    failed = 0
    for p in pins:
        try:
            with np.errstate(all="ignore"):
                p()
        except AssertionError:
            failed += 1
    return failed


@pytest.mark.parametrize("kind", ["no_max_sub", "wrong_axis", "causal_strict", "pad_off_by_one",
                                  "no_scale", "transposed", "neg_sign"])
def test_planted_mistakes_are_caught(kind, monkeypatch):
    mod = oracle.attention
    orig_attn = mod.attention_fp64
    sm, mk = _mutant(kind)
    if kind in ("no_max_sub", "wrong_axis"):
        monkeypatch.setattr(mod, "softmax_rows_fp64", sm)
    if kind in ("causal_strict", "pad_off_by_one"):
        monkeypatch.setattr(mod, "allowed_mask", mk)
    if kind in ("no_scale", "transposed", "neg_sign"):
        def attn(q, k, v, scale, *a, **kw):
            if kind == "no_scale":
                return orig_attn(q, k, v, 1.0, *a, **kw)
            if kind == "neg_sign":
                return orig_attn(q, k, v, -scale, *a, **kw)
            # transposed: use the keys as queries where the shapes allow it
            if q.shape == k.shape:
                return orig_attn(k, q, v, scale, *a, **kw)
            return orig_attn(q, k, v, scale, *a, **kw)[..., ::-1, :]
        monkeypatch.setattr(mod, "attention_fp64", attn)
        monkeypatch.setattr(oracle, "attention_fp64", attn)
        monkeypatch.setitem(globals(), "attention_fp64", attn)
    assert _run_pins() >= 1
