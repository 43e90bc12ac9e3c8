"""Reference (oracle) implementation of scaled dot-product attention, fp64, CPU.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this module:
only the tests, the smoke check of the entry module and the CPU-baseline leg of
the benchmark call it.  It shares no code with the HIP library and imports
nothing from the package.

What it computes (the plain definition; the fused GPU kernel reaches the same
value by reassociating the sums):

    Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V

  * formula: "Attention Is All You Need" overview (azimuth.plus), section "The
    idea: every word queries every word"; the LaTeX form in the notebook
    chapter (antoniofranca.me), section "Multi-Head Self-Attention"; the
    cuijiawei.cn summary, section "The core idea: scaled dot-product attention".
  * the scores are divided by sqrt(d_k) (aiany.app explainer, Step 5 "Scale:
    divide by 8" and Step 6 matrix form S = QK^T / sqrt(dk); the division sign
    is lost in that page's one-line formula, every other statement has it).
    Here the caller passes the scale explicitly, normally 1/sqrt(d_k).
  * softmax is taken per query row, after subtracting the row maximum (the
    overview page's NumPy snippet, "stable softmax"); every row of weights sums
    to one (aiany.app Step 6, A = softmax(S), "each row sums to 1").
  * masked scores are -inf before the softmax, so their weight is exactly 0:
    causal rule e_tj = -inf for j > t (notebook chapter, section "Masked
    Attention in the Decoder"); generic mask `masked_fill(mask == 0, -inf)`
    (cuijiawei.cn, section "Minimal PyTorch implementation").  Key padding is
    read as that generic mask with mask[b, :, :, j] = (j < L_b).
  * output row = weighted sum of the value rows (aiany.app Step 5, "Weigh each
    value" / "Sum -- and you have z1"; Step 6, Z = AV).

Readings where the pages are silent (each also listed in the design notes):
  * causal with Tq != Tk: the literal rule j <= i (top-left aligned).
  * a row with no allowed key (L_b = 0, or Tk = 0) outputs zeros.
  * key lengths outside [0, Tk] are clamped to that range.

The softmax is deliberately the two-pass form (max, then exp / sum), not the
running (online) form the kernel uses, so agreement between the two pins the
kernel's rescaling.
"""
from __future__ import annotations

import numpy as np

__all__ = ["allowed_mask", "attention_backward_fp64", "attention_backward_sampled_fp64", "attention_fp64",
           "attention_lse_fp64", "multi_head_attention_fp64", "softmax_rows_fp64"]


def allowed_mask(rows: np.ndarray, Tk: int, causal: bool, key_len: int | None) -> np.ndarray:
    """Boolean [len(rows), Tk]: True where query row `rows[i]` may attend key j.

    Key j is allowed iff (not causal or j <= row) and (no key length or j < L),
    with L clamped to [0, Tk] (causal rule: notebook chapter, "Masked Attention
    in the Decoder"; padding as the generic mask of the cuijiawei.cn snippet).
    """
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(Tk, dtype=np.int64)[None, :]
    ok = np.ones((rows.shape[0], Tk), dtype=bool)
    if causal:
        ok &= j <= rows[:, None]
    if key_len is not None:
        L = min(max(int(key_len), 0), Tk)
        ok &= j < L
    return ok


def softmax_rows_fp64(scores: np.ndarray, allowed: np.ndarray) -> np.ndarray:
    """Row softmax of fp64 `scores` restricted to `allowed`; masked weights are 0.

    Two passes: row max over allowed entries, then exp(s - max) / sum (the
    overview page's stable softmax).  A row with no allowed entry gets all-zero
    weights.
    """
    s = np.where(allowed, scores, -np.inf)
    any_ok = allowed.any(axis=-1, keepdims=True)
    m = np.where(any_ok, s.max(axis=-1, keepdims=True, initial=-np.inf), 0.0)
    e = np.exp(s - m)  # exp(-inf) = 0 for masked entries
    z = e.sum(axis=-1, keepdims=True)
    return np.where(any_ok, e / np.where(any_ok, z, 1.0), 0.0)


def attention_fp64(q, k, v, scale: float, causal: bool = False, key_lens=None,
                   rows=None, heads=None, return_weights: bool = False, block: int = 256):
    """Scaled dot-product attention in fp64 for [B, h, T, d] inputs.

    q: [B, h, Tq, d_k], k: [B, h, Tk, d_k], v: [B, h, Tk, d_v]; any real dtype,
    widened exactly to fp64 (pass the values the GPU sees, e.g. bf16-rounded).
    scale: the score multiplier (normally 1/sqrt(d_k)), used as given.
    key_lens: None or int sequence [B] (valid key count per batch entry).
    rows: None (all query rows) or a 1-D index array: only those rows are
      computed, for every (b, head) selected.
    heads: None (all) or a list of (b, head) pairs to compute; others are left 0.
    Returns out [B, h, R, d_v] fp64 (R = Tq or len(rows)) and, when
    return_weights, the weights [B, h, R, Tk].
    Processes each (b, head) in blocks of `block` query rows so the score
    matrix is never held whole.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, H, Tq, dk = q.shape
    Tk = k.shape[2]
    dv = v.shape[3]
    assert k.shape == (B, H, Tk, dk) and v.shape == (B, H, Tk, dv)
    row_idx = np.arange(Tq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = row_idx.shape[0]
    out = np.zeros((B, H, R, dv), dtype=np.float64)
    wts = np.zeros((B, H, R, Tk), dtype=np.float64) if return_weights else None
    pairs = [(b, hh) for b in range(B) for hh in range(H)] if heads is None else list(heads)
    sc = float(scale)
    for b, hh in pairs:
        L = None if key_lens is None else int(np.asarray(key_lens)[b])
        kb = k[b, hh].astype(np.float64)
        vb = v[b, hh].astype(np.float64)
        for r0 in range(0, R, block):
            ridx = row_idx[r0:r0 + block]
            qb = q[b, hh, ridx].astype(np.float64)
            s = (qb @ kb.T) * sc
            w = softmax_rows_fp64(s, allowed_mask(ridx, Tk, causal, L))
            out[b, hh, r0:r0 + block] = w @ vb
            if return_weights:
                wts[b, hh, r0:r0 + block] = w
    return (out, wts) if return_weights else out


def attention_lse_fp64(q, k, v, scale: float, causal: bool = False, key_lens=None, block: int = 256,
                       rows=None):
    """Attention output plus the per-row log-sum-exp of the scaled scores, fp64.

    lse[b, h, i] = log sum_{j allowed} exp(scale * q_i . k_j)   (natural log),
    -inf for a row with no allowed key.  This is the normaliser of the row
    softmax (overview page, stable softmax: the row sum of exp) kept in log
    form, so that the weights can be recomputed as exp(s_ij - lse_i).
    rows: None (all query rows) or a 1-D index array: out and lse are then
    [B, h, len(rows), ...] for those rows only.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, H, Tq, dk = q.shape
    Tk = k.shape[2]
    row_idx = np.arange(Tq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = row_idx.shape[0]
    out = attention_fp64(q, k, v, scale, causal=causal, key_lens=key_lens, rows=rows, block=block)
    lse = np.full((B, H, R), -np.inf, dtype=np.float64)
    sc = float(scale)
    for b in range(B):
        L = None if key_lens is None else int(np.asarray(key_lens)[b])
        for hh in range(H):
            kb = k[b, hh].astype(np.float64)
            for r0 in range(0, R, block):
                ridx = row_idx[r0:r0 + block]
                s = (q[b, hh, ridx].astype(np.float64) @ kb.T) * sc
                ok = allowed_mask(ridx, Tk, causal, L)
                s = np.where(ok, s, -np.inf)
                any_ok = ok.any(axis=-1)
                m = np.where(any_ok, s.max(axis=-1, initial=-np.inf), 0.0)
                with np.errstate(divide="ignore"):
                    lse[b, hh, r0:r0 + block] = np.where(
                        any_ok, m + np.log(np.exp(s - m[:, None]).sum(axis=-1)), -np.inf)
    return out, lse


def attention_backward_fp64(q, k, v, dout, scale: float, causal: bool = False, key_lens=None):
    """Gradients of O = softmax(scale * Q K^T) V with respect to Q, K, V, fp64.

    Training the model on the pages means back-propagating a loss through
    this formula (aiany.app Step 11, cross-entropy training nudging every
    weight; notebook chapter, "Layer Normalization and Residual Connections",
    gradients flowing through each sublayer).  With P the row-softmax weights
    (zero where masked) and dO the gradient of the loss with respect to O, the
    chain rule through O = P V and the row softmax gives:
        dV = P^T dO
        dP = dO V^T
        D_i = sum_j P_ij dP_ij  (= dO_i . O_i)
        dS = P * (dP - D)       (elementwise, D broadcast along rows)
        dQ = scale * dS K,   dK = scale * dS^T Q
    Rows with no allowed key contribute nothing.  Returns (dq, dk, dv, delta)
    with delta = D of shape [B, h, Tq].  Whole score matrices per (b, head):
    for test sizes only.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    dout = np.asarray(dout)
    B, H, Tq, dk = q.shape
    Tk = k.shape[2]
    dq = np.zeros(q.shape, dtype=np.float64)
    dkk = np.zeros(k.shape, dtype=np.float64)
    dvv = np.zeros(v.shape, dtype=np.float64)
    delta = np.zeros((B, H, Tq), dtype=np.float64)
    sc = float(scale)
    rows = np.arange(Tq)
    for b in range(B):
        L = None if key_lens is None else int(np.asarray(key_lens)[b])
        ok = allowed_mask(rows, Tk, causal, L)
        for hh in range(H):
            qb = q[b, hh].astype(np.float64)
            kb = k[b, hh].astype(np.float64)
            vb = v[b, hh].astype(np.float64)
            gb = dout[b, hh].astype(np.float64)
            p = softmax_rows_fp64((qb @ kb.T) * sc, ok)
            dvv[b, hh] = p.T @ gb
            dp = gb @ vb.T
            d_row = (p * dp).sum(axis=-1)
            ds = p * (dp - d_row[:, None])
            dq[b, hh] = sc * (ds @ kb)
            dkk[b, hh] = sc * (ds.T @ qb)
            delta[b, hh] = d_row
    return dq, dkk, dvv, delta


def attention_backward_sampled_fp64(q, k, v, dout, scale: float, causal: bool = False, key_lens=None,
                                    rows=None, keys=None, heads=None, block: int = 256):
    """The gradients of attention_backward_fp64 at a subset of positions, fp64.

    dq at query rows `rows` and dk, dv at key positions `keys` (1-D index
    arrays, None = none), for the (b, head) pairs in `heads` (None = all).
    Same formulas; the score matrix is never held whole:
      * dq_i needs only row i of P and dP: dS_i = P_i * (dP_i - D_i),
        dq_i = scale * dS_i K;
      * dk_j, dv_j need column j of P and dP over every row, and D_i for every
        row, so all rows are swept in blocks of `block`, each block taking its
        full rows of P (two-pass softmax) and dP, and contributing
        dv_j += P_bj^T dO_b and dk_j += scale * dS_bj^T Q_b.
    Returns (dq [B, h, len(rows), d], dk [B, h, len(keys), d], dv [...]);
    pairs not selected are left 0.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    dout = np.asarray(dout)
    B, H, Tq, dk_ = q.shape
    Tk = k.shape[2]
    dv_ = v.shape[3]
    rows = np.zeros(0, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    keys = np.zeros(0, dtype=np.int64) if keys is None else np.asarray(keys, dtype=np.int64)
    gq = np.zeros((B, H, rows.shape[0], dk_))
    gk = np.zeros((B, H, keys.shape[0], dk_))
    gv = np.zeros((B, H, keys.shape[0], dv_))
    pairs = [(b, hh) for b in range(B) for hh in range(H)] if heads is None else list(heads)
    sc = float(scale)
    for b, hh in pairs:
        L = None if key_lens is None else int(np.asarray(key_lens)[b])
        kb = k[b, hh].astype(np.float64)
        vb = v[b, hh].astype(np.float64)
        if rows.shape[0]:
            qr = q[b, hh, rows].astype(np.float64)
            gr = dout[b, hh, rows].astype(np.float64)
            p = softmax_rows_fp64((qr @ kb.T) * sc, allowed_mask(rows, Tk, causal, L))
            dp = gr @ vb.T
            ds = p * (dp - (p * dp).sum(axis=-1, keepdims=True))
            gq[b, hh] = sc * (ds @ kb)
        if keys.shape[0]:
            for r0 in range(0, Tq, block):
                ridx = np.arange(r0, min(r0 + block, Tq))
                qb = q[b, hh, ridx].astype(np.float64)
                gb = dout[b, hh, ridx].astype(np.float64)
                p = softmax_rows_fp64((qb @ kb.T) * sc, allowed_mask(ridx, Tk, causal, L))
                dp = gb @ vb.T
                d_row = (p * dp).sum(axis=-1, keepdims=True)
                pc = p[:, keys]
                gv[b, hh] += pc.T @ gb
                gk[b, hh] += sc * ((pc * (dp[:, keys] - d_row)).T @ qb)
    return gq, gk, gv


def multi_head_attention_fp64(xq, xk, xv, wq, wk, wv, wo, heads: int, scale: float, causal: bool = False,
                              key_lens=None, rows=None, batches=None):
    """Multi-head attention in fp64, as the pages define it.

        head_i = Attention(Xq W_i^Q, Xk W_i^K, Xv W_i^V),
        MultiHead = Concat(head_1, ..., head_h) W^O
    (notebook chapter, "Multi-Head Self-Attention"; cuijiawei.cn, "The core idea:
    scaled dot-product attention" and its MultiHeadAttention snippet; overview
    page, multi_head_attention()).  Read without bias terms: the formula and the
    NumPy version have none (the PyTorch snippet's nn.Linear layers would add
    them).  Head i uses columns i*d .. i*d+d-1 of each projection (the snippet's
    view(B, T, h, d) of the projected rows) and rows i*d .. of W^O.

    xq [B, Tq, dm], xk, xv [B, Tk, dm]; wq, wk, wv [dm, h*d]; wo [h*d, dm] (row
    vectors times matrices, x @ W).  scale, causal, key_lens as attention_fp64.
    rows: None or query-row indices (only those output rows); batches: None or
    batch indices to compute (others left 0).  Returns y [B, R, dm] fp64.
    """
    xq = np.asarray(xq)
    xk = np.asarray(xk)
    xv = np.asarray(xv)
    B, Tq, dm = xq.shape
    Tk = xk.shape[1]
    hd = np.asarray(wq).shape[1]
    d = hd // heads
    assert hd == heads * d and np.asarray(wo).shape == (hd, dm)
    wq, wk, wv, wo = (np.asarray(w, dtype=np.float64) for w in (wq, wk, wv, wo))
    row_idx = np.arange(Tq) if rows is None else np.asarray(rows, dtype=np.int64)
    y = np.zeros((B, row_idx.shape[0], dm))
    for b in (range(B) if batches is None else batches):
        q = (xq[b].astype(np.float64) @ wq).reshape(Tq, heads, d).transpose(1, 0, 2)[None]
        k = (xk[b].astype(np.float64) @ wk).reshape(Tk, heads, d).transpose(1, 0, 2)[None]
        v = (xv[b].astype(np.float64) @ wv).reshape(Tk, heads, d).transpose(1, 0, 2)[None]
        kl = None if key_lens is None else [int(np.asarray(key_lens)[b])]
        o = attention_fp64(q, k, v, scale, causal=causal, key_lens=kl, rows=rows)[0]   # [h, R, d]
        y[b] = o.transpose(1, 0, 2).reshape(row_idx.shape[0], hd) @ wo
    return y
