"""Seeded synthetic workloads for scaled dot-product attention.

This module only describes shapes and draws inputs; it holds none of the
attention arithmetic, so both the HIP path and the fp64 oracle can take their
inputs from it.

Shapes follow the base model of "Attention Is All You Need" as the pages give
it: h = 8 heads with d_k = d_v = d_model / h = 64 (notebook chapter,
"Multi-Head Self-Attention"; cuijiawei.cn, "Architecture"), the three
attention kinds of the decoder/encoder (encoder self-attention with padded
sentences, decoder masked self-attention, encoder-decoder cross-attention with
Tq != Tk: aiany.app Step 10; muhitai.com "What Is Masked Attention?" and
"Encoder-Decoder Attention") and one long-sequence case with d = 128.  The
pages measure on WMT 2014 translation; these seeded tensors stand in for the
attention shapes of that workload, no text data is involved.

Recipe (fixed order): g = torch.Generator('cpu').manual_seed(seed); Q, K, V
each from torch.randn(shape, generator=g, dtype=float32); Q and K multiplied by
`qk_mul`; then key lengths from torch.randint(lo, hi + 1, (B,), generator=g,
dtype=int32) when the workload has key padding; finally one round-to-nearest-
even cast to the workload dtype.  The values handed to the GPU are exactly the
values the oracle sees (widened to fp64).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

# scale values as fp32 literals: 1/sqrt(64) = 0.125 exactly; 1/sqrt(128) rounded
# once from fp64 to fp32.
SCALE_D64 = 0.125
SCALE_D128 = 0.0883883461356163  # float32(0.08838834764831845)

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_KEYPAD = 2


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    h: int
    Tq: int
    Tk: int
    d: int
    dtype: str            # "f32" or "bf16"
    mask: int             # MASK_* bits
    scale: float
    qk_mul: float = 1.0
    key_len_range: tuple | None = None   # (lo, hi), inclusive, for key padding
    desc: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def causal(self) -> bool:
        return bool(self.mask & MASK_CAUSAL)

    @property
    def keypad(self) -> bool:
        return bool(self.mask & MASK_KEYPAD)

    def with_mask(self, mask: int, name: str | None = None) -> "Workload":
        return Workload(name or self.name, self.B, self.h, self.Tq, self.Tk, self.d, self.dtype,
                        mask, self.scale, self.qk_mul, self.key_len_range, self.desc)


WORKLOADS = {
    "sdpa_f32_b1h8t64d64": Workload(
        "sdpa_f32_b1h8t64d64", 1, 8, 64, 64, 64, "f32", MASK_NONE, SCALE_D64,
        desc="fp32 SDPA, no mask, B1 h8 T64 d64"),
    "enc_self_bf16_b32h8t256d64_keypad": Workload(
        "enc_self_bf16_b32h8t256d64_keypad", 32, 8, 256, 256, 64, "bf16", MASK_KEYPAD, SCALE_D64,
        key_len_range=(128, 256), desc="encoder self-attention, key padding L~U[128,256]"),
    "dec_causal_bf16_b16h16t1024d64": Workload(
        "dec_causal_bf16_b16h16t1024d64", 16, 16, 1024, 1024, 64, "bf16", MASK_CAUSAL, SCALE_D64,
        qk_mul=3.0, desc="decoder causal self-attention, Q,K ~ 3 N(0,1)"),
    "cross_bf16_b16h16q512k1024d64_keypad": Workload(
        "cross_bf16_b16h16q512k1024d64_keypad", 16, 16, 512, 1024, 64, "bf16", MASK_KEYPAD,
        SCALE_D64, key_len_range=(512, 1024), desc="cross-attention, encoder lengths U[512,1024]"),
    "long_bf16_b1h16t16384d128": Workload(
        "long_bf16_b1h16t16384d128", 1, 16, 16384, 16384, 128, "bf16", MASK_NONE, SCALE_D128,
        desc="long-sequence attention, unmasked"),
    "long_causal_bf16_b1h16t16384d128": Workload(
        "long_causal_bf16_b1h16t16384d128", 1, 16, 16384, 16384, 128, "bf16", MASK_CAUSAL,
        SCALE_D128, desc="long-sequence attention, causal"),
    # one query row per (b, head) against a key/value cache: the decoder's generation step
    "decode_bf16_b8h16k16384d128": Workload(
        "decode_bf16_b8h16k16384d128", 8, 16, 1, 16384, 128, "bf16", MASK_NONE, SCALE_D128,
        desc="decode step: one new row per head against a 16384-entry cache (K+V 1 GiB)"),
    "decode_keypad_bf16_b64h8k4096d64": Workload(
        "decode_keypad_bf16_b64h8k4096d64", 64, 8, 1, 4096, 64, "bf16", MASK_KEYPAD, SCALE_D64,
        key_len_range=(256, 4096), desc="decode step, ragged caches L~U[256,4096] (K+V 512 MiB)"),
}

# the workload the throughput figure is quoted on (non-causal, T >= 1024)
HEADLINE = "long_bf16_b1h16t16384d128"
# the workload the decode measurement is quoted on
DECODE_HEADLINE = "decode_bf16_b8h16k16384d128"

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def make_inputs(w: Workload, seed: int = 0, device: str | torch.device = "cpu"):
    """Draw (q, k, v, key_lens) for workload `w` with the fixed recipe above.

    q, k, v are [B, h, T, d] tensors of the workload dtype, contiguous;
    key_lens is an int32 [B] tensor, or None without key padding.
    """
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn((w.B, w.h, w.Tq, w.d), generator=g, dtype=torch.float32)
    k = torch.randn((w.B, w.h, w.Tk, w.d), generator=g, dtype=torch.float32)
    v = torch.randn((w.B, w.h, w.Tk, w.d), generator=g, dtype=torch.float32)
    if w.qk_mul != 1.0:
        q.mul_(w.qk_mul)
        k.mul_(w.qk_mul)
    key_lens = None
    if w.keypad:
        lo, hi = w.key_len_range if w.key_len_range is not None else (0, w.Tk)
        key_lens = torch.randint(lo, hi + 1, (w.B,), generator=g, dtype=torch.int32)
    dt = TORCH_DTYPES[w.dtype]
    q, k, v = (t.to(dt).contiguous() for t in (q, k, v))
    if device != "cpu":
        q, k, v = (t.to(device) for t in (q, k, v))
        if key_lens is not None:
            key_lens = key_lens.to(device)
    return q, k, v, key_lens


def grad_output(B, h, Tq, dv, dtype="bf16", seed=0):
    """Upstream gradient dO [B, h, Tq, d_v] for the backward pass: torch.randn
    from a generator seeded with seed + 1 (so it never repeats the Q/K/V
    stream of the same seed), rounded once to the dtype."""
    g = torch.Generator("cpu").manual_seed(seed + 1)
    x = torch.randn((B, h, Tq, dv), generator=g, dtype=torch.float32)
    return x.to(TORCH_DTYPES[dtype]).contiguous()


# multi-head attention (projections + attention + W^O) at the base model's width:
# d_model 512, 8 heads of 64 (notebook chapter, "Multi-Head Self-Attention")
MHA_WORKLOADS = {
    "mha_self_bf16_b32t1024dm512h8": dict(B=32, Tq=1024, Tk=1024, d_model=512, heads=8, causal=False),
}


def mha_inputs(B, Tq, Tk, d_model, seed=0, cross=False):
    """(xq, xk, xv, wq, wk, wv, wo) for multi-head attention, bf16 on the CPU.

    Recipe: g = torch.Generator('cpu').manual_seed(seed); xq [B, Tq, d_model]
    ~ N(0, 1); when `cross`, xk [B, Tk, d_model] ~ N(0, 1) and xv likewise,
    else xk = xv = xq (self-attention, Tk = Tq); then wq, wk, wv, wo, each
    [d_model, d_model] ~ N(0, 1) / sqrt(d_model) (random-init weights that keep
    the projected rows at unit variance); one round-to-nearest-even cast to bf16.
    """
    g = torch.Generator("cpu").manual_seed(seed)
    xq = torch.randn((B, Tq, d_model), generator=g, dtype=torch.float32)
    if cross:
        xk = torch.randn((B, Tk, d_model), generator=g, dtype=torch.float32)
        xv = torch.randn((B, Tk, d_model), generator=g, dtype=torch.float32)
    else:
        xk = xv = xq
    ws = [torch.randn((d_model, d_model), generator=g, dtype=torch.float32) / d_model ** 0.5 for _ in range(4)]
    bf = lambda t: t.to(torch.bfloat16).contiguous()
    xq_b = bf(xq)
    xk_b = xq_b if xk is xq else bf(xk)
    xv_b = xq_b if xv is xq else bf(xv)
    return (xq_b, xk_b, xv_b, *(bf(w) for w in ws))


def random_inputs(B, h, Tq, Tk, d, dtype="bf16", seed=0, qk_mul=1.0, dv=None):
    """Same recipe for an ad-hoc shape (edge-case tests); d_v defaults to d."""
    dv = d if dv is None else dv
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn((B, h, Tq, d), generator=g, dtype=torch.float32) * qk_mul
    k = torch.randn((B, h, Tk, d), generator=g, dtype=torch.float32) * qk_mul
    v = torch.randn((B, h, Tk, dv), generator=g, dtype=torch.float32)
    dt = TORCH_DTYPES[dtype]
    return tuple(t.to(dt).contiguous() for t in (q, k, v))


def sample_rows(Tq: int, n: int, seed: int = 0) -> torch.Tensor:
    """`n` distinct query-row indices, seeded, with rows 0 and Tq-1 always in."""
    g = torch.Generator("cpu").manual_seed(seed)
    perm = torch.randperm(Tq, generator=g)[:n]
    rows = set(int(x) for x in perm.tolist())
    rows.update({0, Tq - 1})
    rows = sorted(rows)
    while len(rows) > n:
        # drop interior picks until n remain, keeping both ends
        rows.pop(len(rows) // 2)
    return torch.tensor(rows, dtype=torch.int64)
