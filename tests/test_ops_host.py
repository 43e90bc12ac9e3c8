"""Host-side checks of the tensor wrapper (ops.py): a tensor in the wrong memory
must raise ValueError before any library call.

A CPU tensor's address passes every check the C ABI can make (non-null,
aligned, not overlapping the inputs), so only the wrapper can stop a kernel
from writing to it.  The device inputs here are stand-ins that report a GPU
device without owning memory; every library entry point is replaced by a
trap, so a missing check fails the test instead of launching anything.
"""
from __future__ import annotations

import pytest
import torch

from transformer_scaled_dot_03_amd import _lib, ops

DEV = torch.device("cuda:0")


class FakeDeviceTensor:
    """Just enough of torch.Tensor for the wrapper's checks: a contiguous tensor on cuda:0."""

    def __init__(self, shape, dtype, device=DEV):
        self.shape = torch.Size(shape)
        self.dtype = dtype
        self.device = torch.device(device)
        self.is_cuda = self.device.type == "cuda"

    def dim(self):
        return len(self.shape)

    def is_contiguous(self):
        return True

    def contiguous(self):
        return self

    def numel(self):
        n = 1
        for s in self.shape:
            n *= s
        return n

    def data_ptr(self):
        return 0x7F0000000000


@pytest.fixture(autouse=True)
def trap_library(monkeypatch):
    def trap(*_a, **_k):
        raise AssertionError("the library was called although an argument check should have failed")

    for name in ("attn_fwd", "attn_fwd_f32", "attn_fwd_lse", "attn_fwd_weights", "attn_bwd", "attn_decode",
                 "attn_mha_fwd"):
        monkeypatch.setattr(_lib, name, trap)
    monkeypatch.setattr(_lib, "attn_decode_workspace_bytes", lambda *a: 4096)
    monkeypatch.setattr(_lib, "attn_mha_workspace_bytes", lambda *a: 4096)
    # the wrapper takes the current stream of the inputs' device; no GPU here
    monkeypatch.setattr(torch.cuda, "current_stream", lambda *_a, **_k: type("S", (), {"cuda_stream": 0})())


B, H, T, D = 2, 3, 16, 64
BF = torch.bfloat16


def qkv(dtype=BF, Tq=T):
    return (FakeDeviceTensor((B, H, Tq, D), dtype), FakeDeviceTensor((B, H, T, D), dtype),
            FakeDeviceTensor((B, H, T, D), dtype))


def cpu(shape, dtype):
    return torch.empty(shape, dtype=dtype)


@pytest.mark.parametrize("dtype", [BF, torch.float32])
def test_attention_out_on_host_is_rejected(dtype):
    q, k, v = qkv(dtype)
    with pytest.raises(ValueError, match="out"):
        ops.attention(q, k, v, out=cpu((B, H, T, D), dtype))


def test_attention_out_on_other_gpu_is_rejected():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="out"):
        ops.attention(q, k, v, out=FakeDeviceTensor((B, H, T, D), BF, "cuda:1"))


def test_inputs_on_different_devices_are_rejected():
    q, k, v = qkv()
    k = FakeDeviceTensor((B, H, T, D), BF, "cuda:1")
    with pytest.raises(ValueError, match="k must be"):
        ops.attention(q, k, v)


def test_key_lens_on_host_is_rejected():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="key_lens"):
        ops.attention(q, k, v, key_lens=torch.full((B,), T, dtype=torch.int32),
                      out=FakeDeviceTensor((B, H, T, D), BF))


@pytest.mark.parametrize("which", ["out", "lse"])
def test_attention_lse_outputs_on_host_are_rejected(which):
    q, k, v = qkv()
    kw = {"out": FakeDeviceTensor((B, H, T, D), BF), "lse": FakeDeviceTensor((B, H, T), torch.float32)}
    kw[which] = cpu(kw[which].shape, kw[which].dtype)
    with pytest.raises(ValueError, match=which):
        ops.attention_lse(q, k, v, **kw)


@pytest.mark.parametrize("which", ["out", "lse", "weights"])
def test_attention_weights_outputs_on_host_are_rejected(which):
    q, k, v = qkv()
    shapes = {"out": ((B, H, T, D), BF), "lse": ((B, H, T), torch.float32),
              "weights": ((B, H, T, T), torch.float32)}
    kw = {n: FakeDeviceTensor(*sd) for n, sd in shapes.items()}
    kw[which] = cpu(*shapes[which])
    with pytest.raises(ValueError, match=which):
        ops.attention_weights(q, k, v, **kw)


@pytest.mark.parametrize("which", ["out", "dout", "lse", "dq", "dk", "dv", "delta"])
def test_attention_backward_tensors_on_host_are_rejected(which):
    q, k, v = qkv()
    args = {"out": FakeDeviceTensor((B, H, T, D), BF), "dout": FakeDeviceTensor((B, H, T, D), BF),
            "lse": FakeDeviceTensor((B, H, T), torch.float32)}
    shapes = {"out": ((B, H, T, D), BF), "dout": ((B, H, T, D), BF), "lse": ((B, H, T), torch.float32),
              "dq": ((B, H, T, D), BF), "dk": ((B, H, T, D), BF), "dv": ((B, H, T, D), BF),
              "delta": ((2, B, H, T), torch.float32)}
    for n in ("dq", "dk", "dv", "delta"):
        args[n] = FakeDeviceTensor(*shapes[n])
    args[which] = cpu(*shapes[which])
    with pytest.raises(ValueError, match=which):
        ops.attention_backward(q, k, v, args["out"], args["dout"], args["lse"],
                               **{kk: vv for kk, vv in args.items() if kk not in ("out", "dout", "lse")})


@pytest.mark.parametrize("which", ["out", "workspace"])
def test_decode_outputs_on_host_are_rejected(which):
    q, k, v = qkv(Tq=1)
    kw = {"out": FakeDeviceTensor((B, H, 1, D), BF), "workspace": FakeDeviceTensor((4096,), torch.uint8)}
    kw[which] = cpu(kw[which].shape, kw[which].dtype)
    with pytest.raises(ValueError, match=which):
        ops.decode_attention(q, k, v, **kw)


@pytest.mark.parametrize("which", ["out", "workspace", "wo"])
def test_multi_head_tensors_on_host_are_rejected(which):
    dm = 128
    x = FakeDeviceTensor((B, T, dm), BF)
    ws = {n: FakeDeviceTensor((dm, dm), BF) for n in ("wq", "wk", "wv", "wo")}
    kw = {"out": FakeDeviceTensor((B, T, dm), BF), "workspace": FakeDeviceTensor((4096,), torch.uint8)}
    if which in kw:
        kw[which] = cpu(kw[which].shape, kw[which].dtype)
    else:
        ws["wo"] = cpu((dm, dm), BF)
    with pytest.raises(ValueError, match=which):
        ops.multi_head_attention(x, ws["wq"], ws["wk"], ws["wv"], ws["wo"], heads=2, **kw)


def test_valid_fake_call_reaches_the_library():
    """The stand-ins pass every wrapper check: the trap fires, so the tests above fail on the check."""
    q, k, v = qkv()
    with pytest.raises(AssertionError, match="library was called"):
        ops.attention(q, k, v, out=FakeDeviceTensor((B, H, T, D), BF))


class FakeStream:
    """A HIP stream stand-in on a given GPU."""

    def __init__(self, device):
        self.device = torch.device(device)
        self.cuda_stream = 0x1234


def _all_calls(stream):
    q, k, v = qkv()
    dm = 128
    x = FakeDeviceTensor((B, T, dm), BF)
    w = FakeDeviceTensor((dm, dm), BF)
    return {
        "attention": lambda: ops.attention(q, k, v, out=FakeDeviceTensor((B, H, T, D), BF), stream=stream),
        "attention_lse": lambda: ops.attention_lse(q, k, v, stream=stream,
                                                   out=FakeDeviceTensor((B, H, T, D), BF),
                                                   lse=FakeDeviceTensor((B, H, T), torch.float32)),
        "attention_weights": lambda: ops.attention_weights(
            q, k, v, stream=stream, out=FakeDeviceTensor((B, H, T, D), BF),
            lse=FakeDeviceTensor((B, H, T), torch.float32), weights=FakeDeviceTensor((B, H, T, T), torch.float32)),
        "attention_backward": lambda: ops.attention_backward(
            q, k, v, FakeDeviceTensor((B, H, T, D), BF), FakeDeviceTensor((B, H, T, D), BF),
            FakeDeviceTensor((B, H, T), torch.float32), stream=stream,
            dq=FakeDeviceTensor((B, H, T, D), BF), dk=FakeDeviceTensor((B, H, T, D), BF),
            dv=FakeDeviceTensor((B, H, T, D), BF), delta=FakeDeviceTensor((2, B, H, T), torch.float32)),
        "decode_attention": lambda: ops.decode_attention(
            FakeDeviceTensor((B, H, 1, D), BF), k, v, stream=stream, out=FakeDeviceTensor((B, H, 1, D), BF),
            workspace=FakeDeviceTensor((4096,), torch.uint8)),
        "multi_head_attention": lambda: ops.multi_head_attention(
            x, w, w, w, w, heads=2, stream=stream, out=FakeDeviceTensor((B, T, dm), BF),
            workspace=FakeDeviceTensor((4096,), torch.uint8)),
    }


@pytest.mark.parametrize("name", ["attention", "attention_lse", "attention_weights", "attention_backward",
                                  "decode_attention", "multi_head_attention"])
def test_stream_of_another_gpu_is_rejected(name):
    with pytest.raises(ValueError, match="stream is on cuda:1"):
        _all_calls(FakeStream("cuda:1"))[name]()


@pytest.mark.parametrize("name", ["attention", "attention_lse", "attention_weights", "attention_backward",
                                  "decode_attention", "multi_head_attention"])
def test_stream_of_the_inputs_gpu_reaches_the_library(name):
    with pytest.raises(AssertionError, match="library was called"):
        _all_calls(FakeStream("cuda:0"))[name]()
