"""The torch wrappers reject caller-supplied outputs that the kernels could
not write safely (the C ABI sees only addresses, so shape, type and layout
are checked in the binding), before anything reaches the library or a
device.  CPU tensors suffice: every call here fails its checks first."""
import pytest
import torch

import exact_attention_32_amd as fa


def _qkv(dtype=torch.bfloat16, shape=(1, 2, 8, 16)):
    return tuple(torch.zeros(shape, dtype=dtype) for _ in range(3))


def test_forward_rejects_bad_out_and_lse():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="shape"):
        fa.forward(q, k, v, out=torch.empty(1, 2, 8, 8, dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="out must be"):
        fa.forward(q, k, v, out=torch.empty(1, 2, 8, 16, dtype=torch.float32))
    with pytest.raises(ValueError, match="last dimension"):
        fa.forward(q, k, v, out=torch.empty(1, 2, 16, 8, dtype=torch.bfloat16).transpose(2, 3))
    with pytest.raises(ValueError, match="shape"):
        fa.forward(q, k, v, lse=torch.empty(1, 2, 7))
    with pytest.raises(TypeError, match="lse must be"):
        fa.forward(q, k, v, lse=torch.empty(1, 2, 8, dtype=torch.float16))
    with pytest.raises(ValueError, match="contiguous"):
        fa.forward(q, k, v, lse=torch.empty(1, 8, 2).transpose(1, 2))
    q32, k32, v32 = _qkv(torch.float32)
    with pytest.raises(ValueError, match="contiguous"):
        fa.forward(q32, k32, v32, out=torch.empty(1, 8, 2, 16).transpose(1, 2))
    # well-formed outputs, but host tensors: rejected as such
    with pytest.raises(ValueError, match="device tensors"):
        fa.forward(q, k, v, out=torch.empty_like(q), lse=torch.empty(1, 2, 8))


def test_backward_rejects_bad_outputs():
    q, k, v = _qkv()
    o, dout = torch.zeros_like(q), torch.zeros_like(q)
    lse = torch.zeros(1, 2, 8)
    with pytest.raises(ValueError, match="shape"):
        fa.backward(q, k, v, o, torch.zeros(1, 2, 9), dout)
    with pytest.raises(TypeError, match="lse must be"):
        fa.backward(q, k, v, o, torch.zeros(1, 2, 8, dtype=torch.float64), dout)
    good = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q))
    with pytest.raises(ValueError, match="dk must have shape"):
        fa.backward(q, k, v, o, lse, dout, out=(good[0], torch.empty(1, 2, 8, 32, dtype=q.dtype),
                                                good[2]))
    with pytest.raises(TypeError, match="dv must be"):
        fa.backward(q, k, v, o, lse, dout, out=(good[0], good[1], torch.empty(1, 2, 8, 16)))
    with pytest.raises(ValueError, match="triple"):
        fa.backward(q, k, v, o, lse, dout, out=good[:2])
    with pytest.raises(ValueError, match="device tensors"):
        fa.backward(q, k, v, o, lse, dout, out=good)


def test_decode_rejects_bad_out():
    q = torch.zeros(1, 2, 1, 16, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 40, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="shape"):
        fa.decode(q, k, k.clone(), out=torch.empty(1, 2, 2, 16, dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="out must be"):
        fa.decode(q, k, k.clone(), out=torch.empty(1, 2, 1, 16, dtype=torch.float16))
    with pytest.raises(ValueError, match="device tensors"):
        fa.decode(q, k, k.clone(), out=torch.empty_like(q))
