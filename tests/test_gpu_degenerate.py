"""Degenerate inputs through every quantizer, bit-exact against the oracle:
all zeros (the 1e-12 scale floor decides the scale), values so small that the
floor still binds, a constant tensor (every element is the amax and encodes
to the largest code), signed zeros (-0 keeps its sign bit), and infinite
inputs (the amax, and with it the scale, is infinite)."""
import numpy as np
import pytest
import torch

import fp8_scaled_quantization_amax_amd as fq
import oracle
from gpu_util import announce, codes_equal, dev, host_input, scales_equal

pytestmark = pytest.mark.gpu

SHAPE = (256, 384)


def cases():
    zeros = torch.zeros(SHAPE, dtype=torch.float32)
    tiny = torch.full(SHAPE, 1e-30, dtype=torch.float32)
    tiny[::3, ::5] = -3e-31
    const = torch.full(SHAPE, -2.5, dtype=torch.float32)
    signed_zero = torch.zeros(SHAPE, dtype=torch.float32)
    signed_zero[1::2] = -0.0
    signed_zero[0, 0] = 1.0
    inf = torch.linspace(-4, 4, SHAPE[0] * SHAPE[1], dtype=torch.float32).reshape(SHAPE)
    inf[3, 7] = float("inf")
    return {"zeros": zeros, "tiny": tiny, "const": const, "signed_zero": signed_zero, "inf": inf}


CASES = cases()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("fmt", [fq.E4M3, fq.E5M2])
@pytest.mark.parametrize("name", list(CASES))
def test_degenerate_inputs(name, fmt, dtype):
    announce("degenerate", name, fmt, dtype)
    x = CASES[name].to(dtype)
    xd = x.to(dev())
    hx = host_input(x)
    # per-tensor current, flat and tiled (transposed copy) paths
    for emit_t in (False, True):
        q, qT, s, a = fq.fp8_quantize_per_tensor(xd, fmt, emit_t=emit_t)
        oq, os_, oa = oracle.quantize_per_tensor(hx, fmt)
        assert scales_equal(s.cpu().numpy(), np.array([os_], np.float32)), (emit_t, s.item(), os_)
        assert scales_equal(a.cpu().numpy(), np.array([oa], np.float32))
        assert codes_equal(q.cpu().numpy(), oq.reshape(SHAPE), fmt), emit_t
        if emit_t:
            assert codes_equal(qT.cpu().numpy(), oq.reshape(SHAPE).T, fmt)
    # 1x128 tiles along rows and 128x1 along columns
    for axis in (0, 1):
        q, _, sc = fq.fp8_quantize_tile1x128(xd, axis, fmt)
        oq, osc = oracle.quantize_tiles(hx, axis, 128, fmt)
        assert codes_equal(q.cpu().numpy(), oq, fmt) and scales_equal(sc.cpu().numpy(), osc), axis
    # 128x128 blocks
    q, _, sc = fq.fp8_quantize_block128x128(xd, fmt)
    oq, osc = oracle.quantize_blocks(hx, 128, 128, fmt)
    assert codes_equal(q.cpu().numpy(), oq, fmt) and scales_equal(sc.cpu().numpy(), osc)
    # MX32 along rows and along columns
    for axis in (0, 1):
        q, _, e8 = fq.fp8_quantize_mx32(xd, axis, fmt)
        oq, oe8 = oracle.quantize_tiles(hx, axis, 32, fmt, mx=True)
        assert codes_equal(q.cpu().numpy(), oq, fmt) and np.array_equal(e8.cpu().numpy(), oe8), axis
    if name == "zeros":
        assert (q.cpu().numpy() == 0).all()
    if name == "const":
        q, _, _, _ = fq.fp8_quantize_per_tensor(xd, fmt)
        top = 0x7E if fmt == fq.E4M3 else 0x7B
        assert (q.cpu().numpy() == (0x80 | top)).all()   # -2.5 is the amax: every code is -max


@pytest.mark.parametrize("fmt", [fq.E4M3, fq.E5M2])
@pytest.mark.parametrize("name", list(CASES))
def test_degenerate_inputs_rowwise_sr_rht(name, fmt):
    """The same inputs through the rowwise, stochastically rounded and
    Hadamard-transformed quantizers (bf16 in)."""
    announce("degenerate rowwise/sr/rht", name, fmt)
    x = CASES[name].to(torch.bfloat16)
    xd = x.to(dev())
    hx = host_input(x)
    for axis in (0, 1):
        q, _, sc = fq.fp8_quantize_rowwise(xd, axis, fmt, emit_t=axis == 1)
        oq, osc = oracle.quantize_rowwise(hx, axis, fmt)
        assert codes_equal(q.cpu().numpy(), oq.reshape(SHAPE), fmt), axis
        assert scales_equal(sc.cpu().numpy(), osc), axis
    q, _, s, a = fq.fp8_quantize_per_tensor_sr(xd, fmt, 1234, 5)
    oq, os_, oa = oracle.quantize_per_tensor_sr(hx, fmt, 1234, 5)
    assert scales_equal(s.cpu().numpy(), np.array([os_], np.float32))
    assert codes_equal(q.cpu().numpy(), oq.reshape(SHAPE), fmt)
    q, _, s, a = fq.fp8_quantize_per_tensor_rht(xd, fmt, 99)
    oq, os_, oa = oracle.quantize_per_tensor_rht(hx, fmt, 99)
    assert scales_equal(s.cpu().numpy(), np.array([os_], np.float32))
    assert codes_equal(q.cpu().numpy(), oq.reshape(SHAPE), fmt)
