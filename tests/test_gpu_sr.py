"""GPU parity of the stochastically rounded cast (per-tensor current scaling,
Philox4x32-10 words): codes bit-exact against the oracle for the same seed and
offset, at small ragged shapes and at a full [15872, 4096] gradient."""
import numpy as np
import pytest
import torch

import fp8_scaled_quantization_amax_amd as fq
import oracle
import workloads
from gpu_util import announce, codes_equal, dev, host_input

pytestmark = pytest.mark.gpu


def check_sr(x, fmt, seed, offset, emit_t=False, saturate=False):
    q, qT, s, a = fq.fp8_quantize_per_tensor_sr(x.to(dev()), fmt, seed, offset, emit_t=emit_t, saturate=saturate)
    torch.cuda.synchronize()
    oq, os_, oa = oracle.quantize_per_tensor_sr(host_input(x), fmt, seed, offset, saturate)
    oq = oq.reshape(q.shape)
    assert s.item() == os_ or (np.isnan(s.item()) and np.isnan(os_))
    assert a.item() == oa or (np.isnan(a.item()) and np.isnan(oa))
    assert codes_equal(q.cpu().numpy(), oq, fmt)
    if emit_t:
        assert codes_equal(qT.cpu().numpy(), oq.T, fmt)
    return q


@pytest.mark.parametrize("shape", [(1, 1), (3, 5), (37, 53), (16, 4096), (129, 136), (1000, 24)],
                         ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("fmt", [fq.E5M2, fq.E4M3], ids=["e5m2", "e4m3"])
def test_sr_bit_exact(shape, dtype, fmt):
    announce("sr", shape, dtype, fmt)
    x = workloads.normal(shape, 1.0, 9000 + shape[0] + shape[1], dtype)
    check_sr(x, fmt, seed=0x0123456789ABCDEF, offset=(1 << 40) + 5, emit_t=shape[0] > 1)


def test_sr_is_deterministic_and_offset_sensitive():
    announce("sr determinism")
    x = workloads.normal((256, 512), 1.0, 9100, torch.bfloat16).to(dev())
    q1 = fq.fp8_quantize_per_tensor_sr(x, fq.E5M2, 7, 0)[0]
    q2 = fq.fp8_quantize_per_tensor_sr(x, fq.E5M2, 7, 0)[0]
    q3 = fq.fp8_quantize_per_tensor_sr(x, fq.E5M2, 7, 1)[0]
    q4 = fq.fp8_quantize_per_tensor_sr(x, fq.E5M2, 8, 0)[0]
    assert torch.equal(q1, q2)
    assert not torch.equal(q1, q3) and not torch.equal(q1, q4)


def test_sr_saturate_and_nan():
    announce("sr saturate / nan")
    x = workloads.normal((64, 96), 1.0, 9200, torch.float32)
    check_sr(x, fq.E4M3, 3, 4, saturate=True)
    x[7, 9] = float("nan")
    check_sr(x, fq.E5M2, 3, 4)


def test_sr_full_size_gradient():
    """A gradient-shaped tensor at full size: bf16 [15872, 4096] ~ N(0,1), E5M2,
    with the K-major copy a wgrad operand needs."""
    announce("sr full size")
    g = workloads.normal((workloads.M_TOKENS, workloads.HIDDEN), 1.0, 9300, torch.bfloat16)
    check_sr(g, fq.E5M2, seed=2024, offset=17, emit_t=True)


@pytest.mark.parametrize("fmt", [fq.E4M3, fq.E5M2], ids=["e4m3", "e5m2"])
def test_sr_amax_element_stays_finite(fmt):
    """The amax element's quotient lands one ulp above fmax and its word would
    round it up: the code is the largest finite one, on the GPU as in the
    oracle (a step past fmax would be NaN / Inf)."""
    import sr_search
    fmax = 448.0 if fmt == fq.E4M3 else 57344.0
    a = sr_search.bf16_amax_one_ulp_above(fmax)
    s = np.float32(a) / np.float32(fmax)
    v = float(np.float32(a) / s)
    D = 32.0 if fmt == fq.E4M3 else 8192.0
    frac32 = int(np.floor((v / D - np.floor(v / D)) * 2.0 ** 32))
    seed = 0x5EED
    off = sr_search.find_offset(seed, 0, (1 << 32) - frac32)
    assert off is not None and oracle.sr_word(seed, off, 0) >= (1 << 32) - frac32
    announce("sr amax element", fmt, off)
    x = torch.from_numpy((np.random.default_rng(12).standard_normal(4096) * 0.25).astype(np.float32))
    x[0] = a
    x = x.to(torch.bfloat16).reshape(16, 256)
    q = check_sr(x, fmt, seed, off)
    assert int(q[0, 0].item()) == (0x7E if fmt == fq.E4M3 else 0x7B)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("fmt", [fq.E5M2, fq.E4M3], ids=["e5m2", "e4m3"])
def test_sr_outliers_misaligned(dtype, fmt):
    """Outliers x1e4 put most quotients below the format's smallest normal,
    where the rounding takes its below-2^emin path in nearly every wave; the
    input starts one element past an aligned address (no vector loads), and
    the element count leaves a partial group of four."""
    announce("sr outliers misaligned", dtype, fmt)
    rows, cols = 300, 257
    flat = workloads.normal((rows * cols + 1,), 1.0, 9400, dtype)
    big = 1e4 if fmt == fq.E4M3 else 1e9   # E5M2's normal range reaches 2^-14 * fmax below the amax
    flat[1 + torch.randperm(rows * cols, generator=torch.Generator().manual_seed(9401))[:40]] *= big
    x = flat[1:].view(rows, cols)
    xd = flat.to(dev())[1:].view(rows, cols)
    assert xd.data_ptr() % 8 != 0
    q, _, s, a = fq.fp8_quantize_per_tensor_sr(xd, fmt, 0xABCDEF, 3)
    torch.cuda.synchronize()
    oq, os_, oa = oracle.quantize_per_tensor_sr(host_input(x), fmt, 0xABCDEF, 3, False)
    assert s.item() == os_ and a.item() == oa
    assert codes_equal(q.cpu().numpy(), oq.reshape(q.shape), fmt)
    small = (q.cpu().numpy() & 0x7F) < (0x08 if fmt == fq.E4M3 else 0x04)   # below the smallest normal code
    assert small.mean() > 0.5
