"""GPU parity of the random Hadamard transform + per-tensor quantization of
wgrad operands: codes, scale and amax bit-exact against the oracle (same fp32
butterfly order, same Philox signs), and the wgrad GEMM on two operands
transformed with one seed within the fp32-output tolerance."""
import numpy as np
import pytest
import torch

import fp8_scaled_quantization_amax_amd as fq
import oracle
import workloads
from gpu_util import announce, codes_equal, dev, gemm_close, host_input

pytestmark = pytest.mark.gpu


def check_rht(x, fmt, seed, emit_t=True):
    q, qT, s, a = fq.fp8_quantize_per_tensor_rht(x.to(dev()), fmt, seed, emit_t=emit_t)
    torch.cuda.synchronize()
    oq, os_, oa = oracle.quantize_per_tensor_rht(host_input(x), fmt, seed)
    assert s.item() == os_ and a.item() == oa
    assert codes_equal(q.cpu().numpy(), oq, fmt)
    if emit_t:
        assert codes_equal(qT.cpu().numpy(), oq.T, fmt)
    return q, qT, s, oq, os_


@pytest.mark.parametrize("shape", [(16, 8), (32, 24), (16, 64), (48, 512), (256, 4096), (1024, 520)],
                         ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("fmt", [fq.E5M2, fq.E4M3], ids=["e5m2", "e4m3"])
def test_rht_bit_exact(shape, dtype, fmt):
    """16x64: one partial wave of 8 units in one 16-row block (the wave-shared
    signs with lanes 8-63 idle); 48x512: every wave inside one block; 32x24 and
    1024x520: waves spanning blocks (per-lane signs)."""
    announce("rht", shape, dtype, fmt)
    x = workloads.normal(shape, 1.0, 9500 + shape[0] + shape[1], dtype)
    x[shape[0] // 3, shape[1] // 2] = 500.0   # an outlier to spread
    check_rht(x, fmt, seed=0xFEEDFACE12345678)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("fmt", [fq.E5M2, fq.E4M3], ids=["e5m2", "e4m3"])
@pytest.mark.parametrize("outlier", [1.0, None], ids=["with_outlier", "all_tiny"])
def test_rht_tiny_values(dtype, fmt, outlier):
    """Subnormal inputs, so that H16 (d x) falls below 2^-124 and a quarter of it
    is inexact: with a normal outlier setting the scale (tiny quotients, zero
    codes of either sign) and with every value tiny (the amax itself a rounded
    quarter, the scale at its 1e-12 floor).  Codes, scale and amax bit-exact."""
    announce("rht tiny", dtype, fmt, outlier)
    x = workloads.normal((64, 520), 1e-39, 9800, dtype)
    assert (x != 0).float().mean() > 0.5 and x.abs().max() < 1e-37
    if outlier is not None:
        x[17, 300] = outlier
    check_rht(x, fmt, seed=0x5EED)


def test_rht_full_size_gradient():
    """bf16 [15872, 4096] ~ N(0,1) with a few outliers, E5M2, with the K-major copy."""
    announce("rht full size")
    g = workloads.normal((workloads.M_TOKENS, workloads.HIDDEN), 1.0, 9600, torch.bfloat16)
    g[123, 45] = 1e3
    g[9000, 4000] = -2e3
    check_rht(g, fq.E5M2, seed=31)


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_rht_wgrad_gemm(out):
    """dW = (R G)^T (R X): both operands transformed with one seed and quantized
    (E5M2 gradient, E4M3 activation), the TN GEMM on their K-major copies, against
    the oracle's exact product of the same codes."""
    announce("rht wgrad", out)
    T, N, K = 1024, 256, 384
    G = workloads.normal((T, N), 1.0, 9700, torch.bfloat16)
    G[77, 5] = 800.0
    X = workloads.normal((T, K), 1.0, 9701, torch.bfloat16)
    qg, qgT, sg, oqg, osg = check_rht(G, fq.E5M2, seed=99)
    qx, qxT, sx, oqx, osx = check_rht(X, fq.E4M3, seed=99)
    Q = fq.GemmOperand.quantized
    C = fq.fp8_gemm_scaled_TN(N, K, T, Q(qg, fq.E5M2, sg, kmajor=qgT), Q(qx, fq.E4M3, sx, kmajor=qxT), out)
    ref = oracle.gemm_tn(oqg, oqx, fq.E5M2, fq.E4M3, oracle.Scale("tensor", osg), oracle.Scale("tensor", osx))
    assert gemm_close(C, ref, out)
