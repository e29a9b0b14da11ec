"""FP8Q_COUNT_OVERFLOW against the oracle: the number of elements a delayed
cast overflows (E4M3 NaN, E5M2 Inf from finite inputs; clamped under
saturation) lands in the delayed state, equal to the oracle's count with the
same delayed scale, on the flat and the tiled (transposing) cast, in the
quantize call and inside an autocast GEMM."""
import numpy as np
import pytest
import torch

import fp8_scaled_quantization_amax_amd as fq
import oracle
import workloads
from gpu_util import announce, codes_equal, dev, host_input

pytestmark = pytest.mark.gpu

FMTS = [fq.E4M3, fq.E5M2]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("emit_t", [False, True])
@pytest.mark.parametrize("shape", [(512, 1024), (300, 200)])
def test_count_through_delayed_sequence_with_spike(shape, emit_t, fmt):
    """17 delayed steps (16 warm-up, then the 40-sigma spike): after every
    call the state holds the oracle's count for that step's scale."""
    announce("overflow count sequence", shape, emit_t, fmt)
    st = fq.DelayedState(dev())
    ost = oracle.DelayedState()
    for t, x, spike in workloads.delayed_steps(M=shape[0], K=shape[1], steps=17):
        q, _, s, _ = fq.fp8_quantize_per_tensor(x.to(dev()), fmt, fq.DELAYED, st, emit_t=emit_t,
                                                count_overflow=True)
        oq, os_, _ = oracle.quantize_delayed(host_input(x), fmt, ost)
        assert s.item() == os_, t
        want = oracle.overflow_count(host_input(x), os_, fmt)
        assert st.overflows.item() == want, (t, st.overflows.item(), want)
        if spike is not None and fmt == fq.E4M3:
            assert want >= 1   # the spike overflows the delayed scale, as in check [3]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("emit_t", [False, True])
def test_count_many_overflows_with_and_without_saturation(emit_t, fmt):
    """A history far below the data: most elements overflow; the count is
    the same whether they become NaN / Inf or are clamped, and a call
    without the flag leaves 0."""
    announce("overflow count many", emit_t, fmt)
    x = workloads.normal((256, 384), 1.0, 31, torch.float32)
    x[3, 4] = float("inf")     # non-finite inputs are not counted
    x[7, 9] = float("nan")
    small = (x.nan_to_num(0.0, 0.0, 0.0) * 1e-3).contiguous()
    for sat in (False, True):
        st = fq.DelayedState(dev())
        ost = oracle.DelayedState()
        fq.fp8_quantize_per_tensor(small.to(dev()), fmt, fq.DELAYED, st, count_overflow=True)
        oracle.quantize_delayed(host_input(small), fmt, ost)
        assert st.overflows.item() == 0
        q, _, s, _ = fq.fp8_quantize_per_tensor(x.to(dev()), fmt, fq.DELAYED, st, emit_t=emit_t, saturate=sat,
                                                count_overflow=True)
        oq, os_, _ = oracle.quantize_delayed(host_input(x), fmt, ost, saturate=sat)
        assert s.item() == os_
        assert codes_equal(q.cpu().numpy(), oq.reshape(q.shape), fmt)
        want = oracle.overflow_count(host_input(x), os_, fmt)
        assert want > 1000
        assert st.overflows.item() == want
        # the same cast without the flag: nothing counted
        fq.fp8_quantize_per_tensor(x.to(dev()), fmt, fq.DELAYED, st, saturate=sat)
        assert st.overflows.item() == 0


def test_count_inside_autocast_gemm():
    """A delayed autocast operand with the flag: the GEMM's own cast counts."""
    announce("overflow count autocast gemm")
    M, N, K = 256, 128, 256
    A = workloads.normal((M, K), 1.0, 41, torch.bfloat16)
    B = workloads.normal((N, K), 1.0 / 16, 42, torch.bfloat16)
    st = fq.DelayedState(dev())
    ost = oracle.DelayedState()
    ws_small = (A.float() * 1e-2).to(torch.bfloat16)
    C = None
    for step, a in enumerate((ws_small, A)):
        opa = fq.GemmOperand.autocast(a.to(dev()), fq.E4M3, fq.PER_TENSOR, fq.DELAYED, st, count_overflow=True)
        opb = fq.GemmOperand.autocast(B.to(dev()), fq.E4M3)
        C = fq.fp8_gemm_scaled_NT(M, N, K, opa, opb, torch.float32)
        torch.cuda.synchronize()
        _, os_, _ = oracle.quantize_delayed(host_input(a), fq.E4M3, ost)
        want = oracle.overflow_count(host_input(a), os_, fq.E4M3)
        assert st.overflows.item() == want, step
    assert want > 100
    assert C is not None
