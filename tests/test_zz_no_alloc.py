"""The allocation-free per-tensor quantizer (fp8_quantize_per_tensor_noalloc):
called through the C ABI, it gives bitwise the workspace form's outputs and the
oracle's, on consecutive calls of different sizes (the second smaller), under
current and delayed scaling, and inside a replayed graph."""
import numpy as np
import pytest
import torch

import fp8_scaled_quantization_amax_amd as fq
import oracle
import workloads
from gpu_util import announce, codes_equal, dev, host_input

pytestmark = pytest.mark.gpu


def both(x, fmt, emit_t, scaling=fq.CURRENT, st_ws=None, st_na=None, count_overflow=False):
    """The workspace form and the allocation-free form on the same input."""
    a = fq.fp8_quantize_per_tensor(x, fmt, scaling, st_ws, emit_t=emit_t, count_overflow=count_overflow)
    b = fq.fp8_quantize_per_tensor_noalloc(x, fmt, scaling, st_na, emit_t=emit_t, count_overflow=count_overflow)
    torch.cuda.synchronize()
    return a, b


def assert_same(a, b):
    for u, v in zip(a, b):
        if u is None:
            assert v is None
        else:
            assert torch.equal(u, v)


def test_consecutive_calls_second_smaller():
    """A full-size bf16 tensor with its K-major copy, then a small ragged fp32
    one: each call equals the workspace form and the oracle bit for bit."""
    big = workloads.quantize_tensor()
    small = workloads.normal((1000, 24), 3.0, 9900, torch.float32)
    for x, fmt, emit_t in ((big, fq.E4M3, True), (small, fq.E5M2, True), (small[:37, :5].contiguous(), fq.E4M3,
                                                                             False)):
        announce("no-alloc current", tuple(x.shape), x.dtype, fmt)
        a, b = both(x.to(dev()), fmt, emit_t)
        assert_same(a, b)
        oq, os_, oa = oracle.quantize_per_tensor(host_input(x), fmt)
        assert b[2].item() == os_ and b[3].item() == oa
        assert codes_equal(b[0].cpu().numpy(), oq.reshape(x.shape), fmt)


def test_delayed_sequence_matches_workspace_form():
    """The 17-step delayed sequence with its 40-sigma spike (overflow counted):
    codes, scales and the whole state equal the workspace form's at every
    step, and the state walks the oracle's history."""
    M, K = 2048, 1024
    st_ws, st_na = fq.DelayedState(dev()), fq.DelayedState(dev())
    ost = oracle.DelayedState()
    for t, x, spike in workloads.delayed_steps(M=M, K=K, steps=17):
        announce("no-alloc delayed step", t)
        a, b = both(x.to(dev()), fq.E4M3, t % 2 == 0, fq.DELAYED, st_ws, st_na, count_overflow=True)
        assert_same(a, b)
        assert torch.equal(st_ws.buf, st_na.buf)
        oq, os_, _ = oracle.quantize_delayed(host_input(x), fq.E4M3, ost)
        assert b[2].item() == os_ and np.array_equal(st_na.history.cpu().numpy(), ost.hist)
        if spike is not None:
            assert st_na.overflows.item() == 1


def test_graph_replays_match_eager():
    """Delayed then current calls captured in one graph and replayed three
    times, with eager calls between the replays: every replay's outputs equal
    the eager ones (the counters are cleared by a kernel in the graph)."""
    announce("no-alloc graph")
    x1 = workloads.normal((1536, 640), 1.0, 9910, torch.bfloat16).to(dev())
    x2 = workloads.normal((384, 2048), 2.0, 9911, torch.bfloat16).to(dev())
    out1 = (torch.empty((1536, 640), dtype=torch.uint8, device=dev()), None,
            torch.empty(1, device=dev()), torch.empty(1, device=dev()))
    out2 = (torch.empty((384, 2048), dtype=torch.uint8, device=dev()),
            torch.empty((2048, 384), dtype=torch.uint8, device=dev()),
            torch.empty(1, device=dev()), torch.empty(1, device=dev()))
    st_g, st_e = fq.DelayedState(dev()), fq.DelayedState(dev())
    # warm the history so the graph's delayed call takes the single-pass path
    for st in (st_g, st_e):
        fq.fp8_quantize_per_tensor_noalloc(x1, fq.E4M3, fq.DELAYED, st)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fq.fp8_quantize_per_tensor_noalloc(x1, fq.E4M3, fq.DELAYED, st_g, out=out1)
            fq.fp8_quantize_per_tensor_noalloc(x2, fq.E5M2, fq.CURRENT, None, emit_t=True, out=out2)
    for r in range(3):
        g.replay()
        torch.cuda.synchronize()
        e1 = fq.fp8_quantize_per_tensor_noalloc(x1, fq.E4M3, fq.DELAYED, st_e)
        e2 = fq.fp8_quantize_per_tensor_noalloc(x2, fq.E5M2, fq.CURRENT, None, emit_t=True)
        torch.cuda.synchronize()
        assert_same(out1, e1)
        assert_same(out2, e2)
        assert torch.equal(st_g.buf, st_e.buf), r
        x1.mul_(1.5)   # the next step's activation grows: the history moves on


def test_errors_before_any_gpu_work():
    L = fq.lib()
    fake = torch.empty(16, dtype=torch.uint8, device=dev())
    p = fake.data_ptr()
    assert L.fp8_quantize_per_tensor_noalloc(None, fq.BF16, 4, 4, fq.E4M3, fq.CURRENT, None, p, None, p, None, 0,
                                             None) == fq.EINVAL
    assert L.fp8_quantize_per_tensor_noalloc(p, fq.BF16, 4, 4, fq.E4M3, fq.DELAYED, None, p, None, p, None, 0,
                                             None) == fq.EINVAL
    assert L.fp8_quantize_per_tensor_noalloc(p, fq.BF16, 4, 4, fq.E4M3, fq.CURRENT, None, p, None, p, None,
                                             fq.COUNT_OVERFLOW, None) == fq.EINVAL
