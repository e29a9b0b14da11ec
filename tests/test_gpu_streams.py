"""The library enqueues on the caller's stream and keeps no state between
calls beyond what the caller owns, so its calls run on a side stream and
inside a captured HIP graph exactly as they run eagerly (bitwise)."""
import pytest
import torch

import fp8_scaled_quantization_amax_amd as fq
import workloads
from gpu_util import announce, dev

pytestmark = pytest.mark.gpu

AC = fq.GemmOperand.autocast
Q = fq.GemmOperand.quantized


def inputs():
    A = workloads.normal((528, 1024), 1.0 / 32, 501, torch.bfloat16).to(dev())
    B = workloads.normal((400, 1024), 1.0 / 32, 502, torch.bfloat16).to(dev())
    return A, B


def test_side_stream_matches_default_stream():
    announce("side stream")
    A, B = inputs()
    q0, _, s0, a0 = fq.fp8_quantize_per_tensor(A, fq.E4M3)
    C0 = fq.fp8_gemm_scaled_NT(528, 400, 1024, AC(A, fq.E4M3), AC(B, fq.E4M3), torch.bfloat16)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=dev())
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q1, _, s1, a1 = fq.fp8_quantize_per_tensor(A, fq.E4M3)
        C1 = fq.fp8_gemm_scaled_NT(528, 400, 1024, AC(A, fq.E4M3), AC(B, fq.E4M3), torch.bfloat16)
    side.synchronize()
    assert torch.equal(q0, q1) and torch.equal(s0, s1) and torch.equal(a0, a1)
    assert torch.equal(C0, C1)


def test_graph_replays_match_eager():
    """Quantize (per-tensor current, with a K-major copy) and a pre-quantized
    GEMM on those codes, captured once and replayed three times with eager
    library calls in between; every replay equals the eager result."""
    announce("graph replay")
    A, B = inputs()
    ws = fq.reduce_workspace(dev())
    qb, _, sb, _ = fq.fp8_quantize_per_tensor(B, fq.E4M3)
    C = torch.empty((528, 400), dtype=torch.bfloat16, device=dev())
    q = torch.empty((528, 1024), dtype=torch.uint8, device=dev())

    def work():
        qa, qaT, sa, _ = fq.fp8_quantize_per_tensor(A, fq.E4M3, emit_t=True, ws=ws)
        q.copy_(qa)
        fq.fp8_gemm_scaled_NT(528, 400, 1024, Q(qa, fq.E4M3, sa), Q(qb, fq.E4M3, sb), torch.bfloat16, out=C)
        return qaT

    qT_eager = work().clone()
    torch.cuda.synchronize()
    q_eager, C_eager = q.clone(), C.clone()
    s = torch.cuda.Stream(device=dev())
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        qT_graph = work()
    other = workloads.normal((256, 512), 4.0, 503, torch.bfloat16).to(dev())
    for replay in range(3):
        q.zero_()
        C.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(q, q_eager), replay
        assert torch.equal(qT_graph, qT_eager), replay
        assert torch.equal(C, C_eager), replay
        fq.fp8_quantize_per_tensor(other, fq.E5M2, ws=ws)   # eager work between replays
        torch.cuda.synchronize()


def test_graph_replays_granular_and_autocast_gemms():
    """The persistent block-scaled GEMM (128x128-block B on fprop, row scales
    on both wgrad operands), the MX32 GEMM and an autocast GEMM (amax grid,
    cast and completion counters in its workspace), captured in one graph and
    replayed three times with eager library calls in between: every replay
    equals the eager results bitwise."""
    from test_gpu_gemm import block_scaled_codes, mx_codes
    announce("graph replay: block-scaled, MX and autocast GEMMs")
    M, N, K = 528, 400, 1024   # K % 512 == 0: the persistent granular kernels
    A, B = inputs()
    At, Bt = workloads.gemm_operands("TN", M, N, K, seed=511, std=1.0, outlier_rows=0.01)
    ba, bb = block_scaled_codes("NT", A, B, fq.E4M3, fq.E4M3)[:2]
    ta, tb = block_scaled_codes("TN", At, Bt, fq.E5M2, fq.E4M3)[:2]
    ma, mb = mx_codes("NT", A, B, fq.E4M3, fq.E4M3)[:2]
    need = fq.gemm_workspace_bytes("NT", M, N, K, AC(A, fq.E4M3), AC(B, fq.E4M3))
    ws = fq._ws(need, dev())
    outs = [torch.empty((M, N), dtype=torch.bfloat16, device=dev()) for _ in range(4)]

    def work():
        fq.fp8_gemm_scaled_NT(M, N, K, ba, bb, torch.bfloat16, out=outs[0])
        fq.fp8_gemm_scaled_TN(M, N, K, ta, tb, torch.bfloat16, out=outs[1])
        fq.fp8_gemm_scaled_NT(M, N, K, ma, mb, torch.bfloat16, out=outs[2])
        fq.fp8_gemm_scaled_NT(M, N, K, AC(A, fq.E4M3), AC(B, fq.E4M3), torch.bfloat16, out=outs[3], ws=ws)

    work()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    s = torch.cuda.Stream(device=dev())
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    other = workloads.normal((256, 512), 4.0, 512, torch.bfloat16).to(dev())
    for replay in range(3):
        for o in outs:
            o.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for k, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o, e), (replay, k)
        fq.fp8_gemm_scaled_NT(256, 256, 512, AC(other[:, :512], fq.E5M2), AC(other[:256], fq.E4M3),
                              torch.bfloat16)   # eager work between replays
        torch.cuda.synchronize()


def test_delayed_scaling_replayed_graph_follows_the_oracle():
    """The delayed state lives in device memory, so one captured delayed cast,
    replayed once per step with that step's data copied into its input
    buffer, walks the same 17-step sequence (16 warm-up steps, then a
    40-sigma spike) as the oracle: scale, codes and history at every step."""
    import numpy as np
    import oracle
    from gpu_util import codes_equal, host_input
    announce("delayed scaling in a graph")
    shape = (256, 512)
    steps = list(workloads.delayed_steps(M=shape[0], K=shape[1], steps=17))
    x_buf = torch.empty(shape, dtype=torch.bfloat16, device=dev())
    st = fq.DelayedState(dev())
    ws = fq.reduce_workspace(dev())
    s = torch.cuda.Stream(device=dev())
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm-up on a throwaway state
        fq.fp8_quantize_per_tensor(x_buf.zero_(), fq.E4M3, fq.DELAYED, fq.DelayedState(dev()), ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        q, _, sc, _ = fq.fp8_quantize_per_tensor(x_buf, fq.E4M3, fq.DELAYED, st, ws=ws, count_overflow=True)
    ost = oracle.DelayedState()
    for t, x, spike in steps:
        x_buf.copy_(x.to(dev()))
        graph.replay()
        torch.cuda.synchronize()
        oq, os_, _ = oracle.quantize_delayed(host_input(x), fq.E4M3, ost)
        assert sc.item() == os_, t
        assert codes_equal(q.cpu().numpy(), oq.reshape(shape), fq.E4M3), t
        assert np.array_equal(st.history.cpu().numpy(), ost.hist), t
        assert st.overflows.item() == oracle.overflow_count(host_input(x), os_, fq.E4M3), t


def test_concurrent_streams_with_their_own_workspaces():
    """Two streams running autocast GEMMs and quantize calls at the same time,
    each with its own workspace: every result equals the eager one."""
    announce("concurrent streams")
    A, B = inputs()
    A2 = (A * 3).contiguous()
    C_ref = fq.fp8_gemm_scaled_NT(528, 400, 1024, AC(A, fq.E4M3), AC(B, fq.E4M3), torch.bfloat16)
    C2_ref = fq.fp8_gemm_scaled_NT(528, 400, 1024, AC(A2, fq.E5M2), AC(B, fq.E4M3), torch.bfloat16)
    q_ref = fq.fp8_quantize_per_tensor(A2, fq.E5M2)[0]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(device=dev()), torch.cuda.Stream(device=dev())
    need = fq.gemm_workspace_bytes("NT", 528, 400, 1024, AC(A, fq.E4M3), AC(B, fq.E4M3))
    ws1, ws2 = fq._ws(need, dev()), fq._ws(need, dev())
    r1, r2 = fq.reduce_workspace(dev()), fq.reduce_workspace(dev())
    outs1, outs2 = [], []
    for it in range(8):
        with torch.cuda.stream(s1):
            outs1.append(fq.fp8_gemm_scaled_NT(528, 400, 1024, AC(A, fq.E4M3), AC(B, fq.E4M3), torch.bfloat16,
                                               ws=ws1))
            outs1.append(fq.fp8_quantize_per_tensor(A2, fq.E5M2, ws=r1)[0])
        with torch.cuda.stream(s2):
            outs2.append(fq.fp8_gemm_scaled_NT(528, 400, 1024, AC(A2, fq.E5M2), AC(B, fq.E4M3), torch.bfloat16,
                                               ws=ws2))
            outs2.append(fq.fp8_quantize_per_tensor(A2, fq.E5M2, ws=r2)[0])
    torch.cuda.synchronize()
    for k in range(0, len(outs1), 2):
        assert torch.equal(outs1[k], C_ref) and torch.equal(outs2[k], C2_ref)
        assert torch.equal(outs1[k + 1], q_ref) and torch.equal(outs2[k + 1], q_ref)
