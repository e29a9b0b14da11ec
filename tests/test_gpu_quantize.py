"""GPU parity of amax and the quantizers against the CPU oracle: codes and
scales bit-exact, on seeded inputs spanning several tiles with ragged tails,
and at the full quantize workload size (bf16 [15872, 4096])."""
import numpy as np
import pytest
import torch

import fp8_scaled_quantization_amax_amd as fq
import oracle
import workloads
from gpu_util import announce, codes_equal, dev, host_input, scales_equal

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1), (3, 200), (300, 200), (257, 1030), (128, 128), (1000, 4096)]
FMTS = [fq.E4M3, fq.E5M2]
DTYPES = [torch.bfloat16, torch.float32]


def make(shape, dtype, seed):
    x = workloads.quantize_tensor(rows=shape[0], cols=shape[1], seed=seed)
    return x.to(dtype)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", SHAPES + [(1, 1000003)])
def test_amax(shape, dtype):
    announce("amax", shape, dtype)
    x = make(shape, dtype, 10)
    got = fq.fp8_amax(x.to(dev())).item()
    assert got == oracle.amax(host_input(x))
    # unaligned start (offset of one element) takes the scalar path
    if x.numel() > 1:
        xd = x.reshape(-1).to(dev())[1:]
        assert fq.fp8_amax(xd).item() == oracle.amax(host_input(x.reshape(-1)[1:]))


def test_amax_reused_workspace():
    """One workspace across many calls (the completion counter resets itself),
    sizes from one block to the full grid, both element types."""
    announce("amax reused workspace")
    ws = fq.reduce_workspace(dev())
    for i, (n, dtype) in enumerate([(7, torch.float32), (1 << 20, torch.bfloat16), (15872 * 4096, torch.bfloat16),
                                    (3 << 18, torch.float32), (5, torch.bfloat16)]):
        x = workloads.quantize_tensor(rows=1, cols=n, seed=70 + i).to(dtype)
        for _ in range(2):
            assert fq.fp8_amax(x.to(dev()), ws=ws).item() == oracle.amax(host_input(x.reshape(-1)))


def test_amax_nan_propagates():
    announce("amax nan")
    x = make((64, 512), torch.bfloat16, 11)
    x[17, 300] = float("nan")
    assert np.isnan(fq.fp8_amax(x.to(dev())).item())


# Without a transposed copy, row-major outputs with cols % 8 == 0 take the flat
# streaming kernel; with one (or ragged cols) the 128 x 128 tiled kernel.
@pytest.mark.parametrize("emit_t", [True, False])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", SHAPES + [(7, 1000008)])
def test_per_tensor_current(shape, dtype, fmt, emit_t):
    announce("per-tensor current", shape, dtype, fmt, emit_t)
    x = make(shape, dtype, 20)
    q, qT, s, a = fq.fp8_quantize_per_tensor(x.to(dev()), fmt, emit_t=emit_t)
    oq, os_, oa = oracle.quantize_per_tensor(host_input(x), fmt)
    oq = oq.reshape(shape)
    assert s.item() == os_ and a.item() == oa
    assert codes_equal(q.cpu().numpy(), oq, fmt)
    if emit_t:
        assert codes_equal(qT.cpu().numpy(), oq.T, fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_per_tensor_saturate(fmt):
    announce("per-tensor saturate", fmt)
    # a given-scale cast is reached through delayed scaling with a warm history
    # whose maximum is far below the data: most values overflow
    x = make((200, 384), torch.float32, 21)
    st = fq.DelayedState(dev())
    ost = oracle.DelayedState()
    small = (x * 1e-3).contiguous()
    for sat in (False, True):
        for step in range(2):
            inp = small if step == 0 else x
            q, _, s, a = fq.fp8_quantize_per_tensor(inp.to(dev()), fmt, fq.DELAYED, st, saturate=sat)
            oq, os_, oa = oracle.quantize_delayed(host_input(inp), fmt, ost, saturate=sat)
            assert s.item() == os_ and a.item() == oa
            assert codes_equal(q.cpu().numpy(), oq.reshape(q.shape), fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_per_tensor_full_size(fmt):
    announce("per-tensor full size", fmt)
    x = workloads.quantize_tensor()
    q, qT, s, a = fq.fp8_quantize_per_tensor(x.to(dev()), fmt, emit_t=True)
    oq, os_, oa = oracle.quantize_per_tensor(host_input(x), fmt)
    assert s.item() == os_ and a.item() == oa
    assert codes_equal(q.cpu().numpy(), oq, fmt)
    assert codes_equal(qT.cpu().numpy(), oq.T, fmt)


def test_nan_input_gives_nan_codes():
    announce("per-tensor nan")
    x = make((64, 256), torch.bfloat16, 22)
    x[5, 5] = float("nan")
    q, _, s, a = fq.fp8_quantize_per_tensor(x.to(dev()), fq.E4M3)
    assert np.isnan(a.item()) and np.isnan(s.item())
    assert ((q.cpu().numpy() & 0x7F) == 0x7F).all()


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(512, 1024), (300, 200)])
def test_delayed_sequence_with_spike(shape, fmt):
    """17 delayed-scaling steps (16 warm-up, then a 40-sigma spike) against the
    oracle step by step, including the device-resident history."""
    announce("delayed sequence", shape, fmt)
    st = fq.DelayedState(dev())
    ost = oracle.DelayedState()
    spike_seen = False
    for t, x, spike in workloads.delayed_steps(M=shape[0], K=shape[1], steps=17):
        q, qT, s, a = fq.fp8_quantize_per_tensor(x.to(dev()), fmt, fq.DELAYED, st, emit_t=True)
        oq, os_, oa = oracle.quantize_delayed(host_input(x), fmt, ost)
        assert s.item() == os_ and a.item() == oa, t
        assert codes_equal(q.cpu().numpy(), oq.reshape(shape), fmt), t
        assert codes_equal(qT.cpu().numpy(), oq.reshape(shape).T, fmt), t
        assert np.array_equal(st.history.cpu().numpy(), ost.hist), t
        assert st.pos.item() == ost.pos[0]
        assert st.buf[68:76].view(torch.int32).cpu().tolist() == [0, 0]   # working fields reset
        if spike is not None:
            spike_seen = True
            code = int(q[spike].item())
            if fmt == fq.E4M3:   # the spike overflows the delayed scale: NaN, as in check [3]
                assert (code & 0x7F) == 0x7F
    assert spike_seen


def test_delayed_full_size_spike():
    """Delayed scaling at the single-GEMM activation size: 16 warm-up steps,
    then a 40-sigma spike that overflows (E4M3 NaN) under the delayed scale."""
    announce("delayed full size")
    st = fq.DelayedState(dev())
    ost = oracle.DelayedState()
    for t, x, spike in workloads.delayed_steps():
        xd = x.to(dev())
        q, _, s, a = fq.fp8_quantize_per_tensor(xd, fq.E4M3, fq.DELAYED, st)
        if spike is None:
            ost.hist[ost.pos[0]] = oracle.amax(host_input(x))
            ost.pos[0] = (ost.pos[0] + 1) % 16
            continue
        oq, os_, oa = oracle.quantize_delayed(host_input(x), fq.E4M3, ost)
        assert s.item() == os_ and a.item() == oa
        assert codes_equal(q.cpu().numpy(), oq, fq.E4M3)
        assert (int(q[spike].item()) & 0x7F) == 0x7F
        qc, _, sc, _ = fq.fp8_quantize_per_tensor(xd, fq.E4M3)
        v = oracle.decode(int(qc[spike].item()), fq.E4M3) * sc.item()
        assert abs(v - 0.625) <= 0.625 * 2 ** -4


@pytest.mark.parametrize("emit_t", [True, False])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", [(3, 200), (300, 200), (257, 1030), (1000, 4096), (33, 3968)])
def test_tile1x128(shape, dtype, axis, fmt, emit_t):
    announce("tile1x128", shape, dtype, axis, fmt, emit_t)
    x = make(shape, dtype, 30)
    q, qT, sc = fq.fp8_quantize_tile1x128(x.to(dev()), axis, fmt, emit_t=emit_t)
    oq, osc = oracle.quantize_tiles(host_input(x), axis, 128, fmt)
    assert scales_equal(sc.cpu().numpy(), osc)
    assert codes_equal(q.cpu().numpy(), oq, fmt)
    if emit_t:
        assert codes_equal(qT.cpu().numpy(), oq.T, fmt)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(3, 200), (300, 200), (257, 1030), (1024, 4096)])
def test_block128x128(shape, fmt):
    announce("block128", shape, fmt)
    x = make(shape, torch.bfloat16, 40)
    q, qT, sc = fq.fp8_quantize_block128x128(x.to(dev()), fmt, emit_t=True)
    oq, osc = oracle.quantize_blocks(host_input(x), 128, 128, fmt)
    assert scales_equal(sc.cpu().numpy(), osc)
    assert codes_equal(q.cpu().numpy(), oq, fmt)
    assert codes_equal(qT.cpu().numpy(), oq.T, fmt)


@pytest.mark.parametrize("emit_t", [True, False])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", [(3, 200), (300, 200), (257, 1030), (1000, 4096), (33, 3968)])
def test_mx32(shape, dtype, axis, fmt, emit_t):
    announce("mx32", shape, dtype, axis, fmt, emit_t)
    x = make(shape, dtype, 50)
    q, qT, e8 = fq.fp8_quantize_mx32(x.to(dev()), axis, fmt, emit_t=emit_t)
    oq, oe8 = oracle.quantize_tiles(host_input(x), axis, 32, fmt, mx=True)
    assert np.array_equal(e8.cpu().numpy(), oe8)
    assert codes_equal(q.cpu().numpy(), oq, fmt)
    if emit_t:
        assert codes_equal(qT.cpu().numpy(), oq.T, fmt)


@pytest.mark.parametrize("kind", ["tile", "mx", "block"])
def test_granular_full_size(kind):
    announce("granular full size", kind)
    x = workloads.quantize_tensor()
    xd = x.to(dev())
    if kind == "tile":
        q, _, sc = fq.fp8_quantize_tile1x128(xd, 0, fq.E4M3)
        oq, osc = oracle.quantize_tiles(host_input(x), 0, 128, fq.E4M3)
        assert scales_equal(sc.cpu().numpy(), osc)
    elif kind == "mx":
        q, _, sc = fq.fp8_quantize_mx32(xd, 0, fq.E4M3)
        oq, osc = oracle.quantize_tiles(host_input(x), 0, 32, fq.E4M3, mx=True)
        assert np.array_equal(sc.cpu().numpy(), osc)
    else:
        q, _, sc = fq.fp8_quantize_block128x128(xd, fq.E4M3)
        oq, osc = oracle.quantize_blocks(host_input(x), 128, 128, fq.E4M3)
        assert scales_equal(sc.cpu().numpy(), osc)
    assert codes_equal(q.cpu().numpy(), oq, fq.E4M3)


def test_deterministic_reruns():
    announce("reruns")
    x = make((1000, 4096), torch.bfloat16, 60).to(dev())
    r1 = fq.fp8_quantize_per_tensor(x, fq.E4M3, emit_t=True)
    r2 = fq.fp8_quantize_per_tensor(x, fq.E4M3, emit_t=True)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


def test_per_tensor_beyond_32_bit_offsets():
    """Per-tensor current quantization of a bf16 tensor larger than 2^32 bytes,
    its maximum in the very last element: amax and scale exact, and the codes
    of sampled rows (both ends included) equal to the oracle's cast."""
    rows, cols = 65536, 32784
    assert rows * cols * 2 > 2 ** 32
    announce("per-tensor beyond 32-bit offsets", rows, cols)
    g = torch.Generator(device=dev()).manual_seed(99)
    x = torch.randn((rows, cols), dtype=torch.bfloat16, device=dev(), generator=g)
    x[-1, -1] = 1000.0
    q, _, s, a = fq.fp8_quantize_per_tensor(x, fq.E4M3)
    torch.cuda.synchronize()
    bits = workloads.bf16_bits(x.cpu())
    oa = oracle.amax(bits)
    os_ = oracle.scale_from_amax(oa, fq.E4M3)
    assert a.item() == oa == 1000.0 and s.item() == os_
    sample = np.array([0, 1, rows // 2, rows - 2, rows - 1], np.int64)
    got = q[torch.as_tensor(sample, device=dev())].cpu().numpy()
    want = oracle.cast(bits[sample], os_, fq.E4M3)
    assert codes_equal(got, want, fq.E4M3)
    assert got[-1, -1] == 0x7E   # the maximum encodes to the largest code
