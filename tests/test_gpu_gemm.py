"""GPU parity of the scaled FP8 GEMMs (fprop NT, dgrad NN, wgrad TN) against
the exact-integer CPU oracle, to the stated tolerance (fp32 output: 1e-3 of
max|y|; bf16 output: 2^-7 of max|y|), for per-tensor, 1x128 / 128x128 block
and MX32 scaling, pre-quantized and autocast operands, at small shapes with
ragged tiles and at the full layer shapes on sampled rows."""
import zlib

import numpy as np
import pytest
import torch

import fp8_scaled_quantization_amax_amd as fq
import oracle
import workloads
from gpu_util import announce, contract_rows, dev, gemm_close, host_input, sample_rows

pytestmark = pytest.mark.gpu

Q = fq.GemmOperand.quantized
AC = fq.GemmOperand.autocast
GEMM = {"NT": fq.fp8_gemm_scaled_NT, "NN": fq.fp8_gemm_scaled_NN, "TN": fq.fp8_gemm_scaled_TN}
OGEMM = {"NT": oracle.gemm_nt, "NN": oracle.gemm_nn, "TN": oracle.gemm_tn}


def kcontig(op, which):
    """Is operand `which` ('A' or 'B') of op stored with K contiguous?"""
    return {"NT": (True, True), "NN": (True, False), "TN": (False, False)}[op][which == "B"]


def quantize_pt(x, fmt, emit_t):
    """Per-tensor quantization on the GPU and in the oracle (both from the same input)."""
    q, qT, s, _ = fq.fp8_quantize_per_tensor(x.to(dev()), fmt, emit_t=emit_t)
    oq, os_, _ = oracle.quantize_per_tensor(host_input(x), fmt)
    assert s.item() == os_
    return q, qT, s, oq.reshape(x.shape), os_


# ------------------------------------------------------------------ tiny layer
def test_tiny_layer_all_ops_fp32_out():
    """X[512,32], W1[64,32], G[512,64]: fprop E4M3 x E4M3, dgrad E5M2 x E4M3,
    wgrad E5M2^T x E4M3, fp32 accumulate and output; also the W2 fprop."""
    announce("tiny layer")
    X, W1, W2, G = workloads.tiny_layer()
    qx, qxT, sx, oqx, osx = quantize_pt(X, fq.E4M3, True)
    qw, qwT, sw, oqw, osw = quantize_pt(W1, fq.E4M3, True)
    qg, qgT, sg, oqg, osg = quantize_pt(G, fq.E5M2, True)
    S = oracle.Scale
    y = fq.fp8_gemm_scaled_NT(512, 64, 32, Q(qx, fq.E4M3, sx), Q(qw, fq.E4M3, sw), torch.float32)
    ry = oracle.gemm_nt(oqx, oqw, 0, 0, S("tensor", osx), S("tensor", osw))
    assert gemm_close(y, ry, torch.float32)
    for kmaj in (True, False):
        dx = fq.fp8_gemm_scaled_NN(512, 32, 64, Q(qg, fq.E5M2, sg), Q(qw, fq.E4M3, sw, kmajor=qwT if kmaj else None),
                                   torch.float32)
        assert gemm_close(dx, oracle.gemm_nn(oqg, oqw, 1, 0, S("tensor", osg), S("tensor", osw)), torch.float32)
        dw = fq.fp8_gemm_scaled_TN(64, 32, 512, Q(qg, fq.E5M2, sg, kmajor=qgT if kmaj else None),
                                   Q(qx, fq.E4M3, sx, kmajor=qxT if kmaj else None), torch.float32)
        assert gemm_close(dw, oracle.gemm_tn(oqg, oqx, 1, 0, S("tensor", osg), S("tensor", osx)), torch.float32)
    # second layer: relu(y) quantized, times W2 [16, 64]
    H = torch.relu(torch.from_numpy(ry.astype(np.float32)))
    qh, _, sh, oqh, osh = quantize_pt(H, fq.E4M3, False)
    qw2, _, sw2, oqw2, osw2 = quantize_pt(W2, fq.E4M3, False)
    y2 = fq.fp8_gemm_scaled_NT(512, 16, 64, Q(qh, fq.E4M3, sh), Q(qw2, fq.E4M3, sw2), torch.float32)
    assert gemm_close(y2, oracle.gemm_nt(oqh, oqw2, 0, 0, S("tensor", osh), S("tensor", osw2)), torch.float32)


# ------------------------------------------------------------------ per-tensor, ragged shapes
# K % 128 != 0 or K = 128 take the register-staged kernel; K = 256, 384, 1152
# (2, 3 and 9 K steps, ragged M and N) the persistent direct-to-LDS kernel.
SHAPES = [(16, 16, 16), (528, 272, 1040), (256, 256, 128), (1040, 784, 272), (528, 272, 256), (1040, 784, 384),
          (784, 1040, 1152)]
FMT_PAIRS = [(fq.E4M3, fq.E4M3), (fq.E5M2, fq.E4M3), (fq.E5M2, fq.E5M2)]


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("fa,fb", FMT_PAIRS)
@pytest.mark.parametrize("op", ["NT", "NN", "TN"])
@pytest.mark.parametrize("shape", SHAPES)
def test_per_tensor_prequantized(shape, op, fa, fb, out_dtype):
    M, N, K = shape
    announce("gemm per-tensor", op, shape, fa, fb, out_dtype)
    A, B = workloads.gemm_operands(op, M, N, K, seed=100 + M + N + K)
    qa, qaT, sa, oqa, osa = quantize_pt(A, fa, True)
    qb, qbT, sb, oqb, osb = quantize_pt(B, fb, True)
    ref = OGEMM[op](oqa, oqb, fa, fb, oracle.Scale("tensor", osa), oracle.Scale("tensor", osb))
    for use_kmajor in (False, True):
        oa = Q(qa, fa, sa, kmajor=qaT if (use_kmajor and not kcontig(op, "A")) else None)
        ob = Q(qb, fb, sb, kmajor=qbT if (use_kmajor and not kcontig(op, "B")) else None)
        C = GEMM[op](M, N, K, oa, ob, out_dtype)
        assert gemm_close(C, ref, out_dtype), use_kmajor


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", [(4112, 4112, 384), (4368, 4096, 256)])
@pytest.mark.parametrize("op", ["NT", "NN"])
def test_per_tensor_persistent_multi_tile(op, shape, out_dtype):
    """More output tiles than workgroups: some workgroups run two tiles, the
    second starting in the other LDS buffer when the K step count is odd.
    Sampled rows (tile edges included) against the oracle."""
    M, N, K = shape
    announce("gemm per-tensor multi-tile", op, shape, out_dtype)
    A, B = workloads.gemm_operands(op, M, N, K, seed=500 + M + K)
    qa, qaT, sa, oqa, osa = quantize_pt(A, fq.E4M3, False)
    qb, qbT, sb, oqb, osb = quantize_pt(B, fq.E4M3, False)
    rows = sample_rows(M, seed=M + K)
    ref = OGEMM[op](oqa, oqb, 0, 0, oracle.Scale("tensor", osa), oracle.Scale("tensor", osb), rows=rows)
    C = GEMM[op](M, N, K, Q(qa, fq.E4M3, sa), Q(qb, fq.E4M3, sb), out_dtype)
    assert gemm_close(C[torch.as_tensor(rows, device=C.device)], ref, out_dtype)


@pytest.mark.parametrize("op", ["NT", "NN", "TN"])
def test_autocast_current_equals_prequantized(op):
    """Autocast (quantize inside the call) gives bitwise the same C as quantizing
    first and calling the GEMM on the codes."""
    M, N, K = 528, 400, 656
    announce("autocast current", op)
    A, B = workloads.gemm_operands(op, M, N, K, seed=7)
    Ad, Bd = A.to(dev()), B.to(dev())
    sa_out = torch.empty(1, device=dev())
    amax_out = torch.empty(1, device=dev())
    C1 = GEMM[op](M, N, K, AC(Ad, fq.E5M2, scale_out=sa_out, amax_out=amax_out), AC(Bd, fq.E4M3), torch.bfloat16)
    qa, qaT, sa, oqa, osa = quantize_pt(A, fq.E5M2, True)
    qb, qbT, sb, oqb, osb = quantize_pt(B, fq.E4M3, True)
    C2 = GEMM[op](M, N, K, Q(qa, fq.E5M2, sa, kmajor=qaT if not kcontig(op, "A") else None),
                  Q(qb, fq.E4M3, sb, kmajor=qbT if not kcontig(op, "B") else None), torch.bfloat16)
    assert torch.equal(C1, C2)
    assert sa_out.item() == osa and amax_out.item() == oracle.amax(host_input(A))
    ref = OGEMM[op](oqa, oqb, 1, 0, oracle.Scale("tensor", osa), oracle.Scale("tensor", osb))
    assert gemm_close(C1, ref, torch.bfloat16)


def test_autocast_delayed_spike_row_is_nan():
    """Delayed scaling inside the GEMM: after 16 warm-up steps a 40-sigma spike
    in A overflows (E4M3 NaN), so that output row is NaN; current scaling keeps it."""
    M, K, N = 512, 1024, 256
    announce("autocast delayed")
    st = fq.DelayedState(dev())
    ost = oracle.DelayedState()
    _, B = workloads.attn_out_operands(M=M, K=K, N=N)
    qb, _, sb, oqb, osb = quantize_pt(B, fq.E4M3, False)
    for t, x, spike in workloads.delayed_steps(M=M, K=K, steps=17):
        C = fq.fp8_gemm_scaled_NT(M, N, K, AC(x.to(dev()), fq.E4M3, scaling=fq.DELAYED, state=st),
                                  Q(qb, fq.E4M3, sb), torch.bfloat16)
        oqa, osa, _ = oracle.quantize_delayed(host_input(x), fq.E4M3, ost)
        ref = oracle.gemm_nt(oqa.reshape(M, K), oqb, 0, 0, oracle.Scale("tensor", osa), oracle.Scale("tensor", osb))
        assert gemm_close(C, ref, torch.bfloat16), t
        if spike is not None:
            Cn = C.float().cpu().numpy()
            assert np.isnan(Cn[spike[0]]).all() and not np.isnan(np.delete(Cn, spike[0], 0)).any()
            Cc = fq.fp8_gemm_scaled_NT(M, N, K, AC(x.to(dev()), fq.E4M3), Q(qb, fq.E4M3, sb), torch.bfloat16)
            assert not torch.isnan(Cc).any()


# ------------------------------------------------------------------ block-scaled and MX
def block_operands(op, M, N, K, seed):
    """Activation / gradient operand A with 1x128 tiles along K (128x1 for a
    wgrad operand), weight-like operand B with 128x128 blocks (fprop, dgrad) or
    128x1 tiles along K (wgrad)."""
    A, B = workloads.gemm_operands(op, M, N, K, seed=seed, std=1.0, outlier_rows=0.01)
    return A, B


# K = 128 or K % 512 != 0: the register-staged kernel; K % 512 == 0 (8, 4 and
# 12 K steps, ragged M and N): the persistent block-scaled kernel, with one
# scale per wave for 128x128-block B (NT, NN) and per-row B scales (TN).
@pytest.mark.parametrize("op", ["NT", "NN", "TN"])
@pytest.mark.parametrize("shape", [(256, 128, 128), (528, 400, 640), (1024, 1536, 1024), (1040, 784, 512),
                                   (784, 1040, 1536)])
def test_block_scaled(op, shape):
    M, N, K = shape
    announce("gemm block-scaled", op, shape)
    A, B = block_operands(op, M, N, K, seed=200 + M)
    fa, fb = (fq.E5M2, fq.E4M3) if op != "NT" else (fq.E4M3, fq.E4M3)
    axis_a = 0 if kcontig(op, "A") else 1
    qa, qaT, sa = fq.fp8_quantize_tile1x128(A.to(dev()), axis_a, fa, emit_t=not kcontig(op, "A"))
    oqa, osa = oracle.quantize_tiles(host_input(A), axis_a, 128, fa)
    if op == "TN":   # both wgrad operands: 128x1 tiles along the token (contraction) axis
        qb, qbT, sb = fq.fp8_quantize_tile1x128(B.to(dev()), 1, fb, emit_t=True)
        oqb, osb = oracle.quantize_tiles(host_input(B), 1, 128, fb)
        gb, oscale_b = fq.TILE_1x128, oracle.Scale("rowk", osb, kblk=128)
    else:            # weights: 128x128 blocks in their stored layout
        qb, qbT, sb = fq.fp8_quantize_block128x128(B.to(dev()), fb, emit_t=not kcontig(op, "B"))
        oqb, osb = oracle.quantize_blocks(host_input(B), 128, 128, fb)
        gb = fq.BLOCK_128x128
        oscale_b = oracle.Scale("block" if op == "NT" else "blockT", osb, kblk=128, rblk=128)
    ref = OGEMM[op](oqa, oqb, fa, fb, oracle.Scale("rowk", osa, kblk=128), oscale_b)
    for use_kmajor in (False, True):
        oa = Q(qa, fa, sa, fq.TILE_1x128, kmajor=qaT if (use_kmajor and qaT is not None) else None)
        ob = Q(qb, fb, sb, gb, kmajor=qbT if (use_kmajor and qbT is not None) else None)
        C = GEMM[op](M, N, K, oa, ob, torch.float32)
        assert gemm_close(C, ref, torch.float32), use_kmajor
    # autocast with the same granularities gives the same result
    Ca = GEMM[op](M, N, K, AC(A.to(dev()), fa, fq.TILE_1x128), AC(B.to(dev()), fb, gb), torch.float32)
    assert gemm_close(Ca, ref, torch.float32)


def block_scaled_codes(op, A, B, fa, fb):
    """Device codes and oracle codes / scales of a block-scaled GEMM's operands."""
    axis_a = 0 if kcontig(op, "A") else 1
    qa, qaT, sa = fq.fp8_quantize_tile1x128(A.to(dev()), axis_a, fa, emit_t=not kcontig(op, "A"))
    oqa, osa = oracle.quantize_tiles(host_input(A), axis_a, 128, fa)
    if op == "TN":
        qb, qbT, sb = fq.fp8_quantize_tile1x128(B.to(dev()), 1, fb, emit_t=True)
        oqb, osb = oracle.quantize_tiles(host_input(B), 1, 128, fb)
        gb, oscale_b = fq.TILE_1x128, oracle.Scale("rowk", osb, kblk=128)
    else:
        qb, qbT, sb = fq.fp8_quantize_block128x128(B.to(dev()), fb, emit_t=not kcontig(op, "B"))
        oqb, osb = oracle.quantize_blocks(host_input(B), 128, 128, fb)
        gb = fq.BLOCK_128x128
        oscale_b = oracle.Scale("block" if op == "NT" else "blockT", osb, kblk=128, rblk=128)
    oa = Q(qa, fa, sa, fq.TILE_1x128, kmajor=qaT)
    ob = Q(qb, fb, sb, gb, kmajor=qbT)
    return oa, ob, oqa, oqb, oracle.Scale("rowk", osa, kblk=128), oscale_b


@pytest.mark.parametrize("op", ["NT", "NN", "TN"])
def test_block_scaled_persistent_multi_tile(op):
    """Block-scaled with more output tiles than workgroups, an odd number of
    four-step scale groups and bf16 output: sampled rows (tile edges
    included) against the oracle."""
    M, N, K = 4112, 4112, 1536
    announce("gemm block-scaled multi-tile", op)
    A, B = block_operands(op, M, N, K, seed=250)
    fa, fb = (fq.E5M2, fq.E4M3) if op != "NT" else (fq.E4M3, fq.E4M3)
    oa, ob, oqa, oqb, osa, osb = block_scaled_codes(op, A, B, fa, fb)
    rows = sample_rows(M, seed=M + K + 2)
    ref = OGEMM[op](oqa, oqb, fa, fb, osa, osb, rows=rows)
    C = GEMM[op](M, N, K, oa, ob, torch.bfloat16)
    assert gemm_close(C[torch.as_tensor(rows, device=C.device)], ref, torch.bfloat16)


def test_gemm_beyond_32_bit_offsets():
    """A GEMM whose A operand spans more than 2^32 bytes (M * K > 2^32), so
    the persistent kernel's 32-bit buffer offsets do not reach it and the
    register-staged kernel takes it: sampled rows, those that straddle the
    2^32-byte offset included, against the oracle."""
    M, N, K = 262160, 256, 16384
    assert M * K > 2 ** 32
    announce("gemm beyond 32-bit offsets", M, N, K)
    g = torch.Generator(device=dev()).manual_seed(4242)
    # E4M3 codes with magnitude codes 0x00..0x76 (|v| <= 224) and random signs: no NaN code
    A = torch.randint(0, 0x77, (M, K), dtype=torch.uint8, device=dev(), generator=g)
    A |= torch.randint(0, 2, (M, K), dtype=torch.uint8, device=dev(), generator=g) << 7
    B = torch.randint(0, 0x77, (N, K), dtype=torch.uint8, device=dev(), generator=g)
    sa = torch.tensor([2.0 ** -10], dtype=torch.float32, device=dev())
    sb = torch.tensor([2.0 ** -6], dtype=torch.float32, device=dev())
    C = fq.fp8_gemm_scaled_NT(M, N, K, Q(A, fq.E4M3, sa, fq.PER_TENSOR), Q(B, fq.E4M3, sb, fq.PER_TENSOR),
                              torch.bfloat16)
    torch.cuda.synchronize()
    edge = 2 ** 32 // K   # first row whose bytes start at or past 2^32
    rows = np.array(sorted(set(sample_rows(M, seed=7).tolist()) | {edge - 1, edge, edge + 1, M - 16}), np.int64)
    ra = torch.as_tensor(rows, device=dev())
    oa = A[ra].cpu().numpy()
    ob = B.cpu().numpy()
    ref = oracle.gemm_nt(oa, ob, fq.E4M3, fq.E4M3, oracle.Scale("tensor", np.float32(2.0 ** -10)),
                         oracle.Scale("tensor", np.float32(2.0 ** -6)))
    del A
    assert gemm_close(C[ra], ref, torch.bfloat16)


# K = 128 or K % 128 != 0: the register-staged kernel; K >= 256 with K % 128 == 0
# (here 3, 8 and 9 K steps, ragged M and N): the persistent kernel's MX mode.
@pytest.mark.parametrize("op", ["NT", "NN", "TN"])
@pytest.mark.parametrize("shape", [(256, 256, 128), (528, 400, 96), (1024, 1536, 1024), (1040, 784, 384),
                                   (784, 1040, 1152)])
def test_mx32(op, shape):
    M, N, K = shape
    announce("gemm mx32", op, shape)
    A, B = block_operands(op, M, N, K, seed=300 + M)
    fa, fb = (fq.E5M2, fq.E4M3) if op != "NT" else (fq.E4M3, fq.E4M3)
    axa = 0 if kcontig(op, "A") else 1
    axb = 0 if kcontig(op, "B") else 1
    qa, qaT, ea = fq.fp8_quantize_mx32(A.to(dev()), axa, fa, emit_t=axa == 1)
    qb, qbT, eb = fq.fp8_quantize_mx32(B.to(dev()), axb, fb, emit_t=axb == 1)
    oqa, oea = oracle.quantize_tiles(host_input(A), axa, 32, fa, mx=True)
    oqb, oeb = oracle.quantize_tiles(host_input(B), axb, 32, fb, mx=True)
    ref = OGEMM[op](oqa, oqb, fa, fb, oracle.Scale("rowk", oea, kblk=32, e8m0=True),
                    oracle.Scale("rowk", oeb, kblk=32, e8m0=True))
    C = GEMM[op](M, N, K, Q(qa, fa, ea, fq.MX32, kmajor=qaT), Q(qb, fb, eb, fq.MX32, kmajor=qbT), torch.float32)
    assert gemm_close(C, ref, torch.float32)
    Ca = GEMM[op](M, N, K, AC(A.to(dev()), fa, fq.MX32), AC(B.to(dev()), fb, fq.MX32), torch.float32)
    assert gemm_close(Ca, ref, torch.float32)


@pytest.mark.parametrize("op", ["NT", "TN"])
def test_mx32_persistent_multi_tile(op):
    """MX32 with more output tiles than workgroups and an odd K-step count:
    sampled rows (tile edges included) against the oracle."""
    M, N, K = 4112, 4112, 384
    announce("gemm mx32 multi-tile", op)
    A, B = block_operands(op, M, N, K, seed=350)
    fa, fb = (fq.E5M2, fq.E4M3) if op != "NT" else (fq.E4M3, fq.E4M3)
    axa = 0 if kcontig(op, "A") else 1
    axb = 0 if kcontig(op, "B") else 1
    qa, qaT, ea = fq.fp8_quantize_mx32(A.to(dev()), axa, fa, emit_t=axa == 1)
    qb, qbT, eb = fq.fp8_quantize_mx32(B.to(dev()), axb, fb, emit_t=axb == 1)
    oqa, oea = oracle.quantize_tiles(host_input(A), axa, 32, fa, mx=True)
    oqb, oeb = oracle.quantize_tiles(host_input(B), axb, 32, fb, mx=True)
    rows = sample_rows(M, seed=M + K + 1)
    ref = OGEMM[op](oqa, oqb, fa, fb, oracle.Scale("rowk", oea, kblk=32, e8m0=True),
                    oracle.Scale("rowk", oeb, kblk=32, e8m0=True), rows=rows)
    C = GEMM[op](M, N, K, Q(qa, fa, ea, fq.MX32, kmajor=qaT), Q(qb, fb, eb, fq.MX32, kmajor=qbT), torch.bfloat16)
    assert gemm_close(C[torch.as_tensor(rows, device=C.device)], ref, torch.bfloat16)


def test_gemm_reruns_bitwise_identical():
    announce("gemm reruns")
    A, B = workloads.attn_out_operands(M=1024, K=1024, N=512)
    qa, _, sa, _, _ = quantize_pt(A, fq.E4M3, False)
    qb, _, sb, _, _ = quantize_pt(B, fq.E4M3, False)
    C1 = fq.fp8_gemm_scaled_NT(1024, 512, 1024, Q(qa, fq.E4M3, sa), Q(qb, fq.E4M3, sb))
    C2 = fq.fp8_gemm_scaled_NT(1024, 512, 1024, Q(qa, fq.E4M3, sa), Q(qb, fq.E4M3, sb))
    assert torch.equal(C1, C2)


# ------------------------------------------------------------------ full sizes, sampled rows
def test_full_attn_out_prequantized_and_autocast():
    """Attention-output GEMM 15872 x 4096 x 4096, E4M3, bf16 out (the launch
    configuration the benchmark times), on sampled rows."""
    M, K, N = workloads.M_TOKENS, workloads.HIDDEN, workloads.HIDDEN
    announce("full attn-out")
    A, B = workloads.attn_out_operands()
    qa, _, sa, oqa, osa = quantize_pt(A, fq.E4M3, False)
    qb, _, sb, oqb, osb = quantize_pt(B, fq.E4M3, False)
    rows = sample_rows(M, 1)
    ref = oracle.gemm_nt(oqa, oqb, 0, 0, oracle.Scale("tensor", osa), oracle.Scale("tensor", osb), rows=rows)
    C = fq.fp8_gemm_scaled_NT(M, N, K, Q(qa, fq.E4M3, sa), Q(qb, fq.E4M3, sb))
    assert gemm_close(C[torch.from_numpy(rows).to(dev())], ref, torch.bfloat16)
    Ca = fq.fp8_gemm_scaled_NT(M, N, K, AC(A.to(dev()), fq.E4M3), AC(B.to(dev()), fq.E4M3))
    assert torch.equal(C, Ca)


def nt_form(op, oqa, oqb, osa, osb):
    """The oracle's operands of op in the NT form: codes K-contiguous ([M, K],
    [N, K]) and the scales indexed the same way (a weight's 128x128 block
    scales, stored [K/128, N/128] for dgrad, transposed with it).  The layouts
    agree exactly (the oracle's NT = NN = TN pin)."""
    if not kcontig(op, "A"):
        oqa = np.ascontiguousarray(oqa.T)
    if not kcontig(op, "B"):
        oqb = np.ascontiguousarray(oqb.T)
    if osb.kind == "blockT":
        osb = oracle.Scale("block", np.ascontiguousarray(osb.arr.T), kblk=osb.kblk, rblk=osb.rblk)
    return oqa, oqb, osa, osb


@pytest.mark.parametrize("gemm", workloads.layer_gemms(), ids=lambda g: g[0])
def test_full_layer_gemm_sampled(gemm):
    """Each of the 12 layer GEMMs at full size (operands ~ N(0,1)/sqrt(K)),
    per-tensor current scaling, fprop E4M3 x E4M3, dgrad and wgrad E5M2 x E4M3,
    autocast, bf16 out -- the benchmark's launch configuration -- on the first
    and last row of every 128-row M tile and 256 random rows, all N columns.
    The same GEMM on pre-quantized codes gives bitwise the same output."""
    name, op, M, N, K = gemm
    announce("full layer", name, op, M, N, K)
    A, B = workloads.gemm_operands(op, M, N, K, seed=4000 + zlib.crc32(name.encode()) % 1000, device=dev())
    fa = fq.E4M3 if op == "NT" else fq.E5M2
    C = GEMM[op](M, N, K, AC(A, fa), AC(B, fq.E4M3))
    qa, qaT, sa, _ = fq.fp8_quantize_per_tensor(A, fa, emit_t=not kcontig(op, "A"))
    qb, qbT, sb, _ = fq.fp8_quantize_per_tensor(B, fq.E4M3, emit_t=not kcontig(op, "B"))
    Cp = GEMM[op](M, N, K, Q(qa, fa, sa, kmajor=qaT), Q(qb, fq.E4M3, sb, kmajor=qbT))
    assert torch.equal(C, Cp)
    del Cp, qa, qaT, qb, qbT
    oqa, osa, _ = oracle.quantize_per_tensor(host_input(A), fa)
    oqb, osb, _ = oracle.quantize_per_tensor(host_input(B), fq.E4M3)
    assert sa.item() == osa and sb.item() == osb
    oqa, oqb, sa_o, sb_o = nt_form(op, oqa.reshape(A.shape), oqb.reshape(B.shape), oracle.Scale("tensor", osa),
                                   oracle.Scale("tensor", osb))
    rows = contract_rows(M, 2)
    ref = oracle.gemm_nt(oqa, oqb, fa, fq.E4M3, sa_o, sb_o, rows=rows)
    assert gemm_close(C[torch.from_numpy(rows).to(dev())], ref, torch.bfloat16)


def mx_codes(op, A, B, fa, fb):
    """Device codes and oracle codes / exponents of an MX32 GEMM's operands."""
    axa = 0 if kcontig(op, "A") else 1
    axb = 0 if kcontig(op, "B") else 1
    qa, qaT, ea = fq.fp8_quantize_mx32(A.to(dev()), axa, fa, emit_t=axa == 1)
    qb, qbT, eb = fq.fp8_quantize_mx32(B.to(dev()), axb, fb, emit_t=axb == 1)
    oqa, oea = oracle.quantize_tiles(host_input(A), axa, 32, fa, mx=True)
    oqb, oeb = oracle.quantize_tiles(host_input(B), axb, 32, fb, mx=True)
    return (Q(qa, fa, ea, fq.MX32, kmajor=qaT), Q(qb, fb, eb, fq.MX32, kmajor=qbT), oqa, oqb,
            oracle.Scale("rowk", oea, kblk=32, e8m0=True), oracle.Scale("rowk", oeb, kblk=32, e8m0=True))


@pytest.mark.parametrize("recipe", ["block", "mx"])
@pytest.mark.parametrize("gemm", workloads.layer_gemms(), ids=lambda g: g[0])
def test_full_layer_granular_sampled(gemm, recipe):
    """All 12 layer GEMMs at full size in the benchmark's block-scaled recipe
    (activations / gradients 1x128 along K, weights 128x128, both wgrad
    operands 128x1 along tokens) and its MX32 recipe (E8M0 per 32 along K),
    on N(0,1) operands with 1% of rows x1e3; fprop E4M3 x E4M3, dgrad / wgrad
    E5M2 x E4M3; bf16 out.  Checked on the first and last row of every
    128-row M tile and 256 random rows, all N columns."""
    name, op, M, N, K = gemm
    announce("full granular", recipe, name, op, M, N, K)
    A, B = workloads.gemm_operands(op, M, N, K, seed=7000 + zlib.crc32(name.encode()) % 1000, std=1.0,
                                   outlier_rows=0.01, device=dev())
    fa, fb = (fq.E4M3, fq.E4M3) if op == "NT" else (fq.E5M2, fq.E4M3)
    codes = block_scaled_codes if recipe == "block" else mx_codes
    oa, ob, oqa, oqb, osa, osb = codes(op, A, B, fa, fb)
    C = GEMM[op](M, N, K, oa, ob, torch.bfloat16)
    del oa, ob, A, B
    oqa, oqb, osa, osb = nt_form(op, oqa, oqb, osa, osb)
    rows = contract_rows(M, 3)
    ref = oracle.gemm_nt(oqa, oqb, fa, fb, osa, osb, rows=rows)
    assert gemm_close(C[torch.as_tensor(rows, device=C.device)], ref, torch.bfloat16)


def test_full_attn_out_delayed_autocast_spike():
    """The attention-output GEMM at full size (A [15872, 4096] activations,
    B [4096, 4096] weight, ~ N(0,1)/64) with delayed scaling of A inside the
    call: 16 warm-up steps fill the 16-entry history, and the 17th step's
    activation carries one 40-sigma element.  Its scale comes from the
    history, so that element overflows E4M3 (NaN): the spike's output row is
    NaN and no other row is; the history, scales and the sampled rows of the
    cold-start and spike steps match the oracle."""
    M, K, N = workloads.M_TOKENS, workloads.HIDDEN, workloads.HIDDEN
    announce("full delayed autocast", M, N, K)
    st = fq.DelayedState(dev())
    ost = oracle.DelayedState()
    _, B = workloads.attn_out_operands()
    qb, _, sb, oqb, osb = quantize_pt(B, fq.E4M3, False)
    ws = torch.zeros(fq.gemm_workspace_bytes("NT", M, N, K, AC(B.to(dev()), fq.E4M3, scaling=fq.DELAYED, state=st),
                                             Q(qb, fq.E4M3, sb)), dtype=torch.uint8, device=dev())
    rows = contract_rows(M, 5)
    for t, x, spike in workloads.delayed_steps(M=M, K=K, steps=17):
        xd = x.to(dev())
        C = fq.fp8_gemm_scaled_NT(M, N, K, AC(xd, fq.E4M3, scaling=fq.DELAYED, state=st), Q(qb, fq.E4M3, sb),
                                  torch.bfloat16, ws=ws)
        oqa, osa, _ = oracle.quantize_delayed(host_input(x), fq.E4M3, ost)
        assert st.last_scale.item() == osa, t
        assert np.array_equal(st.history.cpu().numpy(), ost.hist) and st.pos.item() == ost.pos[0], t
        if t in (0, 16):
            r = rows if spike is None else np.union1d(rows, [spike[0]])
            ref = oracle.gemm_nt(oqa.reshape(M, K), oqb, 0, 0, oracle.Scale("tensor", osa),
                                 oracle.Scale("tensor", osb), rows=r)
            assert gemm_close(C[torch.from_numpy(r).to(dev())], ref, torch.bfloat16), t
        if spike is not None:
            nan_rows = torch.isnan(C.float()).any(dim=1).nonzero().flatten().cpu().tolist()
            assert nan_rows == [spike[0]]
            assert torch.isnan(C[spike[0]].float()).all()


def test_workspace_reused_across_shapes_delayed():
    """One zero-filled workspace serves GEMMs of two different plans in turn
    for five steps: a dgrad with a delayed-autocast A and a pre-quantized B
    that is transposed into the workspace, and an fprop of another shape with
    delayed autocast on both operands.  The outputs equal calls with fresh
    workspaces bitwise, and every delayed state walks the oracle's history."""
    announce("workspace reuse across plans")
    dgrad = ("NN", 1040, 784, 384)
    fprop = ("NT", 528, 400, 656)
    Ag, Bw = workloads.gemm_operands(*dgrad, seed=8800)
    Ax, Bx = workloads.gemm_operands(*fprop, seed=8810)
    qw, _, sw, _ = fq.fp8_quantize_per_tensor(Bw.to(dev()), fq.E4M3)
    states = {k: (fq.DelayedState(dev()), fq.DelayedState(dev()), oracle.DelayedState()) for k in ("g", "x", "w")}

    def operands(step, which):   # which = 0: shared workspace's states, 1: the fresh ones'
        g = (Ag.float() * (1.0 + 0.25 * step)).to(torch.bfloat16)
        x = (Ax.float() * (1.0 - 0.125 * step)).to(torch.bfloat16)
        dl = lambda t, fmt, k: AC(t.to(dev()), fmt, scaling=fq.DELAYED, state=states[k][which])
        return (g, x), ((dl(g, fq.E5M2, "g"), Q(qw, fq.E4M3, sw)), (dl(x, fq.E4M3, "x"), dl(Bx, fq.E4M3, "w")))

    _, ((a0, b0), (a1, b1)) = operands(0, 0)
    need = max(fq.gemm_workspace_bytes(*dgrad, a0, b0), fq.gemm_workspace_bytes(*fprop, a1, b1))
    shared = torch.zeros(need, dtype=torch.uint8, device=dev())
    for step in range(5):
        (g, x), shared_ops = operands(step, 0)
        _, fresh_ops = operands(step, 1)
        for (op, M, N, K), (oa, ob), (fa2, fb2) in zip((dgrad, fprop), shared_ops, fresh_ops):
            C1 = GEMM[op](M, N, K, oa, ob, torch.float32, ws=shared)
            C2 = GEMM[op](M, N, K, fa2, fb2, torch.float32)
            assert torch.equal(C1, C2), (step, op)
        for k, t, fmt in (("g", g, fq.E5M2), ("x", x, fq.E4M3), ("w", Bx, fq.E4M3)):
            oracle.quantize_delayed(host_input(t), fmt, states[k][2])
            assert np.array_equal(states[k][0].history.cpu().numpy(), states[k][2].hist), (step, k)
            assert states[k][0].pos.item() == states[k][2].pos[0]


def test_mx_misaligned_scales():
    """MX32 scales at an address that is not 16-byte aligned take the general
    kernel (the persistent one loads them 16 bytes at a time): same result
    as with aligned scales, within tolerance of the oracle."""
    op, M, N, K = "NT", 528, 400, 1024
    announce("mx misaligned scales")
    A, B = block_operands(op, M, N, K, seed=777)
    oa, ob, oqa, oqb, osa, osb = mx_codes(op, A, B, fq.E4M3, fq.E4M3)
    ea, eb = oa.keep[2], ob.keep[2]
    bufa = torch.empty(ea.numel() + 16, dtype=torch.uint8, device=dev())
    bufb = torch.empty(eb.numel() + 16, dtype=torch.uint8, device=dev())
    ea1 = bufa[1:1 + ea.numel()].view(ea.shape)
    eb1 = bufb[3:3 + eb.numel()].view(eb.shape)
    ea1.copy_(ea)
    eb1.copy_(eb)
    assert ea1.data_ptr() % 16 != 0 and eb1.data_ptr() % 16 != 0
    ref = oracle.gemm_nt(oqa, oqb, 0, 0, osa, osb)
    C = GEMM[op](M, N, K, oa, ob, torch.float32)
    C1 = GEMM[op](M, N, K, Q(oa.keep[0], fq.E4M3, ea1, fq.MX32), Q(ob.keep[0], fq.E4M3, eb1, fq.MX32), torch.float32)
    assert gemm_close(C, ref, torch.float32) and gemm_close(C1, ref, torch.float32)
