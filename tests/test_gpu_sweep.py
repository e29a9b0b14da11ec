"""A seeded sweep of GEMM configurations against the oracle: for each case a
random op (NT / NN / TN), format pair, output type, scaling granularity
(per-tensor, 1x128 with 128x128 weight blocks, MX32), shape (multiples of 16
up to 768 x 768, K up to 1536 within what the granularity allows) and
operand mode (pre-quantized, with or without the K-major copies, or autocast),
so that the kernel choices (persistent or register-staged, odd and even K-step
counts, ragged edges) meet combinations the fixed-shape tests do not list.
Every output row is compared, to the stated tolerance."""
import random

import pytest
import torch

import fp8_scaled_quantization_amax_amd as fq
import oracle
from gpu_util import announce, dev, gemm_close, host_input
from test_gpu_gemm import AC, GEMM, OGEMM, Q, block_operands, kcontig, quantize_pt
import workloads

pytestmark = pytest.mark.gpu

PAIRS = [(fq.E4M3, fq.E4M3), (fq.E5M2, fq.E4M3), (fq.E4M3, fq.E5M2), (fq.E5M2, fq.E5M2)]


def case(i):
    r = random.Random(7000 + i)
    gran = ["tensor", "block", "mx"][i % 3]
    op = r.choice(["NT", "NN", "TN"])
    fa, fb = r.choice(PAIRS)
    out = r.choice([torch.float32, torch.bfloat16])
    M, N = 16 * r.randint(1, 48), 16 * r.randint(1, 48)
    # about half of each granularity's K values take its persistent kernel
    # (per-tensor: K % 128 == 0 and K >= 256; block-scaled and MX: K % 512 == 0)
    if gran == "tensor":
        K = r.choice([16 * r.randint(1, 96), 128 * r.randint(2, 12)])
    elif gran == "block":
        K = 128 * r.choice([1, 2, 3, 4, 4, 8, 12])
    else:
        K = r.choice([32 * r.randint(1, 48), 512 * r.randint(1, 3)])
    mode = r.choice(["quantized", "kmajor", "autocast"])
    return gran, op, fa, fb, out, M, N, K, mode


@pytest.mark.parametrize("i", range(96))
def test_gemm_sweep(i):
    gran, op, fa, fb, out, M, N, K, mode = case(i)
    announce("gemm sweep", i, gran, op, fa, fb, out, (M, N, K), mode)
    if gran == "tensor":
        A, B = workloads.gemm_operands(op, M, N, K, seed=7100 + i)
        qa, qaT, sa, oqa, osa = quantize_pt(A, fa, True)
        qb, qbT, sb, oqb, osb = quantize_pt(B, fb, True)
        ref = OGEMM[op](oqa, oqb, fa, fb, oracle.Scale("tensor", osa), oracle.Scale("tensor", osb))
        if mode == "autocast":
            C = GEMM[op](M, N, K, AC(A.to(dev()), fa), AC(B.to(dev()), fb), out)
        else:
            km = mode == "kmajor"
            C = GEMM[op](M, N, K, Q(qa, fa, sa, kmajor=qaT if km and not kcontig(op, "A") else None),
                         Q(qb, fb, sb, kmajor=qbT if km and not kcontig(op, "B") else None), out)
    elif gran == "block":
        A, B = block_operands(op, M, N, K, seed=7200 + i)
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
        ref = OGEMM[op](oqa, oqb, fa, fb, oracle.Scale("rowk", osa, kblk=128), oscale_b)
        if mode == "autocast":
            C = GEMM[op](M, N, K, AC(A.to(dev()), fa, fq.TILE_1x128), AC(B.to(dev()), fb, gb), out)
        else:
            km = mode == "kmajor"
            C = GEMM[op](M, N, K, Q(qa, fa, sa, fq.TILE_1x128, kmajor=qaT if km and qaT is not None else None),
                         Q(qb, fb, sb, gb, kmajor=qbT if km and qbT is not None else None), out)
    else:
        A, B = block_operands(op, M, N, K, seed=7300 + i)
        axa = 0 if kcontig(op, "A") else 1
        axb = 0 if kcontig(op, "B") else 1
        qa, qaT, ea = fq.fp8_quantize_mx32(A.to(dev()), axa, fa, emit_t=axa == 1)
        qb, qbT, eb = fq.fp8_quantize_mx32(B.to(dev()), axb, fb, emit_t=axb == 1)
        oqa, oea = oracle.quantize_tiles(host_input(A), axa, 32, fa, mx=True)
        oqb, oeb = oracle.quantize_tiles(host_input(B), axb, 32, fb, mx=True)
        ref = OGEMM[op](oqa, oqb, fa, fb, oracle.Scale("rowk", oea, kblk=32, e8m0=True),
                        oracle.Scale("rowk", oeb, kblk=32, e8m0=True))
        if mode == "autocast":
            C = GEMM[op](M, N, K, AC(A.to(dev()), fa, fq.MX32), AC(B.to(dev()), fb, fq.MX32), out)
        else:
            C = GEMM[op](M, N, K, Q(qa, fa, ea, fq.MX32, kmajor=qaT), Q(qb, fb, eb, fq.MX32, kmajor=qbT), out)
    assert gemm_close(C, ref, out)
