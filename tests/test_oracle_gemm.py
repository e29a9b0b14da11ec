"""Pins of the oracle's scaled GEMM.

- Exact rational brute force (Python fractions) on tiny shapes for every
  storage layout (fprop NT, dgrad NN, wgrad TN) and every scale granularity.
- The three layouts agree exactly on transposed copies of the same data.
- Agreement with the fp8_parity.py page's FP8Matmul form (dequantize, then an
  fp64 matmul) on the tiny layer.
- IEEE propagation of NaN / Inf codes.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads

E4M3, E5M2 = 0, 1


def frac_decode(code, fmt):
    """Exact value of a finite code as a Fraction (from the format definition)."""
    mb, bias = (3, 7) if fmt == E4M3 else (2, 15)
    sign = -1 if code & 0x80 else 1
    e = (code >> mb) & ((1 << (7 - mb)) - 1)
    m = code & ((1 << mb) - 1)
    if e == 0:
        v = Fraction(m, 1 << mb) * Fraction(2) ** (1 - bias)
    else:
        v = (1 + Fraction(m, 1 << mb)) * Fraction(2) ** (e - bias)
    return sign * v


def random_codes(rng, shape, fmt):
    """Random finite codes (avoid NaN / Inf patterns)."""
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    if fmt == E4M3:
        bad = (c & 0x7F) == 0x7F
        c[bad] = 0x3A
    else:
        bad = (c & 0x7F) >= 0x7C
        c[bad] = 0x3D
    return c


def brute(M, N, K, a_at, b_at, sa_at, sb_at, kblk):
    """y[m][n] = sum_kb sA(m,kb) sB(n,kb) sum_{k in kb} a(m,k) b(n,k), exactly."""
    out = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for k0 in range(0, K, kblk):
                part = sum((a_at(m, k) * b_at(n, k) for k in range(k0, min(K, k0 + kblk))), Fraction(0))
                tot += part * sa_at(m, k0) * sb_at(n, k0)
            out[m, n] = float(tot)
    return out


@pytest.mark.parametrize("op", ["NT", "NN", "TN"])
@pytest.mark.parametrize("fa,fb", [(E4M3, E4M3), (E5M2, E4M3), (E5M2, E5M2)])
def test_per_tensor_exact(orc, op, fa, fb):
    rng = np.random.default_rng(100 + 7 * fa + 3 * fb + len(op))
    M, N, K = 5, 7, 48
    sa, sb = np.float32(0.0173), np.float32(3.7e-3)
    shape_a = {"NT": (M, K), "NN": (M, K), "TN": (K, M)}[op]
    shape_b = {"NT": (N, K), "NN": (K, N), "TN": (K, N)}[op]
    A, B = random_codes(rng, shape_a, fa), random_codes(rng, shape_b, fb)
    a_at = {"NT": lambda m, k: A[m, k], "NN": lambda m, k: A[m, k], "TN": lambda m, k: A[k, m]}[op]
    b_at = {"NT": lambda n, k: B[n, k], "NN": lambda n, k: B[k, n], "TN": lambda n, k: B[k, n]}[op]
    ref = brute(M, N, K, lambda m, k: frac_decode(int(a_at(m, k)), fa),
                lambda n, k: frac_decode(int(b_at(n, k)), fb),
                lambda m, k: Fraction(float(sa)), lambda n, k: Fraction(float(sb)), K)
    fn = {"NT": orc.gemm_nt, "NN": orc.gemm_nn, "TN": orc.gemm_tn}[op]
    got = fn(A, B, fa, fb, orc.Scale("tensor", sa), orc.Scale("tensor", sb))
    assert np.allclose(got, ref, rtol=1e-14, atol=0)


def test_rowk_tile_scales_exact(orc):
    """1 x 128 scales for A rows and B rows (per K-block), E4M3 x E5M2, ragged K."""
    rng = np.random.default_rng(5)
    M, N, K, T = 4, 3, 300, 128
    nk = -(-K // T)
    A, B = random_codes(rng, (M, K), E4M3), random_codes(rng, (N, K), E5M2)
    SA = (rng.random((M, nk)) + 0.1).astype(np.float32)
    SB = (rng.random((N, nk)) + 0.1).astype(np.float32)
    ref = brute(M, N, K, lambda m, k: frac_decode(int(A[m, k]), E4M3),
                lambda n, k: frac_decode(int(B[n, k]), E5M2),
                lambda m, k: Fraction(float(SA[m, k // T])), lambda n, k: Fraction(float(SB[n, k // T])), T)
    got = orc.gemm_nt(A, B, E4M3, E5M2, orc.Scale("rowk", SA, kblk=T), orc.Scale("rowk", SB, kblk=T))
    assert np.allclose(got, ref, rtol=1e-14, atol=0)


def test_block_scales_fprop_and_dgrad_exact(orc):
    """128 x 128 weight blocks: fprop (weight rows = N) and dgrad (weight rows = K)."""
    rng = np.random.default_rng(6)
    T = 128
    # fprop: A [M,K] 1x128, W [N,K] 128x128
    M, N, K = 3, 260, 256
    A, W = random_codes(rng, (M, K), E4M3), random_codes(rng, (N, K), E4M3)
    SA = (rng.random((M, K // T)) + 0.5).astype(np.float32)
    SW = (rng.random((-(-N // T), K // T)) + 0.5).astype(np.float32)
    ref = brute(M, 5, K, lambda m, k: frac_decode(int(A[m, k]), E4M3),
                lambda n, k: frac_decode(int(W[n * 64, k]), E4M3),
                lambda m, k: Fraction(float(SA[m, k // T])),
                lambda n, k: Fraction(float(SW[(n * 64) // T, k // T])), T)
    got = orc.gemm_nt(A, W, E4M3, E4M3, orc.Scale("rowk", SA, kblk=T),
                      orc.Scale("block", SW, kblk=T, rblk=T))
    assert np.allclose(got[:, ::64], ref, rtol=1e-14, atol=0)
    # dgrad: G [M, Nout] 1x128 E5M2, W [Nout, Kin] 128x128; y = G @ W, contraction over Nout
    Nout, Kin = 256, 260
    G, W = random_codes(rng, (M, Nout), E5M2), random_codes(rng, (Nout, Kin), E4M3)
    SG = (rng.random((M, Nout // T)) + 0.5).astype(np.float32)
    SW = (rng.random((Nout // T, -(-Kin // T))) + 0.5).astype(np.float32)
    cols = [0, 100, 127, 128, 259]
    ref = brute(M, len(cols), Nout, lambda m, k: frac_decode(int(G[m, k]), E5M2),
                lambda j, k: frac_decode(int(W[k, cols[j]]), E4M3),
                lambda m, k: Fraction(float(SG[m, k // T])),
                lambda j, k: Fraction(float(SW[k // T, cols[j] // T])), T)
    got = orc.gemm_nn(G, W, E5M2, E4M3, orc.Scale("rowk", SG, kblk=T),
                      orc.Scale("blockT", SW, kblk=T, rblk=T))
    assert np.allclose(got[:, cols], ref, rtol=1e-14, atol=0)


def test_mx_e8m0_scales_exact(orc):
    rng = np.random.default_rng(7)
    M, N, K, T = 3, 4, 96, 32
    A, B = random_codes(rng, (M, K), E4M3), random_codes(rng, (N, K), E4M3)
    EA = rng.integers(110, 140, (M, K // T)).astype(np.uint8)
    EB = rng.integers(110, 140, (N, K // T)).astype(np.uint8)
    ref = brute(M, N, K, lambda m, k: frac_decode(int(A[m, k]), E4M3),
                lambda n, k: frac_decode(int(B[n, k]), E4M3),
                lambda m, k: Fraction(2) ** (int(EA[m, k // T]) - 127),
                lambda n, k: Fraction(2) ** (int(EB[n, k // T]) - 127), T)
    got = orc.gemm_nt(A, B, E4M3, E4M3, orc.Scale("rowk", EA, kblk=T, e8m0=True),
                      orc.Scale("rowk", EB, kblk=T, e8m0=True))
    assert np.allclose(got, ref, rtol=1e-14, atol=0)


def test_layouts_agree_and_row_sampling(orc):
    rng = np.random.default_rng(8)
    M, N, K = 40, 24, 160
    A, B = random_codes(rng, (M, K), E5M2), random_codes(rng, (N, K), E4M3)
    sa, sb = orc.Scale("tensor", 0.02), orc.Scale("tensor", 0.5)
    nt = orc.gemm_nt(A, B, E5M2, E4M3, sa, sb)
    nn = orc.gemm_nn(A, np.ascontiguousarray(B.T), E5M2, E4M3, sa, sb)
    tn = orc.gemm_tn(np.ascontiguousarray(A.T), np.ascontiguousarray(B.T), E5M2, E4M3, sa, sb)
    assert np.array_equal(nt, nn) and np.array_equal(nt, tn)
    rows = np.array([39, 0, 17])
    assert np.array_equal(orc.gemm_nt(A, B, E5M2, E4M3, sa, sb, rows=rows), nt[rows])


def test_tiny_layer_matches_fake_quant_matmul(orc):
    """fp8_parity.py FP8Matmul computes its forward and backward products on
    dequantized fp32 values.  The oracle's exact-integer GEMM agrees with an fp64
    matmul of the dequantized codes to fp64 rounding."""
    X, W1, _, G = workloads.tiny_layer()
    x, w, g = X.numpy(), W1.numpy(), G.numpy()
    qx, sx, _ = orc.quantize_per_tensor(x, E4M3)
    qw, sw, _ = orc.quantize_per_tensor(w, E4M3)
    qg, sg, _ = orc.quantize_per_tensor(g, E5M2)
    xq = orc.decode_array(qx, E4M3) * float(sx)
    wq = orc.decode_array(qw, E4M3) * float(sw)
    gq = orc.decode_array(qg, E5M2) * float(sg)
    S = lambda s: orc.Scale("tensor", s)
    y = orc.gemm_nt(qx, qw, E4M3, E4M3, S(sx), S(sw))
    assert np.allclose(y, xq @ wq.T, rtol=1e-12, atol=1e-12)
    dx = orc.gemm_nn(qg, qw, E5M2, E4M3, S(sg), S(sw))
    assert np.allclose(dx, gq @ wq, rtol=1e-12, atol=1e-12)
    dw = orc.gemm_tn(qg, qx, E5M2, E4M3, S(sg), S(sx))
    assert np.allclose(dw, gq.T @ xq, rtol=1e-12, atol=1e-12)
    # and to the unquantized fp32 product within FP8 rounding (sanity)
    assert np.abs(y - x @ w.T).max() <= 0.1 * np.abs(x @ w.T).max()


def test_non_finite_codes_propagate(orc):
    A = np.full((2, 32), 0x38, np.uint8)
    B = np.full((3, 32), 0x38, np.uint8)
    A[0, 5] = 0x7F                       # E4M3 NaN in row 0
    y = orc.gemm_nt(A, B, E4M3, E4M3, orc.Scale("tensor", 1.0), orc.Scale("tensor", 1.0))
    assert np.isnan(y[0]).all() and (y[1] == 32.0).all()
    A5 = np.full((2, 32), 0x3C, np.uint8)
    A5[1, 0] = 0x7C                      # E5M2 +Inf in row 1
    y = orc.gemm_nt(A5, B, E5M2, E4M3, orc.Scale("tensor", 1.0), orc.Scale("tensor", 1.0))
    assert (y[0] == 32.0).all() and (y[1] == np.inf).all()
    B[2, 0] = 0x00                       # Inf * 0 -> NaN in column 2
    y = orc.gemm_nt(A5, B, E5M2, E4M3, orc.Scale("tensor", 1.0), orc.Scale("tensor", 1.0))
    assert np.isnan(y[1, 2]) and y[1, 0] == np.inf
