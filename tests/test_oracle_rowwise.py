"""Pins of the oracle's rowwise scaling (the "fp8_parity.py" lab page,
--recipe rowwise: each GEMM input scaled per row along its contraction)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads
from test_oracle_gemm import brute, frac_decode, random_codes

E4M3, E5M2 = 0, 1
FMAX = {E4M3: 448.0, E5M2: 57344.0}
TORCH_FP8 = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("axis", [0, 1])
def test_rowwise_matches_numpy_division_and_torch_cast(orc, fmt, axis):
    """Each row's (column's) scale is numpy's IEEE fp32 amax / fmax (floored at
    1e-12); each code is torch's float8 cast of numpy's fp32 quotient x / s."""
    rng = np.random.default_rng(11 + fmt + 2 * axis)
    x = (rng.standard_normal((37, 53)) * 10.0 ** rng.integers(-3, 3, (37, 1))).astype(np.float32)
    x[5, :] = 0.0          # an all-zero row: the 1e-12 floor
    x[:, 7] = 0.0          # an all-zero column
    q, s = orc.quantize_rowwise(x, axis, fmt)
    xa = x if axis == 0 else x.T
    amax = np.abs(xa).max(axis=1)
    s_ref = np.maximum(amax / np.float32(FMAX[fmt]), np.float32(1e-12)).astype(np.float32)
    assert s.dtype == np.float32 and s.shape == (xa.shape[0],)
    assert np.array_equal(s, s_ref)
    quot = (xa / s_ref[:, None]).astype(np.float32)
    codes = torch.from_numpy(quot).to(TORCH_FP8[fmt]).view(torch.uint8).numpy()
    assert np.array_equal(q if axis == 0 else q.T, codes)


def test_rowwise_beats_per_tensor_on_outlier_row(orc):
    """Check [4]'s tensor (8 x 128, row 0 x 1e4) with one scale per row: the
    seven normal rows come back more accurately than with one scale for all."""
    a = workloads.lab_smoke_inputs()["a"].numpy()
    q, s = orc.quantize_rowwise(a, 0, E4M3)
    y_row = orc.decode_array(q, E4M3) * s[:, None]
    qt, st, _ = orc.quantize_per_tensor(a, E4M3)
    y_t = orc.decode_array(qt, E4M3) * st
    assert ((y_row - a)[1:] ** 2).mean() < ((y_t - a)[1:] ** 2).mean()


@pytest.mark.parametrize("op", ["NT", "NN", "TN"])
def test_rowwise_gemm_exact(orc, op):
    """C[m,n] = sA[m] sB[n] sum_k a(m,k) b(n,k): exact rational brute force,
    every storage layout, E5M2 x E4M3."""
    rng = np.random.default_rng(21 + len(op))
    M, N, K = 6, 5, 40
    fa, fb = E5M2, E4M3
    shape_a = {"NT": (M, K), "NN": (M, K), "TN": (K, M)}[op]
    shape_b = {"NT": (N, K), "NN": (K, N), "TN": (K, N)}[op]
    A, B = random_codes(rng, shape_a, fa), random_codes(rng, shape_b, fb)
    sa = (rng.random(M) * 1e-2 + 1e-4).astype(np.float32)
    sb = (rng.random(N) * 1e-1 + 1e-3).astype(np.float32)
    a_at = {"NT": lambda m, k: A[m, k], "NN": lambda m, k: A[m, k], "TN": lambda m, k: A[k, m]}[op]
    b_at = {"NT": lambda n, k: B[n, k], "NN": lambda n, k: B[k, n], "TN": lambda n, k: B[k, n]}[op]
    ref = brute(M, N, K, lambda m, k: frac_decode(int(a_at(m, k)), fa), lambda n, k: frac_decode(int(b_at(n, k)), fb),
                lambda m, k: Fraction(float(sa[m])), lambda n, k: Fraction(float(sb[n])), K)
    fn = {"NT": orc.gemm_nt, "NN": orc.gemm_nn, "TN": orc.gemm_tn}[op]
    got = fn(A, B, fa, fb, orc.Scale.rowwise(sa, K), orc.Scale.rowwise(sb, K))
    assert np.allclose(got, ref, rtol=1e-14, atol=0)
