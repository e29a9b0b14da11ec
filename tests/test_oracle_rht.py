"""Pins of the oracle's random Hadamard transform of wgrad operands.

Reference: the explicit block-diagonal matrix (1/4) H16 diag(d) built from
scipy's Hadamard matrix (Sylvester order) and applied in fp64.  The token
signs d come from the Philox stream pinned in test_oracle_sr.py."""
import numpy as np
import pytest
import scipy.linalg

E4M3, E5M2 = 0, 1


def ref_matrix(orc, rows, seed):
    H = scipy.linalg.hadamard(16).astype(np.float64)
    R = np.zeros((rows, rows))
    for b in range(rows // 16):
        d = np.array([orc.rht_sign(seed, 16 * b + i) for i in range(16)], np.float64)
        R[16 * b:16 * b + 16, 16 * b:16 * b + 16] = 0.25 * H * d[None, :]
    return R


def test_signs_are_the_top_bits_of_the_stream(orc):
    for t in (0, 1, 5, 16, 1000, (1 << 33) + 3):
        assert orc.rht_sign(77, t) == (-1 if orc.sr_word(77, 0, t) >> 31 else 1)
    s = np.array([orc.rht_sign(77, t) for t in range(4096)])
    assert abs(s.mean()) < 0.1   # both signs occur about equally often


def test_integer_inputs_match_the_matrix_exactly(orc):
    """With small integer inputs every fp32 step is exact, so the butterflies
    must equal the explicit matrix product bit for bit."""
    rng = np.random.default_rng(1)
    x = rng.integers(-50, 51, (64, 24)).astype(np.float32)
    y = orc.rht(x, 9)
    assert np.array_equal(y.astype(np.float64), ref_matrix(orc, 64, 9) @ x.astype(np.float64))


def test_real_inputs_match_the_matrix_to_fp32_rounding(orc):
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((128, 40)) * 10.0 ** rng.integers(-3, 3, (128, 1))).astype(np.float32)
    y = orc.rht(x, 10).astype(np.float64)
    ref = ref_matrix(orc, 128, 10) @ x.astype(np.float64)
    # four rounded additions of terms no larger than max|x| of the block
    bound = 4 * 2.0 ** -24 * np.abs(x).reshape(8, 16, 40).max(axis=1).repeat(16, axis=0)
    assert np.all(np.abs(y - ref) <= bound + 1e-45)


def test_orthogonal_and_wgrad_product_invariant(orc):
    """R^T R = I (R^T applied in fp64 recovers integer inputs exactly), and the
    wgrad product of two operands transformed with one seed is G^T X."""
    rng = np.random.default_rng(3)
    x = rng.integers(-20, 21, (48, 8)).astype(np.float32)
    R = ref_matrix(orc, 48, 4)
    assert np.array_equal(R.T @ orc.rht(x, 4).astype(np.float64), x.astype(np.float64))
    G = rng.standard_normal((256, 32)).astype(np.float32)
    X = rng.standard_normal((256, 24)).astype(np.float32)
    got = orc.rht(G, 11).astype(np.float64).T @ orc.rht(X, 11).astype(np.float64)
    ref = G.astype(np.float64).T @ X.astype(np.float64)
    assert np.abs(got - ref).max() <= 1e-5 * np.abs(ref).max()


def test_single_value_spreads_over_its_block(orc):
    x = np.zeros((32, 3), np.float32)
    x[21, 1] = 8.0
    y = orc.rht(x, 12)
    assert np.all(np.abs(y[16:32, 1]) == 2.0) and np.all(y[:16] == 0) and np.all(y[:, [0, 2]] == 0)


def test_transform_reduces_wgrad_error_with_an_outlier(orc):
    """A gradient with one outlier entry: per-tensor FP8 quantization of the
    transformed operands gives a more accurate wgrad product than of the raw
    ones (the outlier's amax shrinks by 4x inside its block)."""
    rng = np.random.default_rng(5)
    G = rng.standard_normal((512, 64)).astype(np.float32)
    G[100, 7] = 3000.0
    X = rng.standard_normal((512, 48)).astype(np.float32)
    exact = G.astype(np.float64).T @ X.astype(np.float64)

    def wgrad(Gm, Xm):
        qg, sg, _ = orc.quantize_per_tensor(Gm, E5M2)
        qx, sx, _ = orc.quantize_per_tensor(Xm, E4M3)
        return orc.gemm_tn(qg, qx, E5M2, E4M3, orc.Scale("tensor", sg), orc.Scale("tensor", sx))

    err_plain = np.abs(wgrad(G, X) - exact)
    err_rht = np.abs(wgrad(orc.rht(G, 6), orc.rht(X, 6)) - exact)
    rows = [r for r in range(64) if r != 7]      # the outlier's own output row aside
    assert err_rht[rows].mean() < err_plain[rows].mean()
