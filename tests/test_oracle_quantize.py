"""Pins of the oracle's amax / scale / cast / delayed / granular quantizers.

The fp8_parity.py page's smoke() checks [1]-[4] are the page's own contract for
these numerics; they are re-run here against the oracle on the page's inputs
(same seed and draw order).  Closed forms (numpy's IEEE fp32 division, numpy
max), reductions to the per-tensor routine, and invariants pin the rest.
"""
import numpy as np
import pytest
import torch

import workloads

E4M3, E5M2 = 0, 1
FMAX = {E4M3: 448.0, E5M2: 57344.0}


def dequant(orc, q, s, fmt):
    """Dequantization as the lab page does it: fp32 product of the code's value and the scale."""
    return (orc.decode_array(q, fmt).astype(np.float32) * np.float32(s)).astype(np.float32)


# ------------------------------------------------------------------ lab smoke checks
def test_lab_check1_roundtrip_bounds(orc):
    """fp8_parity.py smoke check [1]: scaled round-trip relative error on values
    whose scaled magnitude is at least the smallest normal is <= 2^-4 (E4M3) / 2^-3 (E5M2)."""
    x = workloads.lab_smoke_inputs()["x"].numpy()
    for fmt, sn, bound in ((E4M3, 2.0 ** -6, 2.0 ** -4), (E5M2, 2.0 ** -14, 2.0 ** -3)):
        q, s, amax = orc.quantize_per_tensor(x, fmt)
        y = dequant(orc, q, s, fmt)
        normal = np.abs(x / s) >= sn
        rel = (np.abs(y - x) / np.abs(x))[normal].max()
        assert rel <= bound
        # the bound is not vacuous: most values are normal and errors are non-zero
        assert normal.mean() > 0.9 and rel > bound / 4


def test_lab_check2_unscaled_cast_destroys_out_of_range(orc):
    """fp8_parity.py smoke check [2]: a plain (scale 1) E4M3 cast of [1000, -600, 500]
    leaves no element within 50% of its value."""
    big = workloads.lab_smoke_inputs()["big"].numpy()
    plain = orc.decode_array(orc.cast(big, 1.0, E4M3), E4M3)
    with np.errstate(invalid="ignore"):
        rel_err = np.abs(plain - big) / np.abs(big)
        assert not (rel_err < 0.5).any()
    assert np.isnan(plain).all()
    # The saturating variant would NOT pass the check (-600 -> -448 is only 25% off):
    # this is why non-saturating overflow is the default.
    sat = orc.decode_array(orc.cast(big, 1.0, E4M3, saturate=True), E4M3)
    assert ((np.abs(sat - big) / np.abs(big)) < 0.5).any()


def test_lab_check3_delayed_vs_current_on_spike(orc):
    """fp8_parity.py smoke check [3]: with a 16-step history of earlier amaxes, the
    delayed scale overflows a 40.0 spike; the current scale keeps it within 40*2^-4."""
    d = workloads.lab_smoke_inputs()
    st = orc.DelayedState(16)
    for h in d["history"]:
        orc.quantize_delayed(h.numpy(), E4M3, st)
    assert st.pos[0] == 0
    act = d["act"].numpy()
    qd, sd, amax_d = orc.quantize_delayed(act, E4M3, st)
    y_delayed = dequant(orc, qd, sd, E4M3)
    qc, sc, _ = orc.quantize_per_tensor(act, E4M3)
    y_current = dequant(orc, qc, sc, E4M3)
    with np.errstate(invalid="ignore"):
        assert not (abs(y_delayed[3] - 40.0) < 1.0)
    assert abs(y_current[3] - 40.0) <= 40.0 * 2 ** -4
    # delayed scale = max of the 16 earlier amaxes / 448 (numpy fp32 division)
    hist_max = max(np.float32(np.abs(h.numpy()).max()) for h in d["history"])
    assert sd == np.float32(hist_max) / np.float32(448.0)
    # the spike step's amax was recorded at the ring position after 16 steps
    assert st.hist[0] == np.float32(40.0) and amax_d == np.float32(40.0) and st.pos[0] == 1


def test_lab_check4_tiles_beat_tensor_on_outlier_row(orc):
    """fp8_parity.py smoke check [4]: per-tensor vs 1x128 tiles with one outlier row:
    tile scaling has lower MSE on the 7 normal rows."""
    a = workloads.lab_smoke_inputs()["a"].numpy()
    qt, st_, _ = orc.quantize_per_tensor(a, E4M3)
    y_tensor = dequant(orc, qt, st_, E4M3)
    qtile, stile = orc.quantize_tiles(a, 0, 128, E4M3)
    y_tile = np.stack([dequant(orc, qtile[r], stile[r, 0], E4M3) for r in range(8)])
    err_tensor = ((y_tensor - a)[1:] ** 2).mean()
    err_tile = ((y_tile - a)[1:] ** 2).mean()
    assert err_tile < err_tensor


# ------------------------------------------------------------------ closed forms
def test_amax_closed_form_fp32_and_bf16(orc):
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(10007) * 5).astype(np.float32)
    assert orc.amax(x) == np.abs(x).max()
    xb = torch.from_numpy(x).to(torch.bfloat16)
    bits = workloads.bf16_bits(xb)
    assert orc.amax(bits) == np.float32(xb.abs().max().float().item())
    x[77] = np.nan
    assert np.isnan(orc.amax(x))
    assert orc.amax(np.array([-0.0, 0.0], np.float32)) == 0.0
    assert orc.amax(np.array([-7.5, 3.0], np.float32)) == 7.5


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_scale_closed_form(orc, fmt):
    rng = np.random.default_rng(2)
    amaxes = np.abs(rng.standard_normal(1000) * 10.0 ** rng.integers(-8, 8, 1000)).astype(np.float32)
    for a in amaxes:
        ref = np.float32(a) / np.float32(FMAX[fmt])          # IEEE fp32 division
        ref = max(ref, np.float32(1e-12))
        assert orc.scale_from_amax(a, fmt) == ref
    assert orc.scale_from_amax(0.0, fmt) == np.float32(1e-12)
    assert np.isnan(orc.scale_from_amax(np.nan, fmt))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_cast_matches_fp32_division_then_torch_cast(orc, fmt):
    """A cast is encode(RN32(x / s)): numpy's fp32 division then torch's float8 cast."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(50000) * 3).astype(np.float32)
    for s in (np.float32(0.0137), np.float32(1.0) / np.float32(3.0), np.float32(2.5e-3)):
        ref = torch.from_numpy(x / s).to(torch.float8_e4m3fn if fmt == E4M3 else torch.float8_e5m2)
        assert np.array_equal(orc.cast(x, s, fmt), ref.view(torch.uint8).numpy())


# ------------------------------------------------------------------ invariants
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_per_tensor_invariants(orc, fmt):
    x = workloads.quantize_tensor(rows=96, cols=384, seed=11)
    bits = workloads.bf16_bits(x)
    xf = x.float().numpy()
    q, s, amax = orc.quantize_per_tensor(bits, fmt)
    maxcode = 0x7E if fmt == E4M3 else 0x7B
    # (i) the element achieving amax encodes to the largest finite code
    i = np.argmax(np.abs(xf))
    assert (q.reshape(-1)[i] & 0x7F) == maxcode
    assert not np.isnan(orc.decode_array(q, fmt)).any()
    # (ii) negation flips only the sign bit
    qn, sn, _ = orc.quantize_per_tensor(-xf, fmt)
    assert sn == s and np.array_equal(qn, q ^ 0x80)
    # (iii) scaling the input by 2^k leaves codes unchanged and scales s by 2^k
    for k in (-5, 3):
        qk, sk, _ = orc.quantize_per_tensor((xf * np.float32(2.0 ** k)).astype(np.float32), fmt)
        assert np.array_equal(qk, q) and sk == np.float32(s * 2.0 ** k)
    # (v) decode(q(x)) is monotone in x
    order = np.argsort(xf.reshape(-1), kind="stable")
    dq = orc.decode_array(q.reshape(-1)[order], fmt)
    assert (np.diff(dq) >= 0).all()
    # bf16 input widened exactly: same result as the fp32 copy of the same values
    q32, s32, a32 = orc.quantize_per_tensor(xf, fmt)
    assert np.array_equal(q32, q) and s32 == s and a32 == amax


def test_delayed_cold_start_and_steady_state(orc):
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(4096) * 2).astype(np.float32)
    st = orc.DelayedState(16)
    # cold start (empty history) behaves as current scaling
    qd, sd, ad = orc.quantize_delayed(x, E4M3, st)
    qc, sc, ac = orc.quantize_per_tensor(x, E4M3)
    assert np.array_equal(qd, qc) and sd == sc and ad == ac
    # a later step with the same tensor: history max equals its own amax -> same codes
    qd2, sd2, _ = orc.quantize_delayed(x, E4M3, st)
    assert np.array_equal(qd2, qc) and sd2 == sc
    # a smaller tensor afterwards keeps the larger earlier scale
    qd3, sd3, _ = orc.quantize_delayed(x * np.float32(0.25), E4M3, st)
    assert sd3 == sc
    assert np.array_equal(qd3, orc.cast(x * np.float32(0.25), sc, E4M3))
    # after 16 more steps of the small tensor the large amax has left the window
    for _ in range(15):
        orc.quantize_delayed(x * np.float32(0.25), E4M3, st)
    _, sd4, _ = orc.quantize_delayed(x * np.float32(0.25), E4M3, st)
    assert sd4 == orc.scale_from_amax(np.abs(x * np.float32(0.25)).max(), E4M3)
    assert st.pos[0] == 19 % 16


# ------------------------------------------------------------------ granular
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("cols", [384, 300])
def test_tiles_reduce_to_per_tensor_per_tile(orc, fmt, cols):
    x = workloads.quantize_tensor(rows=20, cols=cols, seed=12)
    xf = x.float().numpy()
    bits = workloads.bf16_bits(x)
    q, sc = orc.quantize_tiles(bits, 0, 128, fmt)
    assert sc.shape == (20, -(-cols // 128))
    for r in range(20):
        for t in range(sc.shape[1]):
            seg = xf[r, t * 128:(t + 1) * 128]
            qs, ss, _ = orc.quantize_per_tensor(seg, fmt)
            assert ss == sc[r, t] and np.array_equal(qs, q[r, t * 128:(t + 1) * 128])
    # axis 1 (128 x 1 tiles along rows) is axis 0 of the transpose
    qT, scT = orc.quantize_tiles(np.ascontiguousarray(bits.T), 0, 128, fmt)
    q1, sc1 = orc.quantize_tiles(bits, 1, 128, fmt)
    assert np.array_equal(q1, qT.T) and np.array_equal(sc1, scT)


def test_blocks_reduce_to_per_tensor_per_block(orc):
    x = workloads.quantize_tensor(rows=300, cols=260, seed=13)
    xf = x.float().numpy()
    q, sc = orc.quantize_blocks(workloads.bf16_bits(x), 128, 128, E4M3)
    assert sc.shape == (3, 3)
    for i in range(3):
        for j in range(3):
            blk = np.ascontiguousarray(xf[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128])
            qb, sb, _ = orc.quantize_per_tensor(blk, E4M3)
            assert sb == sc[i, j]
            assert np.array_equal(qb, q[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128])


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_mx32_power_of_two_scales(orc, fmt):
    """MX32 convention (parity unpinned: the pages name MXFP8 but not its rounding):
    e = ceil(log2(amax/fmax)); codes are the cast with s = 2^e.  Checked: the E8M0
    exponent is the smallest power of two not below amax/fmax, no code overflows,
    and codes equal the cast with that power of two."""
    x = workloads.quantize_tensor(rows=16, cols=320, seed=14)
    xf = x.float().numpy()
    q, e8 = orc.quantize_tiles(workloads.bf16_bits(x), 0, 32, fmt, mx=True)
    assert e8.shape == (16, 10) and e8.dtype == np.uint8
    for r in range(16):
        for t in range(10):
            seg = xf[r, t * 32:(t + 1) * 32]
            need = max(np.float32(np.abs(seg).max()) / np.float32(FMAX[fmt]), np.float32(1e-12))
            s = np.float32(2.0 ** (int(e8[r, t]) - 127))
            assert s >= need and s / 2 < need
            assert np.array_equal(q[r, t * 32:(t + 1) * 32], orc.cast(seg, s, fmt))
    assert not np.isnan(orc.decode_array(q, fmt)).any()


def test_tile_roundtrip_bound_per_tile(orc):
    """Check [1]'s bounds hold per 1x128 tile and per MX32 block as well."""
    x = workloads.lab_smoke_inputs()["x"].numpy().reshape(32, 128)
    for fmt, sn, bound in ((E4M3, 2.0 ** -6, 2.0 ** -4), (E5M2, 2.0 ** -14, 2.0 ** -3)):
        q, sc = orc.quantize_tiles(x, 0, 128, fmt)
        y = dequant(orc, q, 1.0, fmt) * sc[:, :1]
        normal = np.abs(x / sc[:, :1]) >= sn
        assert (np.abs(y - x) / np.abs(x))[normal].max() <= bound
        q, e8 = orc.quantize_tiles(x, 0, 32, fmt, mx=True)
        s = (2.0 ** (e8.astype(np.float64) - 127)).repeat(32, axis=1)
        y = orc.decode_array(q, fmt) * s
        normal = np.abs(x / s) >= sn
        assert (np.abs(y - x) / np.abs(x))[normal].max() <= bound


def test_results_do_not_depend_on_thread_count(orc):
    """The oracle is timed on one core and on all of them: its codes, scale
    and amax must be the same either way (order-free maxima)."""
    x = workloads.normal((257, 384), 3.0, 77, torch.bfloat16)
    bits = workloads.bf16_bits(x)
    n = orc.max_threads()
    try:
        orc.set_threads(1)
        q1, s1, a1 = orc.quantize_per_tensor(bits, E4M3)
        orc.set_threads(max(n, 2))
        qn, sn, an = orc.quantize_per_tensor(bits, E4M3)
    finally:
        orc.set_threads(n)
    assert np.array_equal(q1, qn) and s1 == sn and a1 == an
