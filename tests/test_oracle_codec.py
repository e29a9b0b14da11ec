"""Pins of the oracle's 8-bit float codec (decode / encode) to facts fixed outside it.

- The pages print the format maxima and smallest normals (fp8_parity.py page:
  E4M3_MAX / E5M2_MAX constants and smoke check [1]).
- Every code's value is cross-checked against torch's float8 dtypes (the very
  routine the lab page's numerics run on), and encode against torch's
  float8 cast on every fp32 bit pattern.
- An independent brute-force nearest-value search (numpy) pins round-to-nearest,
  ties-to-even-code and the overflow rule on grid points and midpoints.
"""
import numpy as np
import pytest
import torch

E4M3, E5M2 = 0, 1
TDT = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}


def test_format_constants(orc):
    # fp8_parity.py page: E4M3_MAX = 448, E5M2_MAX = 57344; smallest normals 2^-6, 2^-14
    assert orc.fmax(E4M3) == 448.0
    assert orc.fmax(E5M2) == 57344.0
    assert orc.smallest_normal(E4M3) == 2.0 ** -6
    assert orc.smallest_normal(E5M2) == 2.0 ** -14
    assert orc.decode(0x7E, E4M3) == 448.0
    assert orc.decode(0x7B, E5M2) == 57344.0
    assert orc.decode(0x08, E4M3) == 2.0 ** -6
    assert orc.decode(0x04, E5M2) == 2.0 ** -14
    assert orc.decode(0x01, E4M3) == 2.0 ** -9      # smallest subnormal
    assert orc.decode(0x01, E5M2) == 2.0 ** -16
    assert orc.decode(0x38, E4M3) == 1.0
    assert orc.decode(0x3C, E5M2) == 1.0
    assert np.isnan(orc.decode(0x7F, E4M3)) and np.isnan(orc.decode(0xFF, E4M3))
    assert orc.decode(0x7C, E5M2) == np.inf and orc.decode(0xFC, E5M2) == -np.inf
    assert all(np.isnan(orc.decode(c, E5M2)) for c in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF))
    assert torch.finfo(TDT[E4M3]).max == orc.fmax(E4M3)
    assert torch.finfo(TDT[E5M2]).max == orc.fmax(E5M2)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_decode_all_codes_match_torch(orc, fmt):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(TDT[fmt]).to(torch.float64).numpy()
    got = orc.decode_table(fmt)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(ref[~both_nan], got[~both_nan])
    assert np.array_equal(np.isnan(ref), np.isnan(got))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_every_fp32_pattern_matches_torch(orc, fmt):
    """Exhaustive: all 2^32 fp32 bit patterns, in chunks, against torch's cast."""
    chunk = 1 << 26
    base = np.arange(chunk, dtype=np.uint32)
    bits = np.empty_like(base)
    for lo in range(0, 1 << 32, chunk):
        np.add(base, np.uint32(lo), out=bits)
        ref = torch.from_numpy(bits.view(np.float32)).to(TDT[fmt]).view(torch.uint8).numpy()
        bad, first = orc.encode_compare_range(lo, lo + chunk, fmt, ref)
        assert bad == 0, f"first mismatch at fp32 bits {first:#010x}"


def _brute_force_encode(values, fmt):
    """Nearest of all finite codes plus the first value past the maximum (the
    overflow point); ties go to the code with mantissa LSB 0."""
    tab = np.array([np.nan] * 256)
    for c in range(256):
        e_bits, m_bits = (4, 3) if fmt == E4M3 else (5, 2)
        bias = 7 if fmt == E4M3 else 15
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> m_bits) & ((1 << e_bits) - 1)
        m = c & ((1 << m_bits) - 1)
        if fmt == E4M3 and e == 15 and m == 7:
            continue
        if fmt == E5M2 and e == 31:
            continue
        v = m * 2.0 ** (1 - bias - m_bits) if e == 0 else (1 + m / 2 ** m_bits) * 2.0 ** (e - bias)
        tab[c] = s * v
    pos = [(tab[c], c) for c in range(128) if not np.isnan(tab[c])]
    fmax_v = max(v for v, _ in pos)
    step = fmax_v - sorted(v for v, _ in pos)[-2]
    over = fmax_v + step          # first grid point past the maximum
    over_code_even = (fmt == E5M2)  # 0x7C (even) for E5M2, 0x7F (odd) for E4M3
    out = []
    for v in values:
        if np.isnan(v):
            out.append(("nan", None))
            continue
        a = abs(float(v))
        if a >= over:               # beyond every grid point: nearest is the overflow point
            out.append(("over", np.signbit(v)))
            continue
        cands = pos + [(over, "over")]
        dists = [abs(a - g) for g, _ in cands]
        dmin = min(dists)
        near = [cands[i] for i in range(len(cands)) if dists[i] == dmin]
        if len(near) == 2:
            def even(item):
                g, c = item
                return over_code_even if c == "over" else (c & 1) == 0
            near = [x for x in near if even(x)]
        g, c = near[0]
        if c == "over" or a == np.inf:
            out.append(("over", np.signbit(v)))
        else:
            out.append((c | (0x80 if np.signbit(v) else 0), None))
    return out


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_brute_force_on_grid_and_midpoints(orc, fmt):
    tab = orc.decode_table(fmt)
    fin = np.unique(np.abs(tab[np.isfinite(tab)]))
    mids = (fin[1:] + fin[:-1]) / 2
    fmax_v = fin[-1]
    extra = [fmax_v + (fin[-1] - fin[-2]) / 2, fmax_v + (fin[-1] - fin[-2]), 1e30, np.inf]
    pts = np.concatenate([fin, mids, extra]).astype(np.float32)
    vals = []
    for p in pts:
        for d in (-2, -1, 0, 1, 2):   # neighbouring fp32 values
            b = np.array([p], np.float32).view(np.uint32)[0]
            if p == 0 and d < 0:
                continue
            vals.append(np.array([int(b) + d], np.uint32).view(np.float32)[0])
    rng = np.random.default_rng(7)
    vals += list((rng.standard_normal(2000) * rng.choice([1e-3, 1, 30, 1e4], 2000)).astype(np.float32))
    vals = np.array(vals, np.float32)
    vals = np.concatenate([vals, -vals])
    got = orc.encode(vals, fmt)
    ref = _brute_force_encode(vals, fmt)
    for v, g, (r, neg) in zip(vals, got, ref):
        if r == "nan":
            assert (g & 0x7F) == 0x7F, (v, hex(g))
        elif r == "over":
            if fmt == E4M3:
                assert (g & 0x7F) == 0x7F, (v, hex(g))
            else:
                assert g == (0xFC if neg else 0x7C), (v, hex(g))
        else:
            assert g == r, (float(v), hex(g), hex(r))


def test_encode_hand_derived_cases(orc):
    e = lambda v, f, sat=False: int(orc.encode(np.array([v], np.float32), f, sat)[0])
    # E4M3: 448 = 1.75*2^8 (mantissa 110, even); the next grid point 480 is the NaN code,
    # so the midpoint 464 ties to 448 and anything above it overflows to NaN.
    assert e(448.0, E4M3) == 0x7E
    assert e(464.0, E4M3) == 0x7E
    assert e(np.nextafter(np.float32(464.0), np.float32(1e9)), E4M3) == 0x7F
    assert e(-600.0, E4M3) == 0xFF
    assert e(np.inf, E4M3) == 0x7F
    # 1.0625 is the midpoint of 1 (0x38, even) and 1.125 (0x39): ties to 0x38;
    # 1.1875 is the midpoint of 1.125 (0x39) and 1.25 (0x3A, even): ties to 0x3A.
    assert e(1.0625, E4M3) == 0x38
    assert e(1.1875, E4M3) == 0x3A
    # subnormals: quantum 2^-9; 1.5 q ties to 2 q (even), 2.5 q ties to 2 q; 0.5 q ties to 0
    q = 2.0 ** -9
    assert e(1.5 * q, E4M3) == 0x02
    assert e(2.5 * q, E4M3) == 0x02
    assert e(0.5 * q, E4M3) == 0x00
    assert e(-0.0, E4M3) == 0x80
    assert e(-1e-30, E4M3) == 0x80
    # E5M2: 57344 = 1.75*2^15 (mantissa 11, odd); the next grid point 65536 is Inf (0x7C,
    # even), so the midpoint 61440 ties to Inf and 61439 stays at 57344.
    assert e(57344.0, E5M2) == 0x7B
    assert e(61439.0, E5M2) == 0x7B
    assert e(61440.0, E5M2) == 0x7C
    assert e(-61440.0, E5M2) == 0xFC
    assert (e(np.nan, E5M2) & 0x7F) == 0x7F
    assert e(1.5 * 2.0 ** -16, E5M2) == 0x02
    # saturating variant clamps finite and infinite overflow to the largest finite code
    assert e(1000.0, E4M3, True) == 0x7E
    assert e(-600.0, E4M3, True) == 0xFE
    assert e(np.inf, E4M3, True) == 0x7E
    assert e(1e6, E5M2, True) == 0x7B
    assert (e(np.nan, E4M3, True) & 0x7F) == 0x7F
