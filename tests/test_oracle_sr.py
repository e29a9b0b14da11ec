"""Pins of the oracle's stochastic rounding and its counter-based generator.

The generator is Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random
Numbers: As Easy as 1, 2, 3", SC 2011); its published known-answer vectors
(the Random123 test vectors) pin it.  Stochastic rounding is pinned by what
its definition fixes: grid values are kept, every result is one of the two
neighbouring grid values, the rounding-up count over an evenly spread set of
random words equals the fractional position exactly, and the mean over the
generator's stream is unbiased."""
import numpy as np
import pytest
import torch

E4M3, E5M2 = 0, 1
TORCH_FP8 = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}


def grid(fmt):
    """Sorted finite non-negative values of the format (torch's own decode)."""
    v = torch.arange(128, dtype=torch.uint8).view(TORCH_FP8[fmt]).float().numpy().astype(np.float64)
    return np.unique(v[np.isfinite(v)])


@pytest.mark.parametrize("ctr,key,expect", [
    ((0, 0, 0, 0), (0, 0), (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff,) * 4, (0xffffffff,) * 2, (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
])
def test_philox_known_answers(orc, ctr, key, expect):
    assert tuple(int(v) for v in orc.philox4x32_10(ctr, key)) == expect


def test_sr_word_layout(orc):
    """Element i takes word i mod 4 of the block of counter i / 4 (and offset in
    the upper counter words, seed as the key)."""
    seed, off = 0x0123456789ABCDEF, 0x1122334455667788
    for i in (0, 1, 2, 3, 4, 7, 1 << 33 | 2):
        g = i >> 2
        words = orc.philox4x32_10((g & 0xffffffff, g >> 32, off & 0xffffffff, off >> 32),
                                  (seed & 0xffffffff, seed >> 32))
        assert orc.sr_word(seed, off, i) == int(words[i & 3])


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_grid_values_are_kept(orc, fmt):
    rng = np.random.default_rng(3)
    for v in grid(fmt):
        for sign in (1.0, -1.0):
            ref = orc.encode(sign * v, fmt)
            for r in (0, 0xffffffff, int(rng.integers(0, 1 << 32))):
                assert orc.encode_sr(sign * v, r, fmt) == ref


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_result_is_a_neighbour_and_count_is_exact(orc, fmt):
    """For v = lo + (k/256) D between grid neighbours lo < hi = lo + D, the
    256 random words j * 2^24 round up exactly k times, and every result is
    lo or hi (with the sign of v)."""
    g = grid(fmt)
    rng = np.random.default_rng(4 + fmt)
    for idx in rng.choice(len(g) - 1, 24, replace=False):
        lo, hi = g[idx], g[idx + 1]
        for k in (0, 1, 77, 128, 255):
            v = lo + (hi - lo) * k / 256
            assert np.float32(v) == v
            for sign in (1.0, -1.0):
                codes = [orc.encode_sr(sign * v, j << 24, fmt) for j in range(256)]
                up = sum(c == orc.encode(sign * hi, fmt) for c in codes)
                down = sum(c == orc.encode(sign * lo, fmt) for c in codes)
                assert up == k and down == 256 - k, (lo, hi, k, up, down)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_unbiased_over_the_stream(orc, fmt):
    """The mean of SR(v) over 20000 consecutive words of the stream is v within
    five standard errors (the variance of a two-point rounding is (v-lo)(hi-v))."""
    g = grid(fmt)
    lo, hi = g[40], g[41]
    v = float(np.float32(lo + 0.3 * (hi - lo)))
    codes = np.array([orc.encode_sr(v, orc.sr_word(7, 0, i), fmt) for i in range(20000)], np.uint8)
    vals = torch.from_numpy(codes).view(TORCH_FP8[fmt]).double().numpy()
    se = np.sqrt((v - lo) * (hi - v) / len(vals))
    assert abs(vals.mean() - v) <= 5 * se


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_quantize_sr_against_round_to_nearest(orc, fmt):
    """Same scale as the round-to-nearest cast; every code's value is within one
    grid step of RN32(x / s) and is one of its two grid neighbours."""
    x = (np.random.default_rng(9).standard_normal(5000) * 3).astype(np.float32)
    q, s, a = orc.quantize_per_tensor_sr(x, fmt, seed=11, offset=3)
    q0, s0, a0 = orc.quantize_per_tensor(x, fmt)
    assert s == s0 and a == a0
    v = (x / np.float32(s)).astype(np.float64)   # numpy fp32 division, widened exactly
    got = torch.from_numpy(q).view(TORCH_FP8[fmt]).double().numpy()
    g = grid(fmt)
    lo_i = np.searchsorted(g, np.abs(v), side="right") - 1
    lo = g[lo_i] * np.sign(v)
    hi = g[np.minimum(lo_i + 1, len(g) - 1)] * np.sign(v)
    assert np.all((got == lo) | (got == hi))
    assert np.any(q != q0)


MAXCODE = {E4M3: 0x7E, E5M2: 0x7B}
FMAX = {E4M3: 448.0, E5M2: 57344.0}


@pytest.mark.parametrize("ctr,key,expect", [
    ((0, 0, 0, 0), (0, 0), (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff,) * 4, (0xffffffff,) * 2, (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
])
def test_search_generator_known_answers(ctr, key, expect):
    """The numpy generator the edge-case search uses meets the same published vectors."""
    import sr_search
    assert tuple(int(w) for w in sr_search.philox4x32_10(*ctr, *key)) == expect


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_sr_caps_at_fmax_where_round_to_nearest_is_finite(orc, fmt):
    """A quotient one ulp above fmax (where current scaling can put the amax
    element) never rounds up past fmax, whatever the word; so does the largest
    value whose round-to-nearest cast is finite.  Past that limit the
    stochastic result overflows as the cast does."""
    above = float(np.nextafter(np.float32(FMAX[fmt]), np.float32(np.inf)))
    last_finite = 464.0 if fmt == E4M3 else float(np.nextafter(np.float32(61440.0), np.float32(0)))
    first_over = float(np.nextafter(np.float32(464.0), np.float32(np.inf))) if fmt == E4M3 else 61440.0
    ovf = 0x7F if fmt == E4M3 else 0x7C
    for v in (above, last_finite):
        assert orc.encode(v, fmt) == MAXCODE[fmt]
        for sign in (1.0, -1.0):
            for r in (0, 1 << 31, 0xffffffff):
                assert orc.encode_sr(sign * v, r, fmt) == MAXCODE[fmt] | (0x80 if sign < 0 else 0)
    assert orc.encode(first_over, fmt) & 0x7F == ovf
    assert orc.encode_sr(first_over, 0xffffffff, fmt) & 0x7F == ovf
    assert orc.encode_sr(first_over, 0, fmt) == MAXCODE[fmt]


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_sr_amax_element_stays_finite(orc, fmt):
    """Per-tensor current scaling of a bf16 tensor whose amax element is cast
    from one ulp above fmax, with a stream offset whose word for that element
    would round it up: the element's code is the largest finite code."""
    import sr_search
    a = sr_search.bf16_amax_one_ulp_above(FMAX[fmt])
    assert a is not None
    s = np.float32(a) / np.float32(FMAX[fmt])
    v = np.float32(a) / s
    D = 32.0 if fmt == E4M3 else 8192.0          # grid spacing at fmax
    frac32 = int(np.floor((float(v) / D - np.floor(float(v) / D)) * 2.0 ** 32))
    assert frac32 > 0
    seed = 0x5EED
    off = sr_search.find_offset(seed, 0, (1 << 32) - frac32)
    assert off is not None and orc.sr_word(seed, off, 0) >= (1 << 32) - frac32
    x = (np.random.default_rng(12).standard_normal(4096) * 0.25).astype(np.float32)
    x[0] = a
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    q, s_o, a_o = orc.quantize_per_tensor_sr(bits, fmt, seed=seed, offset=off)
    assert a_o == a and s_o == s
    assert q[0] == MAXCODE[fmt]
