"""Search helpers for stochastic-rounding edge cases (test inputs only).

A vectorised numpy statement of Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011), used to find a
stream offset whose word for a given element is large enough to round a value
up.  It is checked against the generator's published known-answer vectors in
test_oracle_sr.py, and every offset it finds is re-checked with the oracle's
own generator before use.  Neither the oracle nor the HIP library imports it.
"""
import numpy as np

_M0, _M2 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = np.uint64(0x9E3779B9), np.uint64(0xBB67AE85)
_LO = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Ten rounds over arrays (or scalars) of 32-bit counter words; returns the
    four output words as uint64 arrays holding 32-bit values."""
    c0, c1, c2, c3 = (np.asarray(c, np.uint64) & _LO for c in (c0, c1, c2, c3))
    k0, k1 = np.uint64(k0) & _LO, np.uint64(k1) & _LO
    for rnd in range(10):
        if rnd:
            k0 = (k0 + _W0) & _LO
            k1 = (k1 + _W1) & _LO
        p0 = _M0 * c0
        p1 = _M2 * c2
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ k0, p1 & _LO, (p0 >> np.uint64(32)) ^ c3 ^ k1, p0 & _LO)
    return c0, c1, c2, c3


def find_offset(seed, element, min_word, start=0, limit=1 << 25, chunk=1 << 20):
    """Smallest offset >= start whose word for `element` (word element % 4 of
    counter (element / 4, offset)) is >= min_word; None if none below start + limit."""
    g = element >> 2
    for base in range(start, start + limit, chunk):
        off = np.arange(base, base + chunk, dtype=np.uint64)
        words = philox4x32_10(np.uint64(g & 0xFFFFFFFF), np.uint64(g >> 32), off & _LO, off >> np.uint64(32),
                              seed & 0xFFFFFFFF, seed >> 32)[element & 3]
        hit = np.nonzero(words >= np.uint64(min_word))[0]
        if hit.size:
            return int(off[hit[0]])
    return None


def bf16_amax_one_ulp_above(fmax):
    """A bf16 value a (as fp32) whose per-tensor quotient RN32(a / RN32(a /
    fmax)) is the fp32 value one ulp above fmax: the amax element of such a
    tensor is cast from just past the format maximum.  numpy's fp32 division
    is IEEE (correctly rounded)."""
    target = np.nextafter(np.float32(fmax), np.float32(np.inf))
    bits = np.arange(0x3F80, 0x4780, dtype=np.uint32) << np.uint32(16)   # bf16 values in [1, 65536)
    a = bits.view(np.float32)
    s = a / np.float32(fmax)
    v = a / s
    hit = np.nonzero(v == target)[0]
    return float(a[hit[0]]) if hit.size else None
