"""CPU oracle for dynamic FP8 scaling and the scaled FP8 GEMM (ctypes over oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product library.  It shares no code
with the HIP path.  See oracle.c for the definitions and their sources.

High-precision inputs are numpy arrays: float32 (fp32) or uint16 holding
bfloat16 bit patterns.  Codes are uint8 arrays.
"""
import ctypes
import os

import numpy as np

from . import build as _build

E4M3, E5M2 = 0, 1
F32, BF16 = 0, 1

_lib = None


class ScaleDesc(ctypes.Structure):
    _fields_ = [("s", ctypes.c_void_p), ("e8m0", ctypes.c_int32), ("pad", ctypes.c_int32),
                ("rblk", ctypes.c_int64), ("kblk", ctypes.c_int64),
                ("s_rs", ctypes.c_int64), ("s_ks", ctypes.c_int64)]


def lib():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        L = ctypes.CDLL(path)
        P, I64, I32, F, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
        L.orc_fmax.restype, L.orc_fmax.argtypes = D, [I32]
        L.orc_smallest_normal.restype, L.orc_smallest_normal.argtypes = D, [I32]
        L.orc_decode.restype, L.orc_decode.argtypes = D, [ctypes.c_uint8, I32]
        L.orc_encode.restype, L.orc_encode.argtypes = ctypes.c_uint8, [F, I32, I32]
        L.orc_amax.restype, L.orc_amax.argtypes = F, [P, I32, I64]
        L.orc_scale_from_amax.restype, L.orc_scale_from_amax.argtypes = F, [F, I32]
        L.orc_cast1.restype, L.orc_cast1.argtypes = ctypes.c_uint8, [F, F, I32, I32]
        L.orc_cast.restype, L.orc_cast.argtypes = None, [P, I32, I64, F, I32, I32, P]
        L.orc_quantize_per_tensor.restype = None
        L.orc_quantize_per_tensor.argtypes = [P, I32, I64, I32, I32, P, P, P]
        L.orc_quantize_delayed.restype = None
        L.orc_quantize_delayed.argtypes = [P, I32, I64, I32, I32, P, P, I32, P, P, P]
        L.orc_quantize_tiles.restype = None
        L.orc_quantize_tiles.argtypes = [P, I32, I64, I64, I32, I64, I32, I32, I32, P, P, P]
        L.orc_quantize_blocks.restype = None
        L.orc_quantize_blocks.argtypes = [P, I32, I64, I64, I64, I64, I32, I32, P, P]
        L.orc_gemm.restype = None
        L.orc_gemm.argtypes = [I64, I64, I64, P, I64, I64, I32, ctypes.POINTER(ScaleDesc),
                               P, I64, I64, I32, ctypes.POINTER(ScaleDesc), P, I64, P]
        L.orc_encode_array.restype, L.orc_encode_array.argtypes = None, [P, I64, I32, I32, P]
        U32, U64 = ctypes.c_uint32, ctypes.c_uint64
        L.orc_philox4x32_10.restype, L.orc_philox4x32_10.argtypes = None, [P, P, P]
        L.orc_sr_word.restype, L.orc_sr_word.argtypes = U32, [U64, U64, U64]
        L.orc_set_threads.restype, L.orc_set_threads.argtypes = None, [I32]
        L.orc_overflow_count.restype, L.orc_overflow_count.argtypes = I64, [P, I32, I64, F, I32]
        L.orc_max_threads.restype, L.orc_max_threads.argtypes = I32, []
        L.orc_encode_sr.restype, L.orc_encode_sr.argtypes = ctypes.c_uint8, [F, U32, I32, I32]
        L.orc_quantize_per_tensor_sr.restype = None
        L.orc_quantize_per_tensor_sr.argtypes = [P, I32, I64, I32, I32, U64, U64, P, P, P]
        L.orc_rht_sign.restype, L.orc_rht_sign.argtypes = I32, [U64, I64]
        L.orc_rht.restype, L.orc_rht.argtypes = None, [P, I32, I64, I64, U64, P]
        L.orc_encode_compare_range.restype = I64
        L.orc_encode_compare_range.argtypes = [ctypes.c_uint64, ctypes.c_uint64, I32, P,
                                               ctypes.POINTER(ctypes.c_uint64)]
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _hp(x):
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError(f"oracle input must be float32 or uint16 (bf16 bits), got {x.dtype}")


# ---------------------------------------------------------------- codec
def fmax(fmt):
    return lib().orc_fmax(fmt)


def smallest_normal(fmt):
    return lib().orc_smallest_normal(fmt)


def decode(code, fmt):
    return lib().orc_decode(int(code), fmt)


def decode_table(fmt):
    return np.array([decode(c, fmt) for c in range(256)], dtype=np.float64)


def decode_array(codes, fmt):
    return decode_table(fmt)[np.asarray(codes, dtype=np.uint8)]


def encode(v, fmt, saturate=False):
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().orc_encode_array(_ptr(v), v.size, fmt, int(saturate), _ptr(out))
    return out


def encode_compare_range(lo, hi, fmt, ref):
    ref = np.ascontiguousarray(ref, dtype=np.uint8)
    assert ref.size == hi - lo
    first = ctypes.c_uint64(0)
    bad = lib().orc_encode_compare_range(lo, hi, fmt, _ptr(ref), ctypes.byref(first))
    return bad, first.value


# ---------------------------------------------------------------- threads (timing only)
def set_threads(n):
    """Thread count of the oracle's parallel loops (results do not depend on it)."""
    lib().orc_set_threads(int(n))


def max_threads():
    return int(lib().orc_max_threads())


# ---------------------------------------------------------------- amax / scale / cast
def amax(x):
    x, hp = _hp(x)
    return np.float32(lib().orc_amax(_ptr(x), hp, x.size))


def scale_from_amax(a, fmt):
    return np.float32(lib().orc_scale_from_amax(float(a), fmt))


def cast(x, s, fmt, saturate=False):
    x, hp = _hp(x)
    q = np.empty(x.shape, dtype=np.uint8)
    lib().orc_cast(_ptr(x), hp, x.size, float(s), fmt, int(saturate), _ptr(q))
    return q


def overflow_count(x, s, fmt):
    """Finite elements whose non-saturating cast with scale s overflows the
    format (E4M3 NaN code, E5M2 Inf code)."""
    x, hp = _hp(x)
    return int(lib().orc_overflow_count(_ptr(x), hp, x.size, float(s), fmt))


def quantize_per_tensor(x, fmt, saturate=False):
    """Current scaling: returns (codes, scale, amax)."""
    x, hp = _hp(x)
    q = np.empty(x.shape, dtype=np.uint8)
    s = np.zeros(1, np.float32)
    a = np.zeros(1, np.float32)
    lib().orc_quantize_per_tensor(_ptr(x), hp, x.size, fmt, int(saturate), _ptr(q), _ptr(s), _ptr(a))
    return q, s[0], a[0]


def philox4x32_10(ctr, key):
    """Philox4x32-10 of a 4-word counter and a 2-word key -> 4 words."""
    c = np.ascontiguousarray(ctr, np.uint32)
    k = np.ascontiguousarray(key, np.uint32)
    out = np.zeros(4, np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_word(seed, offset, i):
    return int(lib().orc_sr_word(int(seed), int(offset), int(i)))


def encode_sr(v, r, fmt, saturate=False):
    return int(lib().orc_encode_sr(float(v), int(r) & 0xFFFFFFFF, fmt, int(saturate)))


def quantize_per_tensor_sr(x, fmt, seed, offset=0, saturate=False):
    """Current scaling with a stochastically rounded cast: (codes, scale, amax)."""
    x, hp = _hp(x)
    q = np.empty(x.shape, dtype=np.uint8)
    s = np.zeros(1, np.float32)
    a = np.zeros(1, np.float32)
    lib().orc_quantize_per_tensor_sr(_ptr(x), hp, x.size, fmt, int(saturate), int(seed), int(offset), _ptr(q),
                                     _ptr(s), _ptr(a))
    return q, s[0], a[0]


def rht_sign(seed, t):
    return int(lib().orc_rht_sign(int(seed), int(t)))


def rht(x, seed):
    """Random Hadamard transform along rows (16-row blocks): fp32 [rows, cols]."""
    x, hp = _hp(x)
    rows, cols = x.shape
    y = np.empty((rows, cols), np.float32)
    lib().orc_rht(_ptr(x), hp, rows, cols, int(seed), _ptr(y))
    return y


def quantize_per_tensor_rht(x, fmt, seed, saturate=False):
    """The transform, then per-tensor current quantization of its fp32 result:
    (codes, scale, amax of the transformed tensor)."""
    return quantize_per_tensor(rht(x, seed), fmt, saturate)


class DelayedState:
    """Amax history ring (16 entries) and position, as plain host arrays."""

    def __init__(self, length=16):
        self.hist = np.zeros(length, np.float32)
        self.pos = np.zeros(1, np.int32)


def quantize_delayed(x, fmt, state, saturate=False):
    """Delayed scaling step: returns (codes, scale, amax); updates state."""
    x, hp = _hp(x)
    q = np.empty(x.shape, dtype=np.uint8)
    s = np.zeros(1, np.float32)
    a = np.zeros(1, np.float32)
    lib().orc_quantize_delayed(_ptr(x), hp, x.size, fmt, int(saturate), _ptr(state.hist),
                               _ptr(state.pos), state.hist.size, _ptr(q), _ptr(s), _ptr(a))
    return q, s[0], a[0]


def quantize_tiles(x, axis, tile, fmt, saturate=False, mx=False):
    """1 x tile (axis 0) or tile x 1 (axis 1) scaling of a 2-D array.

    Returns (codes [rows, cols], scales): fp32 scales, or E8M0 bytes if mx;
    scales are [rows, ceil(cols/tile)] for axis 0, [cols, ceil(rows/tile)] for axis 1.
    """
    x, hp = _hp(x)
    rows, cols = x.shape
    q = np.empty(x.shape, dtype=np.uint8)
    nt = -(-cols // tile) if axis == 0 else -(-rows // tile)
    outer = rows if axis == 0 else cols
    if mx:
        sc = np.zeros((outer, nt), np.uint8)
        lib().orc_quantize_tiles(_ptr(x), hp, rows, cols, axis, tile, fmt, int(saturate), 1,
                                 _ptr(q), None, _ptr(sc))
    else:
        sc = np.zeros((outer, nt), np.float32)
        lib().orc_quantize_tiles(_ptr(x), hp, rows, cols, axis, tile, fmt, int(saturate), 0,
                                 _ptr(q), _ptr(sc), None)
    return q, sc


def quantize_rowwise(x, axis, fmt, saturate=False):
    """Rowwise scaling (the lab page's "rowwise" recipe): one scale per row
    (axis 0) or per column (axis 1), i.e. a 1 x cols or rows x 1 tile.
    Returns (codes [rows, cols], fp32 scales [rows] or [cols])."""
    rows, cols = np.asarray(x).shape
    q, sc = quantize_tiles(x, axis, cols if axis == 0 else rows, fmt, saturate)
    return q, sc.reshape(-1)


def quantize_blocks(x, br, bc, fmt, saturate=False):
    """br x bc block scaling; returns (codes, fp32 scales [ceil(rows/br), ceil(cols/bc)])."""
    x, hp = _hp(x)
    rows, cols = x.shape
    q = np.empty(x.shape, dtype=np.uint8)
    sc = np.zeros((-(-rows // br), -(-cols // bc)), np.float32)
    lib().orc_quantize_blocks(_ptr(x), hp, rows, cols, br, bc, fmt, int(saturate), _ptr(q), _ptr(sc))
    return q, sc


# ---------------------------------------------------------------- GEMM
class Scale:
    """Scale of one GEMM operand as a function of (operand row, k).

    kind 'tensor': one fp32 scalar.
    kind 'rowk':   array [rows, ceil(K/kblk)] indexed by (row, k // kblk)
                   (1 x 128 tiles, MX32 blocks, 128 x 1 tiles of a wgrad operand).
    kind 'block':  array [ceil(rows/rblk), ceil(K/kblk)] (2-D blocks).
    kind 'blockT': 2-D block scales stored [ceil(K/kblk), ceil(rows/rblk)]
                   (a weight used in dgrad, where its rows are the contraction).
    e8m0: scales are E8M0 bytes (2^(code-127)).
    """

    def __init__(self, kind, value, kblk=None, rblk=None, e8m0=False):
        self.kind, self.kblk, self.rblk, self.e8m0 = kind, kblk, rblk, e8m0
        if kind == "tensor":
            self.arr = np.array([value], dtype=np.float32)
        else:
            self.arr = np.ascontiguousarray(value, dtype=np.uint8 if e8m0 else np.float32)

    @staticmethod
    def rowwise(scales, K):
        """One scale per operand row over all of K: the 1 x K tile of 'rowk'."""
        return Scale("rowk", np.asarray(scales, np.float32).reshape(-1, 1), kblk=max(int(K), 1))

    def desc(self, rows, K):
        d = ScaleDesc()
        d.s = self.arr.ctypes.data
        d.e8m0 = int(self.e8m0)
        if self.kind == "tensor":
            d.rblk, d.kblk, d.s_rs, d.s_ks = max(rows, 1), max(K, 1), 0, 0
        elif self.kind == "rowk":
            d.rblk, d.kblk, d.s_rs, d.s_ks = 1, self.kblk, self.arr.shape[1], 1
        elif self.kind == "block":
            d.rblk, d.kblk, d.s_rs, d.s_ks = self.rblk, self.kblk, self.arr.shape[1], 1
        elif self.kind == "blockT":
            d.rblk, d.kblk, d.s_rs, d.s_ks = self.rblk, self.kblk, 1, self.arr.shape[1]
        else:
            raise ValueError(self.kind)
        return d


def _gemm(M, N, K, A, a_sm, a_sk, fa, sa, B, b_sn, b_sk, fb, sb, rows=None):
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    if rows is None:
        nrows, rp = M, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        nrows, rp = rows.size, _ptr(rows)
    C = np.zeros((nrows, N), np.float64)
    da, db = sa.desc(M, K), sb.desc(N, K)
    lib().orc_gemm(M, N, K, _ptr(A), a_sm, a_sk, fa, ctypes.byref(da),
                   _ptr(B), b_sn, b_sk, fb, ctypes.byref(db), rp, nrows, _ptr(C))
    return C


def gemm_nt(A, B, fa, fb, sa, sb, rows=None):
    """fprop: y[m,n] = sum_k A[m,k] B[n,k] (A [M,K], B [N,K] as stored)."""
    M, K = A.shape
    N = B.shape[0]
    return _gemm(M, N, K, A, K, 1, fa, sa, B, K, 1, fb, sb, rows)


def gemm_nn(A, B, fa, fb, sa, sb, rows=None):
    """dgrad: y[m,n] = sum_k A[m,k] B[k,n] (A [M,K], B [K,N] as stored)."""
    M, K = A.shape
    N = B.shape[1]
    return _gemm(M, N, K, A, K, 1, fa, sa, B, 1, N, fb, sb, rows)


def gemm_tn(A, B, fa, fb, sa, sb, rows=None):
    """wgrad: y[m,n] = sum_k A[k,m] B[k,n] (A [K,M], B [K,N] as stored)."""
    K, M = A.shape
    N = B.shape[1]
    return _gemm(M, N, K, A, 1, M, fa, sa, B, 1, N, fb, sb, rows)
