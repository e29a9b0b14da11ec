"""fp8q: dynamic FP8 scaling and the scaled FP8 GEMM on AMD MI355X (gfx950).

Thin Python binding over the C ABI of libfp8q.so (include/fp8q.h): argument
marshalling only.  Every computation runs in the library's HIP kernels on the
caller's current HIP stream; torch provides device memory and streams.  There
is no fallback: if the library is missing or the device is not a gfx950 the
calls raise.
"""
import ctypes
import os

import torch

E4M3, E5M2 = 0, 1
F32, BF16 = 0, 1
PER_TENSOR, TILE_1x128, BLOCK_128x128, MX32, ROWWISE = 0, 1, 2, 3, 4
CURRENT, DELAYED = 0, 1
SATURATE = 1
COUNT_OVERFLOW = 2
HISTORY_LEN = 16

OK, EINVAL, EALIGN, EUNSUPPORTED, EDEVICE, ELAUNCH, EWORKSPACE = range(7)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp8q.so")
_lib = None

_TORCH_HP = {torch.float32: F32, torch.bfloat16: BF16}
_FP8_DTYPE = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}


class Fp8qError(RuntimeError):
    """A non-OK status from the library (status code in .status)."""

    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


class Operand(ctypes.Structure):
    """fp8q_operand (see include/fp8q.h)."""
    _fields_ = [("data", ctypes.c_void_p), ("data_kmajor", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("quantized", ctypes.c_int32), ("format", ctypes.c_int32), ("granularity", ctypes.c_int32),
                ("hp", ctypes.c_int32), ("scaling", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("state", ctypes.c_void_p), ("scale_out", ctypes.c_void_p), ("amax_out", ctypes.c_void_p)]


def lib():
    """Load libfp8q.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(hipcc for gfx950); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64, U, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint, ctypes.c_size_t
        OP = ctypes.POINTER(Operand)
        sigs = {
            "fp8q_abi_version": (I, []),
            "fp8q_status_string": (ctypes.c_char_p, [I]),
            "fp8q_last_error": (ctypes.c_char_p, []),
            "fp8q_reduce_workspace_bytes": (SZ, []),
            "fp8_amax": (I, [P, I, I64, P, P, SZ, P]),
            "fp8_quantize_per_tensor": (I, [P, I, I64, I64, I, I, P, P, P, P, P, U, P, SZ, P]),
            "fp8_quantize_per_tensor_noalloc": (I, [P, I, I64, I64, I, I, P, P, P, P, P, U, P]),
            "fp8_quantize_tile1x128": (I, [P, I, I64, I64, I, I, P, P, P, U, P]),
            "fp8_quantize_block128x128": (I, [P, I, I64, I64, I, P, P, P, U, P]),
            "fp8_quantize_mx32": (I, [P, I, I64, I64, I, I, P, P, P, U, P]),
            "fp8_quantize_rowwise": (I, [P, I, I64, I64, I, I, P, P, P, U, P]),
            "fp8_quantize_per_tensor_sr": (I, [P, I, I64, I64, I, ctypes.c_uint64, ctypes.c_uint64, P, P, P, P, U, P,
                                               SZ, P]),
            "fp8_quantize_per_tensor_rht": (I, [P, I, I64, I64, I, ctypes.c_uint64, P, P, P, P, U, P, SZ, P]),
            "fp8_gemm_workspace_bytes": (SZ, [I, I64, I64, I64, OP, OP]),
            "fp8_gemm_scaled_NT": (I, [I64, I64, I64, OP, OP, P, I, P, SZ, P]),
            "fp8_gemm_scaled_NN": (I, [I64, I64, I64, OP, OP, P, I, P, SZ, P]),
            "fp8_gemm_scaled_TN": (I, [I64, I64, I64, OP, OP, P, I, P, SZ, P]),
            "fp8q_mfma_loop": (I, [I, I, P, P]),
            "fp8q_mfma_loop_data": (I, [I, I, I, P, P]),
        }
        for name, (res, args) in sigs.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def _check(status):
    if status != OK:
        L = lib()
        msg = f"{L.fp8q_status_string(status).decode()}: {L.fp8q_last_error().decode()}"
        if status in (EINVAL, EALIGN, EUNSUPPORTED, EWORKSPACE):
            raise ValueError(msg)
        raise Fp8qError(status, msg)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _hp(x):
    if x.dtype not in _TORCH_HP:
        raise ValueError(f"input dtype must be float32 or bfloat16, got {x.dtype}")
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("input must be a contiguous CUDA (HIP) tensor")
    return _TORCH_HP[x.dtype]


def _rows_cols(x):
    if x.dim() == 1:
        return 1, x.shape[0]
    return x.reshape(-1, x.shape[-1]).shape


def _ws(nbytes, device):
    """Device workspace, zero-filled: the reduction counters in it must start at 0."""
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def reduce_workspace(device):
    """Reduction workspace (zero-filled: its completion counters must start at 0)."""
    return _ws(lib().fp8q_reduce_workspace_bytes(), device)


# ---------------------------------------------------------------- delayed state
class DelayedState:
    """fp8q_delayed_state in device memory: 16 fp32 amax history entries, the
    ring position and working fields (80 bytes), zero-initialised (cold start)."""
    NBYTES = 16 * 4 + 4 + 4 + 4 + 4

    def __init__(self, device="cuda"):
        self.buf = torch.zeros(self.NBYTES, dtype=torch.uint8, device=device)

    def ptr(self):
        return ctypes.c_void_p(self.buf.data_ptr())

    @property
    def history(self):
        return self.buf[:64].view(torch.float32)

    @property
    def pos(self):
        return self.buf[64:68].view(torch.int32)

    @property
    def overflows(self):
        """Overflowing elements of the last delayed call made with
        count_overflow (0 after a call without it)."""
        return self.buf[68:72].view(torch.int32)

    @property
    def last_scale(self):
        return self.buf[76:80].view(torch.float32)


# ---------------------------------------------------------------- amax / quantize
def fp8q_mfma_loop(blocks, iters, device="cuda", random_operands=False):
    """Measurement aid (not the FP8 path): `blocks` x 256 threads, each wave
    running `iters` rounds of 8 register-only FP8 MFMAs; returns the per-thread
    outputs (each exactly 4096 * iters for iters <= 4096 with the default
    all-ones operands; finite with random_operands, which needs iters % 8 == 0)."""
    out = torch.empty(blocks * 256, dtype=torch.float32, device=device)
    _check(lib().fp8q_mfma_loop_data(blocks, iters, 1 if random_operands else 0, _ptr(out), _stream()))
    return out


def fp8_amax(x, ws=None):
    """amax = max|x| over all elements (float32 tensor [1])."""
    hp = _hp(x)
    out = torch.empty(1, dtype=torch.float32, device=x.device)
    ws = reduce_workspace(x.device) if ws is None else ws
    _check(lib().fp8_amax(_ptr(x), hp, x.numel(), _ptr(out), _ptr(ws), ws.numel(), _stream()))
    return out


def fp8_quantize_per_tensor(x, fmt=E4M3, scaling=CURRENT, state=None, emit_t=False, saturate=False, ws=None,
                            count_overflow=False):
    """Per-tensor quantization of a 2-D (or 1-D) tensor; returns (q, qT, scale, amax).
    count_overflow (delayed scaling): the overflowing elements go to state.overflows."""
    hp = _hp(x)
    rows, cols = _rows_cols(x)
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    qT = torch.empty((cols, rows), dtype=torch.uint8, device=x.device) if emit_t else None
    scale = torch.empty(1, dtype=torch.float32, device=x.device)
    amax = torch.empty(1, dtype=torch.float32, device=x.device)
    ws = reduce_workspace(x.device) if ws is None else ws
    st = state.ptr() if state is not None else None
    _check(lib().fp8_quantize_per_tensor(_ptr(x), hp, rows, cols, fmt, scaling, st, _ptr(q), _ptr(qT),
                                         _ptr(scale), _ptr(amax),
                                         (SATURATE if saturate else 0) | (COUNT_OVERFLOW if count_overflow else 0),
                                         _ptr(ws), ws.numel(), _stream()))
    return q, qT, scale, amax


def fp8_quantize_per_tensor_noalloc(x, fmt=E4M3, scaling=CURRENT, state=None, emit_t=False, saturate=False,
                                    count_overflow=False, out=None):
    """fp8_quantize_per_tensor with the library's own device scratch in place of a
    workspace; returns (q, qT, scale, amax).  out = (q, qT, scale, amax) tensors
    to write into (qT may be None), so that the call itself allocates nothing."""
    hp = _hp(x)
    rows, cols = _rows_cols(x)
    if out is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
        qT = torch.empty((cols, rows), dtype=torch.uint8, device=x.device) if emit_t else None
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
        amax = torch.empty(1, dtype=torch.float32, device=x.device)
    else:
        q, qT, scale, amax = out
    st = state.ptr() if state is not None else None
    _check(lib().fp8_quantize_per_tensor_noalloc(_ptr(x), hp, rows, cols, fmt, scaling, st, _ptr(q), _ptr(qT),
                                                 _ptr(scale), _ptr(amax),
                                                 (SATURATE if saturate else 0) |
                                                 (COUNT_OVERFLOW if count_overflow else 0), _stream()))
    return q, qT, scale, amax


def fp8_quantize_per_tensor_sr(x, fmt=E5M2, seed=0, offset=0, emit_t=False, saturate=False, ws=None):
    """Current scaling with a stochastically rounded cast (Philox4x32-10 words
    from seed and offset); returns (q, qT, scale, amax)."""
    hp = _hp(x)
    rows, cols = _rows_cols(x)
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    qT = torch.empty((cols, rows), dtype=torch.uint8, device=x.device) if emit_t else None
    scale = torch.empty(1, dtype=torch.float32, device=x.device)
    amax = torch.empty(1, dtype=torch.float32, device=x.device)
    ws = reduce_workspace(x.device) if ws is None else ws
    _check(lib().fp8_quantize_per_tensor_sr(_ptr(x), hp, rows, cols, fmt, int(seed) & (2 ** 64 - 1),
                                            int(offset) & (2 ** 64 - 1), _ptr(q), _ptr(qT), _ptr(scale), _ptr(amax),
                                            SATURATE if saturate else 0, _ptr(ws), ws.numel(), _stream()))
    return q, qT, scale, amax


def fp8_quantize_per_tensor_rht(x, fmt=E4M3, seed=0, emit_t=False, saturate=False, ws=None):
    """Random Hadamard transform along rows (16-row blocks, signs from seed),
    then per-tensor current quantization; returns (q, qT, scale, amax)."""
    hp = _hp(x)
    rows, cols = _rows_cols(x)
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    qT = torch.empty((cols, rows), dtype=torch.uint8, device=x.device) if emit_t else None
    scale = torch.empty(1, dtype=torch.float32, device=x.device)
    amax = torch.empty(1, dtype=torch.float32, device=x.device)
    ws = reduce_workspace(x.device) if ws is None else ws
    _check(lib().fp8_quantize_per_tensor_rht(_ptr(x), hp, rows, cols, fmt, int(seed) & (2 ** 64 - 1), _ptr(q),
                                             _ptr(qT), _ptr(scale), _ptr(amax), SATURATE if saturate else 0, _ptr(ws),
                                             ws.numel(), _stream()))
    return q, qT, scale, amax


def fp8_quantize_tile1x128(x, axis=0, fmt=E4M3, emit_t=False, saturate=False):
    """1x128 (axis 0) or 128x1 (axis 1) tiles; returns (q, qT, scales)."""
    hp = _hp(x)
    rows, cols = _rows_cols(x)
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    qT = torch.empty((cols, rows), dtype=torch.uint8, device=x.device) if emit_t else None
    shape = (rows, -(-cols // 128)) if axis == 0 else (cols, -(-rows // 128))
    sc = torch.empty(shape, dtype=torch.float32, device=x.device)
    _check(lib().fp8_quantize_tile1x128(_ptr(x), hp, rows, cols, axis, fmt, _ptr(q), _ptr(qT), _ptr(sc),
                                        SATURATE if saturate else 0, _stream()))
    return q, qT, sc


def fp8_quantize_block128x128(x, fmt=E4M3, emit_t=False, saturate=False):
    """128x128 blocks; returns (q, qT, scales [ceil(rows/128), ceil(cols/128)])."""
    hp = _hp(x)
    rows, cols = _rows_cols(x)
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    qT = torch.empty((cols, rows), dtype=torch.uint8, device=x.device) if emit_t else None
    sc = torch.empty((-(-rows // 128), -(-cols // 128)), dtype=torch.float32, device=x.device)
    _check(lib().fp8_quantize_block128x128(_ptr(x), hp, rows, cols, fmt, _ptr(q), _ptr(qT), _ptr(sc),
                                           SATURATE if saturate else 0, _stream()))
    return q, qT, sc


def fp8_quantize_mx32(x, axis=0, fmt=E4M3, emit_t=False, saturate=False):
    """MX32 blocks with E8M0 scales; returns (q, qT, e8m0)."""
    hp = _hp(x)
    rows, cols = _rows_cols(x)
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    qT = torch.empty((cols, rows), dtype=torch.uint8, device=x.device) if emit_t else None
    shape = (rows, -(-cols // 32)) if axis == 0 else (cols, -(-rows // 32))
    e8 = torch.empty(shape, dtype=torch.uint8, device=x.device)
    _check(lib().fp8_quantize_mx32(_ptr(x), hp, rows, cols, axis, fmt, _ptr(q), _ptr(qT), _ptr(e8),
                                   SATURATE if saturate else 0, _stream()))
    return q, qT, e8


def fp8_quantize_rowwise(x, axis=0, fmt=E4M3, emit_t=False, saturate=False):
    """One scale per row (axis 0) or per column (axis 1); returns (q, qT, scales).
    qT (the K-major copy) is available with axis 1 only."""
    hp = _hp(x)
    rows, cols = _rows_cols(x)
    if emit_t and axis == 0:
        raise ValueError("rowwise axis 0 has no transposed copy")
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    qT = torch.empty((cols, rows), dtype=torch.uint8, device=x.device) if emit_t else None
    sc = torch.empty(rows if axis == 0 else cols, dtype=torch.float32, device=x.device)
    _check(lib().fp8_quantize_rowwise(_ptr(x), hp, rows, cols, axis, fmt, _ptr(q), _ptr(qT), _ptr(sc),
                                      SATURATE if saturate else 0, _stream()))
    return q, qT, sc


# ---------------------------------------------------------------- GEMM
class GemmOperand:
    """Python side of fp8q_operand; keeps the tensors it points at alive."""

    def __init__(self, op, keep):
        self.op, self.keep = op, keep

    @staticmethod
    def quantized(codes, fmt, scale, granularity=PER_TENSOR, kmajor=None):
        for t in (codes, kmajor):
            if t is not None and (t.dtype != torch.uint8 or not t.is_cuda or not t.is_contiguous()):
                raise ValueError("codes must be contiguous uint8 CUDA tensors")
        op = Operand(data=codes.data_ptr(), data_kmajor=None if kmajor is None else kmajor.data_ptr(),
                     scale=scale.data_ptr(), quantized=1, format=fmt, granularity=granularity)
        return GemmOperand(op, (codes, kmajor, scale))

    @staticmethod
    def autocast(x, fmt, granularity=PER_TENSOR, scaling=CURRENT, state=None, scale_out=None, amax_out=None,
                 saturate=False, count_overflow=False):
        hp = _hp(x)
        flags = (SATURATE if saturate else 0) | (COUNT_OVERFLOW if count_overflow else 0)
        op = Operand(data=x.data_ptr(), quantized=0, format=fmt, granularity=granularity, hp=hp, scaling=scaling,
                     flags=flags, state=None if state is None else state.buf.data_ptr(),
                     scale_out=None if scale_out is None else scale_out.data_ptr(),
                     amax_out=None if amax_out is None else amax_out.data_ptr())
        return GemmOperand(op, (x, state, scale_out, amax_out))


_OPS = {"NT": 0, "NN": 1, "TN": 2}


def gemm_workspace_bytes(op, M, N, K, A, B):
    n = lib().fp8_gemm_workspace_bytes(_OPS[op], M, N, K, ctypes.byref(A.op), ctypes.byref(B.op))
    if n == ctypes.c_size_t(-1).value:
        _check(EINVAL)
    return n


def _gemm(op, M, N, K, A, B, out_dtype, out, ws):
    dev = A.keep[0].device
    c_dtype = _TORCH_HP[out_dtype]
    C = torch.empty((M, N), dtype=out_dtype, device=dev) if out is None else out
    need = gemm_workspace_bytes(op, M, N, K, A, B)
    if ws is None and need > 0:
        ws = _ws(need, dev)
    fn = {"NT": lib().fp8_gemm_scaled_NT, "NN": lib().fp8_gemm_scaled_NN, "TN": lib().fp8_gemm_scaled_TN}[op]
    _check(fn(M, N, K, ctypes.byref(A.op), ctypes.byref(B.op), _ptr(C), c_dtype, _ptr(ws),
              0 if ws is None else ws.numel(), _stream()))
    return C


def fp8_gemm_scaled_NT(M, N, K, A, B, out_dtype=torch.bfloat16, out=None, ws=None):
    """fprop: C[M,N] = A[M,K] . B[N,K]^T with scales (A, B: GemmOperand)."""
    return _gemm("NT", M, N, K, A, B, out_dtype, out, ws)


def fp8_gemm_scaled_NN(M, N, K, A, B, out_dtype=torch.bfloat16, out=None, ws=None):
    """dgrad: C[M,N] = A[M,K] . B[K,N] with scales."""
    return _gemm("NN", M, N, K, A, B, out_dtype, out, ws)


def fp8_gemm_scaled_TN(M, N, K, A, B, out_dtype=torch.bfloat16, out=None, ws=None):
    """wgrad: C[M,N] = A[K,M]^T . B[K,N] with scales."""
    return _gemm("TN", M, N, K, A, B, out_dtype, out, ws)


def as_fp8(codes, fmt):
    """View uint8 codes as torch's float8 dtype of the format (no copy)."""
    return codes.view(_FP8_DTYPE[fmt])
