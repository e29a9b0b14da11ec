"""Host-only checks of the C ABI library: it loads, exports every function the
header declares, and rejects invalid arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

import fp8_scaled_quantization_amax_amd as fq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8q.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(fp8[A-Za-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("fp8_amax", "fp8_quantize_per_tensor", "fp8_quantize_tile1x128", "fp8_quantize_block128x128",
              "fp8_quantize_mx32", "fp8_quantize_rowwise", "fp8_quantize_per_tensor_sr",
              "fp8_quantize_per_tensor_rht", "fp8_gemm_scaled_NT", "fp8_gemm_scaled_NN", "fp8_gemm_scaled_TN",
              "fp8_gemm_workspace_bytes", "fp8q_status_string", "fp8q_last_error", "fp8q_abi_version",
              "fp8q_reduce_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(fq.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing


def test_version_and_status_strings():
    L = fq.lib()
    assert L.fp8q_abi_version() == 4
    assert L.fp8q_status_string(0) == b"ok"
    for s in range(1, 7):
        assert L.fp8q_status_string(s) not in (b"ok", b"unknown status")
    assert L.fp8q_status_string(99) == b"unknown status"
    assert L.fp8q_reduce_workspace_bytes() >= 4096


def _status(f, *args):
    return f(*args)


def test_invalid_arguments_are_rejected_before_any_gpu_call():
    L = fq.lib()
    P = ctypes.c_void_p
    fake = P(0x10000)            # never dereferenced: validation fails first
    ws = P(0x20000)
    # amax: null input, bad size, bad dtype, small workspace
    assert L.fp8_amax(None, fq.BF16, 10, fake, ws, 4096, None) == fq.EINVAL
    assert L.fp8_amax(fake, fq.BF16, 0, fake, ws, 4096, None) == fq.EINVAL
    assert L.fp8_amax(fake, 7, 10, fake, ws, 4096, None) == fq.EINVAL
    assert L.fp8_amax(fake, fq.BF16, 10, fake, ws, 16, None) == fq.EWORKSPACE
    assert b"workspace" in L.fp8q_last_error()
    # per-tensor: bad format, bad scaling, delayed without state, unknown flag
    args = (fake, fq.BF16, 4, 4)
    assert L.fp8_quantize_per_tensor(*args, 5, 0, None, fake, None, fake, None, 0, ws, 4096, None) == fq.EINVAL
    assert L.fp8_quantize_per_tensor(*args, 0, 9, None, fake, None, fake, None, 0, ws, 4096, None) == fq.EINVAL
    assert L.fp8_quantize_per_tensor(*args, 0, fq.DELAYED, None, fake, None, fake, None, 0, ws, 4096,
                                     None) == fq.EINVAL
    assert L.fp8_quantize_per_tensor(*args, 0, 0, None, fake, None, fake, None, 8, ws, 4096, None) == fq.EINVAL
    assert L.fp8_quantize_per_tensor(*args, 0, 0, None, fake, None, None, None, 0, ws, 4096, None) == fq.EINVAL
    # overflow count: only with delayed scaling, and only on the per-tensor cast
    assert L.fp8_quantize_per_tensor(*args, 0, fq.CURRENT, None, fake, None, fake, None, fq.COUNT_OVERFLOW, ws,
                                     4096, None) == fq.EINVAL
    assert b"COUNT_OVERFLOW" in L.fp8q_last_error()
    assert L.fp8_quantize_tile1x128(fake, fq.BF16, 4, 4, 0, 0, fake, None, fake, fq.COUNT_OVERFLOW,
                                    None) == fq.EINVAL
    assert L.fp8_quantize_per_tensor_sr(fake, fq.BF16, 4, 4, 1, 1, 0, fake, None, fake, None, fq.COUNT_OVERFLOW,
                                        ws, 4096, None) == fq.EINVAL
    # misaligned element pointer
    assert L.fp8_amax(P(0x10001), fq.BF16, 10, fake, ws, 4096, None) == fq.EALIGN
    # tiles: bad axis; mx: missing scales
    assert L.fp8_quantize_tile1x128(fake, fq.BF16, 4, 4, 2, 0, fake, None, fake, 0, None) == fq.EINVAL
    assert L.fp8_quantize_mx32(fake, fq.BF16, 4, 4, 0, 0, fake, None, None, 0, None) == fq.EINVAL
    assert L.fp8_quantize_block128x128(fake, fq.F32, -1, 4, 0, fake, None, fake, 0, None) == fq.EINVAL
    # stochastic rounding: missing scale_out, small workspace
    assert L.fp8_quantize_per_tensor_sr(fake, fq.BF16, 4, 4, 1, 1, 0, fake, None, None, None, 0, ws, 4096,
                                        None) == fq.EINVAL
    assert L.fp8_quantize_per_tensor_sr(fake, fq.BF16, 4, 4, 1, 1, 0, fake, None, fake, None, 0, ws, 16,
                                        None) == fq.EWORKSPACE
    # Hadamard: rows not a multiple of 16, cols not of 8, misaligned x
    assert L.fp8_quantize_per_tensor_rht(fake, fq.BF16, 24, 16, 0, 1, fake, None, fake, None, 0, ws, 4096,
                                         None) == fq.EALIGN
    assert L.fp8_quantize_per_tensor_rht(fake, fq.BF16, 32, 12, 0, 1, fake, None, fake, None, 0, ws, 4096,
                                         None) == fq.EALIGN
    assert L.fp8_quantize_per_tensor_rht(P(0x10008), fq.BF16, 32, 16, 0, 1, fake, None, fake, None, 0, ws, 4096,
                                         None) == fq.EALIGN
    # rowwise: bad axis, missing scales, a transposed copy with axis 0
    assert L.fp8_quantize_rowwise(fake, fq.BF16, 4, 4, 2, 0, fake, None, fake, 0, None) == fq.EINVAL
    assert L.fp8_quantize_rowwise(fake, fq.BF16, 4, 4, 0, 0, fake, None, None, 0, None) == fq.EINVAL
    assert L.fp8_quantize_rowwise(fake, fq.BF16, 4, 4, 0, 0, fake, fake, fake, 0, None) == fq.EUNSUPPORTED


def _op(**kw):
    base = dict(data=0x10000, scale=0x30000, quantized=1, format=fq.E4M3, granularity=fq.PER_TENSOR)
    base.update(kw)
    return fq.Operand(**base)


def test_gemm_validation():
    L = fq.lib()
    fake = ctypes.c_void_p(0x40000)
    A, B = _op(), _op()
    R = ctypes.byref
    # alignment rule: M, N, K multiples of 16
    assert L.fp8_gemm_scaled_NT(100, 64, 64, R(A), R(B), fake, fq.BF16, None, 0, None) == fq.EALIGN
    assert L.fp8_gemm_scaled_NT(64, 64, 40, R(A), R(B), fake, fq.BF16, None, 0, None) == fq.EALIGN
    # K multiple of 128 for tile / block scaling, of 32 for MX
    At = _op(granularity=fq.TILE_1x128)
    assert L.fp8_gemm_scaled_NT(64, 64, 144, R(At), R(B), fake, fq.BF16, None, 0, None) == fq.EALIGN
    Am, Bm = _op(granularity=fq.MX32), _op(granularity=fq.MX32)
    assert L.fp8_gemm_scaled_NT(64, 64, 48, R(Am), R(Bm), fake, fq.BF16, None, 0, None) == fq.EALIGN
    # MX on one side only is not implemented (and never silently substituted)
    assert L.fp8_gemm_scaled_NT(64, 64, 64, R(Am), R(B), fake, fq.BF16, None, 0, None) == fq.EUNSUPPORTED
    # rowwise combines with rowwise or per-tensor only, and needs pre-quantized codes
    Ar = _op(granularity=fq.ROWWISE)
    assert L.fp8_gemm_scaled_NT(64, 64, 128, R(Ar), R(At), fake, fq.BF16, None, 0, None) == fq.EUNSUPPORTED
    Ara = _op(quantized=0, hp=fq.BF16, granularity=fq.ROWWISE)
    assert L.fp8_gemm_scaled_NT(64, 64, 64, R(Ara), R(B), fake, fq.BF16, None, 0, None) == fq.EUNSUPPORTED
    assert L.fp8_gemm_workspace_bytes(0, 256, 256, 256, R(Ar), R(B)) == 0
    # delayed scaling is per-tensor only
    Ad = _op(quantized=0, hp=fq.BF16, scaling=fq.DELAYED, granularity=fq.TILE_1x128, state=0x50000)
    assert L.fp8_gemm_scaled_NT(64, 64, 128, R(Ad), R(B), fake, fq.BF16, None, 0, None) == fq.EUNSUPPORTED
    # an overflow count needs a delayed per-tensor autocast operand
    Ac = _op(quantized=0, hp=fq.BF16, scaling=fq.CURRENT, flags=fq.COUNT_OVERFLOW)
    assert L.fp8_gemm_scaled_NT(64, 64, 64, R(Ac), R(B), fake, fq.BF16, None, 0, None) == fq.EINVAL
    # misaligned codes
    Amis = _op(data=0x10008)
    assert L.fp8_gemm_scaled_NT(64, 64, 64, R(Amis), R(B), fake, fq.BF16, None, 0, None) == fq.EALIGN
    # missing C / bad output dtype / missing workspace for a transposed operand
    assert L.fp8_gemm_scaled_NT(64, 64, 64, R(A), R(B), None, fq.BF16, None, 0, None) == fq.EINVAL
    assert L.fp8_gemm_scaled_NT(64, 64, 64, R(A), R(B), fake, 5, None, 0, None) == fq.EINVAL
    assert L.fp8_gemm_scaled_NN(64, 64, 64, R(A), R(B), fake, fq.BF16, None, 0, None) == fq.EWORKSPACE


def test_gemm_workspace_sizes():
    L = fq.lib()
    R = ctypes.byref
    A, B = _op(), _op()
    assert L.fp8_gemm_workspace_bytes(0, 256, 256, 256, R(A), R(B)) == 0          # NT: both K-contiguous
    red = -(-L.fp8q_reduce_workspace_bytes() // 256) * 256                        # reduce region, first
    assert L.fp8_gemm_workspace_bytes(1, 256, 512, 128, R(A), R(B)) == red + 512 * 128  # NN: B transposed
    Bk = _op(data_kmajor=0x60000)
    assert L.fp8_gemm_workspace_bytes(1, 256, 512, 128, R(A), R(Bk)) == 0         # K-major copy given
    two = L.fp8_gemm_workspace_bytes(2, 256, 512, 128, R(A), R(B))
    assert two == red + 256 * 128 + 512 * 128                                     # TN: both transposed
    Aa = _op(quantized=0, hp=fq.BF16)
    ws = L.fp8_gemm_workspace_bytes(0, 256, 256, 256, R(Aa), R(B))
    assert ws >= 256 * 256 + L.fp8q_reduce_workspace_bytes()                      # autocast codes + partials
    assert L.fp8_gemm_workspace_bytes(3, 256, 256, 256, R(A), R(B)) == ctypes.c_size_t(-1).value
    assert L.fp8_gemm_workspace_bytes(0, 100, 256, 256, R(A), R(B)) == ctypes.c_size_t(-1).value


def test_mfma_loop_validation():
    L = fq.lib()
    fake = ctypes.c_void_p(0x10000)
    assert L.fp8q_mfma_loop(0, 16, fake, None) == fq.EINVAL
    assert L.fp8q_mfma_loop(4, 0, fake, None) == fq.EINVAL
    assert L.fp8q_mfma_loop(4, 16, None, None) == fq.EINVAL
    assert L.fp8q_mfma_loop_data(4, 16, 2, fake, None) == fq.EINVAL      # unknown data
    assert L.fp8q_mfma_loop_data(4, 12, 1, fake, None) == fq.EINVAL      # random needs iters % 8 == 0
    assert L.fp8q_mfma_loop_data(0, 16, 1, fake, None) == fq.EINVAL


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fq, "_lib", None)
    monkeypatch.setattr(fq, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        fq.lib()
