"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import sys

import numpy as np
import torch

import workloads


def dev():
    return torch.device("cuda:0")


def announce(*what):
    """Name the case on stdout before a GPU step (visible if the run dies)."""
    print("[case]", *what, flush=True)


def host_input(x):
    """Oracle view of a CPU tensor: float32 array or bf16 bit patterns."""
    if x.dtype == torch.bfloat16:
        return workloads.bf16_bits(x)
    return x.detach().cpu().contiguous().numpy()


def codes_equal(got, ref, fmt):
    """Bit-exact code comparison; NaN codes of the format compare equal to each
    other (the sign of a NaN produced by arithmetic is not specified)."""
    got = np.asarray(got, np.uint8)
    ref = np.asarray(ref, np.uint8)
    if got.shape != ref.shape:
        return False
    nan_g = (got & 0x7F) == 0x7F if fmt == 0 else (got & 0x7F) > 0x7C
    nan_r = (ref & 0x7F) == 0x7F if fmt == 0 else (ref & 0x7F) > 0x7C
    same = (got == ref) | (nan_g & nan_r)
    if not same.all():
        idx = np.argwhere(~same)[:5]
        print("first code mismatches (index, gpu, oracle):",
              [(tuple(i), hex(got[tuple(i)]), hex(ref[tuple(i)])) for i in idx], file=sys.stderr)
    return bool(same.all())


def scales_equal(got, ref):
    got = np.asarray(got)
    ref = np.asarray(ref)
    if got.shape != ref.shape:
        return False
    both_nan = np.isnan(got) & np.isnan(ref) if got.dtype.kind == "f" else np.zeros(got.shape, bool)
    return bool(((got == ref) | both_nan).all())


def gemm_close(got, ref, out_dtype):
    """Normwise tolerance: max|got - ref| <= tol * max|ref| over finite entries
    (tol 1e-3 for fp32 output, 2^-7 for bf16), and identical NaN / Inf pattern."""
    got = got.detach().float().cpu().double().numpy() if torch.is_tensor(got) else np.asarray(got, np.float64)
    tol = 1e-3 if out_dtype == torch.float32 else 2.0 ** -7
    fin = np.isfinite(ref)
    if not np.array_equal(np.isnan(got), np.isnan(ref)):
        print("NaN pattern differs", file=sys.stderr)
        return False
    if not np.array_equal(np.isinf(got), np.isinf(ref)):
        print("Inf pattern differs", file=sys.stderr)
        return False
    if not fin.any():
        return True
    rmax = np.abs(ref[fin]).max()
    err = np.abs(got[fin] - ref[fin]).max()
    ok = err <= tol * rmax
    if not ok:
        print(f"gemm error {err:.4g} > {tol:.3g} * {rmax:.4g}", file=sys.stderr)
    return ok


def sample_rows(M, seed, tile=256, n_tiles=6, n_rand=12):
    """Deterministic sample of output rows: both ends, the first and last row of
    a few M tiles, and some random rows."""
    rng = np.random.default_rng(seed)
    nt = -(-M // tile)
    rows = {0, M - 1}
    for t in rng.choice(nt, size=min(n_tiles, nt), replace=False):
        rows.add(int(t) * tile)
        rows.add(min(M - 1, int(t) * tile + tile - 1))
    rows.update(int(r) for r in rng.integers(0, M, n_rand))
    return np.array(sorted(rows), dtype=np.int64)


def contract_rows(M, seed, tile=128, n_rand=256):
    """The full-size sample of output rows: the first and last row of every
    `tile`-row M tile, plus n_rand seeded random rows (all N columns are
    compared)."""
    rng = np.random.default_rng(seed)
    rows = set()
    for t0 in range(0, M, tile):
        rows.add(t0)
        rows.add(min(M, t0 + tile) - 1)
    rows.update(int(r) for r in rng.choice(M, size=min(n_rand, M), replace=False))
    return np.array(sorted(rows), dtype=np.int64)
