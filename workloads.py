"""Seeded synthetic inputs for the FP8 scaling and scaled-GEMM workloads.

This module only draws random numbers and arranges them into tensors; it holds
none of the method's arithmetic (no amax, scale, cast or GEMM).  The same
bytes feed the CPU oracle and, after a copy, the GPU library.

Recipes (distributions follow the workloads described on the pages, the sizes
follow a transformer layer with hidden 4096, FFN 16384, M = 31 x 512 tokens):
  tiny layer     X[512,32], W1[64,32], W2[16,64] ~ N(0,1)/6 fp32, G[512,64] ~ N(0,1)
  quantize       bf16 [15872,4096] ~ N(0,9), 0.1% seeded entries x1e4, one row x1e4
  single GEMM    A bf16 [15872,4096], B bf16 [4096,4096] ~ N(0,1)/64;
                 delayed-scaling steps with a 40-sigma spike (0.625) on the last step
  layer GEMMs    12 fprop/dgrad/wgrad GEMMs, operands ~ N(0,1)/sqrt(K) bf16
  block-scaled   the same shapes, operands ~ N(0,1) bf16 with 1% rows x1e3
  lab MLP        the training-parity draws of the lab page (X[512,32], teacher
                 targets Y = tanh(X . W^T) in plain fp32, W1[64,32]/6, W2[16,64]/8)
Outliers and spikes are applied to the bf16-rounded tensor in fp32 and the
result is rounded to bf16 again.
"""
import math

import torch

M_TOKENS = 31 * 512
HIDDEN = 4096
FFN = 16384
QKV = 3 * HIDDEN

# (name, K_in, N_out) of the four linears of a transformer layer
LINEARS = (("qkv", HIDDEN, QKV), ("attn_out", HIDDEN, HIDDEN),
           ("mlp_up", HIDDEN, FFN), ("mlp_down", FFN, HIDDEN))


def _gen(seed, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, std, seed, dtype=torch.bfloat16, device="cpu"):
    """N(0, std^2) drawn in fp32 with a seeded generator, then cast to dtype."""
    x = torch.randn(shape, generator=_gen(seed, device), dtype=torch.float32, device=device)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def scale_random_rows(x, frac, factor, seed):
    """Multiply a seeded set of round(frac * rows) distinct rows by factor (bf16 re-rounded)."""
    rows = x.shape[0]
    n = max(1, int(round(frac * rows)))
    idx = torch.randperm(rows, generator=_gen(seed))[:n].to(x.device)
    xf = x.float()
    xf[idx] *= factor
    return xf.to(x.dtype), idx.cpu()


# ------------------------------------------------------------------ tiny layer
def tiny_layer(seed=1000):
    """fp32 X[512,32], W1[64,32], W2[16,64] ~ N(0,1)/6 and G[512,64] ~ N(0,1)."""
    X = normal((512, 32), 1.0 / 6, seed + 0, torch.float32)
    W1 = normal((64, 32), 1.0 / 6, seed + 1, torch.float32)
    W2 = normal((16, 64), 1.0 / 6, seed + 2, torch.float32)
    G = normal((512, 64), 1.0, seed + 3, torch.float32)
    return X, W1, W2, G


# ------------------------------------------------------------------ quantize
def quantize_tensor(rows=M_TOKENS, cols=HIDDEN, seed=2000, device="cpu"):
    """bf16 [rows, cols] ~ N(0,9); ~0.1% seeded distinct entries x1e4; one seeded row x1e4."""
    x = normal((rows, cols), 3.0, seed, torch.bfloat16, device)
    n = rows * cols
    k = max(1, n // 1000)
    g = _gen(seed + 1)
    cand = torch.unique(torch.randint(0, n, (k + k // 50 + 16,), generator=g))
    idx = cand[torch.randperm(cand.numel(), generator=g)[:k]].to(x.device)
    row = int(torch.randint(0, rows, (1,), generator=g))
    xf = x.float().view(-1)
    xf[idx] *= 1e4
    xf = xf.view(rows, cols)
    xf[row] *= 1e4
    return xf.to(torch.bfloat16)


# ------------------------------------------------------------------ single GEMM
def attn_out_operands(M=M_TOKENS, K=HIDDEN, N=HIDDEN, seed=3100, device="cpu"):
    """A bf16 [M,K], B bf16 [N,K] (a weight stored [N,K]) ~ N(0,1)/64."""
    A = normal((M, K), 1.0 / 64, seed, torch.bfloat16, device)
    B = normal((N, K), 1.0 / 64, seed + 1, torch.bfloat16, device)
    return A, B


def delayed_steps(M=M_TOKENS, K=HIDDEN, steps=17, seed=3000, spike_seed=3999, device="cpu"):
    """Activations for `steps` delayed-scaling steps (seeds seed..seed+steps-1),
    ~ N(0,1)/64 each; the last one carries one seeded element set to 40 sigma (0.625).
    Yields (step, tensor, spike_index or None)."""
    for t in range(steps):
        x = normal((M, K), 1.0 / 64, seed + t, torch.bfloat16, device)
        spike = None
        if t == steps - 1:
            g = _gen(spike_seed)
            r = int(torch.randint(0, M, (1,), generator=g))
            c = int(torch.randint(0, K, (1,), generator=g))
            x[r, c] = 40.0 / 64
            spike = (r, c)
        yield t, x, spike


# ------------------------------------------------------------------ layer GEMMs
def layer_gemms(M=M_TOKENS):
    """The 12 GEMMs of a layer as (name, op, M, N, K): fprop NT, dgrad NN, wgrad TN."""
    out = []
    for name, k_in, n_out in LINEARS:
        out.append((f"{name}.fprop", "NT", M, n_out, k_in))
        out.append((f"{name}.dgrad", "NN", M, k_in, n_out))
        out.append((f"{name}.wgrad", "TN", n_out, k_in, M))
    return out


def gemm_operands(op, M, N, K, seed, std=None, device="cpu", outlier_rows=0.0, outlier=1e3):
    """bf16 operands in the storage layout of op, ~ N(0,1)/sqrt(K) unless std is given.

    NT: A [M,K], B [N,K];  NN: A [M,K], B [K,N];  TN: A [K,M], B [K,N].
    outlier_rows > 0 multiplies that fraction of the stored rows of each operand by outlier.
    """
    s = 1.0 / math.sqrt(K) if std is None else std
    shape_a = {"NT": (M, K), "NN": (M, K), "TN": (K, M)}[op]
    shape_b = {"NT": (N, K), "NN": (K, N), "TN": (K, N)}[op]
    A = normal(shape_a, s, seed, torch.bfloat16, device)
    B = normal(shape_b, s, seed + 1, torch.bfloat16, device)
    if outlier_rows > 0:
        A, _ = scale_random_rows(A, outlier_rows, outlier, seed + 2)
        B, _ = scale_random_rows(B, outlier_rows, outlier, seed + 3)
    return A, B


# ------------------------------------------------------------------ helpers
def bf16_bits(x):
    """bf16 torch tensor -> numpy uint16 array of its bit patterns (CPU copy)."""
    return x.detach().to("cpu").contiguous().view(torch.int16).numpy().view("uint16")


# ------------------------------------------------------------------ lab smoke checks
def lab_smoke_inputs():
    """The random draws of the fp8_parity.py page's smoke() checks [1]-[4], in its
    order under torch.manual_seed(0): x = randn(4096)*3; 16 history tensors
    randn(1024); act = randn(1024) with act[3] = 40; a = randn(8,128)*0.01 with
    row 0 multiplied by 1e4.  fp32 CPU tensors."""
    torch.manual_seed(0)
    x = torch.randn(4096) * 3.0
    big = torch.tensor([1000.0, -600.0, 500.0])
    history = [torch.randn(1024) for _ in range(16)]
    act = torch.randn(1024)
    act[3] = 40.0
    a = torch.randn(8, 128) * 0.01
    a[0] *= 1e4
    return {"x": x, "big": big, "history": history, "act": act, "a": a}


def lab_mlp_inputs():
    """The draws of the same page's check [5] (small-MLP training): after the
    draws of checks [1]-[4], X = randn(512, 32) and a teacher weight
    randn(16, 32) / 6 giving targets Y = tanh(X . W^T); then, under
    torch.manual_seed(1), the initial weights W1 = randn(64, 32) / 6 and
    W2 = randn(16, 64) / 8.  fp32 CPU tensors."""
    lab_smoke_inputs()
    X = torch.randn(512, 32)
    Y = torch.tanh(X @ (torch.randn(16, 32) / 6).T)
    torch.manual_seed(1)
    W1 = torch.randn(64, 32) / 6
    W2 = torch.randn(16, 64) / 8
    return {"X": X, "Y": Y, "W1": W1, "W2": W2}
