"""Simulated-FP8 training on the library's kernels.

`FP8Matmul` is y = x . w^T with both GEMM inputs quantized to E4M3 in the
forward and the output gradient quantized to E5M2 in the backward, each with
its per-tensor current scale.  Products accumulate in fp32; the optimizer
holds and updates fp32 weights, and only each call's GEMM inputs are 8-bit.
What is computed follows the "fp8_parity.py" lab page: class FP8Matmul and
the small-MLP training run of its smoke check [5].

How the library is used:

- The forward quantizes x and w with their transposed copies.
- It saves the codes, so the backward reuses the forward's E4M3 operands, as
  the page saves `xq` and `wq`.
- fprop is the NT GEMM, dgrad = E5M2(dy) . E4M3(w) is the NN GEMM, and
  wgrad = E5M2(dy)^T . E4M3(x) is the TN GEMM.

Every quantize and GEMM runs in libfp8q's HIP kernels.  The MLP's relu, tanh
targets, loss and AdamW are plain torch ops around them.
"""
import torch

from . import (E4M3, E5M2, ROWWISE, GemmOperand, fp8_gemm_scaled_NN, fp8_gemm_scaled_NT, fp8_gemm_scaled_TN,
               fp8_quantize_per_tensor, fp8_quantize_per_tensor_rht, fp8_quantize_per_tensor_sr,
               fp8_quantize_rowwise)


class FP8Matmul(torch.autograd.Function):
    """y[M,N] = x[M,K] . w[N,K]^T in FP8 (E4M3 forward, E5M2 output gradient).

    x and w are fp32 or bf16 (the same dtype); y, dx and dw come out in that
    dtype (fp32 accumulation, one rounding at the end).  With sr = (seed,
    offset) the output gradient is rounded stochastically
    (fp8_quantize_per_tensor_sr) instead of to nearest.  With rht = seed the
    wgrad GEMM takes dy and x through the random Hadamard transform along the
    tokens (fp8_quantize_per_tensor_rht, one seed for both), which leaves
    dy^T x unchanged and spreads outlier tokens before quantization."""

    @staticmethod
    def forward(ctx, x, w, sr=None, rht=None):
        if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[1]:
            raise ValueError(f"FP8Matmul needs x[M,K] and w[N,K], got {tuple(x.shape)} and {tuple(w.shape)}")
        if x.dtype != w.dtype or x.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError(f"FP8Matmul needs x and w both fp32 or both bf16, got {x.dtype} and {w.dtype}")
        x, w = x.contiguous(), w.contiguous()
        M, K = x.shape
        N = w.shape[0]
        # K-major copies only for the backward GEMMs that will run: x's for
        # wgrad, w's for dgrad (none in forward-only use)
        qx, qxT, sx, _ = fp8_quantize_per_tensor(x, E4M3, emit_t=ctx.needs_input_grad[1] and rht is None)
        qw, qwT, sw, _ = fp8_quantize_per_tensor(w, E4M3, emit_t=ctx.needs_input_grad[0])
        y = fp8_gemm_scaled_NT(M, N, K, GemmOperand.quantized(qx, E4M3, sx),
                               GemmOperand.quantized(qw, E4M3, sw), x.dtype)
        ctx.save_for_backward(qx, qxT, sx, qw, qwT, sw, x if rht is not None and ctx.needs_input_grad[1] else None)
        ctx.dtype, ctx.sr, ctx.rht = x.dtype, sr, rht
        return y

    @staticmethod
    def backward(ctx, dy):
        qx, qxT, sx, qw, qwT, sw, x_hp = ctx.saved_tensors
        dy = dy.to(ctx.dtype).contiguous()
        M, N = dy.shape
        K = qx.shape[1]
        if ctx.sr is None:
            qg, qgT, sg, _ = fp8_quantize_per_tensor(dy, E5M2, emit_t=True)
        else:
            qg, qgT, sg, _ = fp8_quantize_per_tensor_sr(dy, E5M2, ctx.sr[0], ctx.sr[1], emit_t=True)
        dx = dw = None
        if ctx.needs_input_grad[0]:
            dx = fp8_gemm_scaled_NN(M, K, N, GemmOperand.quantized(qg, E5M2, sg),
                                    GemmOperand.quantized(qw, E4M3, sw, kmajor=qwT), ctx.dtype)
        if ctx.needs_input_grad[1] and ctx.rht is not None:
            hg, hgT, shg, _ = fp8_quantize_per_tensor_rht(dy, E5M2, ctx.rht, emit_t=True)
            hx, hxT, shx, _ = fp8_quantize_per_tensor_rht(x_hp, E4M3, ctx.rht, emit_t=True)
            dw = fp8_gemm_scaled_TN(N, K, M, GemmOperand.quantized(hg, E5M2, shg, kmajor=hgT),
                                    GemmOperand.quantized(hx, E4M3, shx, kmajor=hxT), ctx.dtype)
        elif ctx.needs_input_grad[1]:
            dw = fp8_gemm_scaled_TN(N, K, M, GemmOperand.quantized(qg, E5M2, sg, kmajor=qgT),
                                    GemmOperand.quantized(qx, E4M3, sx, kmajor=qxT), ctx.dtype)
        return dx, dw, None, None


class FP8MatmulRowwise(torch.autograd.Function):
    """FP8Matmul with the lab page's "rowwise" recipe: every GEMM input scaled
    per row along that GEMM's contraction, so each of x, w and dy is cast once
    per GEMM it feeds:

    - fprop NT: x and w per row;
    - dgrad NN: dy per row, w per column (its K-major copy);
    - wgrad TN: dy and x per column (K-major copies).

    Each product is sum_k qa qb * sA[m] * sB[n].  With gw_hp (the page's
    "rowwise_with_gw_hp" recipe) the wgrad GEMM is not quantized: dw = dy^T x
    in the inputs' own precision (torch's matmul), fprop and dgrad as above."""

    @staticmethod
    def forward(ctx, x, w, gw_hp=False):
        if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[1]:
            raise ValueError(f"FP8MatmulRowwise needs x[M,K] and w[N,K], got {tuple(x.shape)} and {tuple(w.shape)}")
        if x.dtype != w.dtype or x.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError(f"FP8MatmulRowwise needs x and w both fp32 or both bf16, got {x.dtype} and {w.dtype}")
        x, w = x.contiguous(), w.contiguous()
        M, K = x.shape
        N = w.shape[0]
        qx, _, sx = fp8_quantize_rowwise(x, 0, E4M3)
        qw, _, sw = fp8_quantize_rowwise(w, 0, E4M3)
        y = fp8_gemm_scaled_NT(M, N, K, GemmOperand.quantized(qx, E4M3, sx, ROWWISE),
                               GemmOperand.quantized(qw, E4M3, sw, ROWWISE), x.dtype)
        saved = []
        if ctx.needs_input_grad[1] and gw_hp:   # wgrad in high precision: x itself
            saved += [x]
        elif ctx.needs_input_grad[1]:    # wgrad: x per column (over tokens)
            qx1, qx1T, sx1 = fp8_quantize_rowwise(x, 1, E4M3, emit_t=True)
            saved += [qx1, qx1T, sx1]
        if ctx.needs_input_grad[0]:    # dgrad: w per column (over output features)
            qw1, qw1T, sw1 = fp8_quantize_rowwise(w, 1, E4M3, emit_t=True)
            saved += [qw1, qw1T, sw1]
        ctx.save_for_backward(*saved)
        ctx.dtype, ctx.shape, ctx.gw_hp = x.dtype, (M, N, K), gw_hp
        return y

    @staticmethod
    def backward(ctx, dy):
        M, N, K = ctx.shape
        saved = list(ctx.saved_tensors)
        dy = dy.to(ctx.dtype).contiguous()
        dx = dw = None
        if ctx.needs_input_grad[1] and ctx.gw_hp:
            x = saved[0]
            saved = saved[1:]
            dw = dy.t().contiguous() @ x
        elif ctx.needs_input_grad[1]:
            qx1, qx1T, sx1 = saved[:3]
            saved = saved[3:]
            qg1, qg1T, sg1 = fp8_quantize_rowwise(dy, 1, E5M2, emit_t=True)
            dw = fp8_gemm_scaled_TN(N, K, M, GemmOperand.quantized(qg1, E5M2, sg1, ROWWISE, kmajor=qg1T),
                                    GemmOperand.quantized(qx1, E4M3, sx1, ROWWISE, kmajor=qx1T), ctx.dtype)
        if ctx.needs_input_grad[0]:
            qw1, qw1T, sw1 = saved[:3]
            qg0, _, sg0 = fp8_quantize_rowwise(dy, 0, E5M2)
            dx = fp8_gemm_scaled_NN(M, K, N, GemmOperand.quantized(qg0, E5M2, sg0, ROWWISE),
                                    GemmOperand.quantized(qw1, E4M3, sw1, ROWWISE, kmajor=qw1T), ctx.dtype)
        return dx, dw, None


def fp8_matmul(x, w, recipe="tensorwise", sr=None, rht=None):
    """x . w^T through FP8Matmul ("tensorwise", optionally with stochastically
    rounded gradients, sr = (seed, offset), and a Hadamard-transformed wgrad,
    rht = seed) or FP8MatmulRowwise ("rowwise", or "rowwise_with_gw_hp" with
    the wgrad GEMM in high precision)."""
    if recipe in ("rowwise", "rowwise_with_gw_hp"):
        if sr is not None or rht is not None:
            raise ValueError("stochastic rounding and the Hadamard transform are implemented for the tensorwise recipe")
        return FP8MatmulRowwise.apply(x, w, recipe == "rowwise_with_gw_hp")
    if recipe != "tensorwise":
        raise ValueError(f"unknown recipe {recipe!r}")
    return FP8Matmul.apply(x, w, sr, rht)


def stack_forward(weights, x, matmul):
    """x through a stack of bias-free linears, relu between consecutive ones:
    h_0 = x, h_{j+1} = matmul(act(h_j), W_j, j) with act = relu for j > 0."""
    h = x
    for j, w in enumerate(weights):
        h = matmul(torch.relu(h) if j else h, w, j)
    return h


def train_mlp(X, Y, W1, W2, fp8=True, steps=300, lr=3e-3, recipe="tensorwise", grad_sr_seed=None,
              wgrad_rht_seed=None):
    """Training run of the lab page's smoke check [5]: the two-linear stack
    [W1, W2] is fitted to Y by mean squared error under AdamW(lr), each matmul
    FP8 (`fp8_matmul` with `recipe`; grad_sr_seed: output gradients rounded
    stochastically at stream offset 2 t + j for step t, linear j;
    wgrad_rht_seed: Hadamard-transformed wgrad operands with seed
    wgrad_rht_seed + 2 t + j) or plain fp32.  X, Y, W1, W2 are device tensors;
    the weights are copied, the inputs left unchanged.  Returns the per-step
    losses (floats, read back once at the end)."""
    weights = [w.detach().clone().requires_grad_() for w in (W1, W2)]
    opt = torch.optim.AdamW(weights, lr=lr)

    def matmul_at(t):
        if not fp8:
            return lambda a, b, j: a @ b.T
        return lambda a, b, j: fp8_matmul(a, b, recipe, None if grad_sr_seed is None else (grad_sr_seed, 2 * t + j),
                                          None if wgrad_rht_seed is None else wgrad_rht_seed + 2 * t + j)

    def step(t):
        opt.zero_grad(set_to_none=True)
        loss = torch.nn.functional.mse_loss(stack_forward(weights, X, matmul_at(t)), Y)
        loss.backward()
        opt.step()
        return loss.detach()

    return [float(v) for v in torch.stack([step(t) for t in range(steps)]).cpu()]
