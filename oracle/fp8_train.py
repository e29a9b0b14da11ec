"""Oracle side of simulated-FP8 training (the "fp8_parity.py" lab page, class
FP8Matmul and smoke check [5]).

TEST INFRASTRUCTURE ONLY, like the rest of oracle/.  `OracleFP8Matmul` is the
page's FP8Matmul written on the oracle's own definitions:

- each GEMM input is quantized with the oracle's per-tensor current scaling
  (E4M3 for x and w, E5M2 for the output gradient);
- the product is the oracle's exact integer GEMM, scaled in fp64 and then
  rounded once to fp32.

The page multiplies dequantized fp32 tensors (xq @ wq.T).  That is the same
product up to fp32 summation order.  `train_mlp` runs the check-[5] training
on the CPU.
"""
import numpy as np
import torch

from . import (E4M3, E5M2, Scale, gemm_nn, gemm_nt, gemm_tn, quantize_per_tensor, quantize_per_tensor_rht,
               quantize_per_tensor_sr, quantize_rowwise)


def _q(t, fmt):
    q, s, _ = quantize_per_tensor(t.detach().contiguous().numpy(), fmt)
    return q, Scale("tensor", s)


class OracleFP8Matmul(torch.autograd.Function):
    """y = x . w^T with E4M3 inputs forward and an E5M2 output gradient backward
    (rounded stochastically with sr = (seed, offset)); with rht = seed, the
    wgrad operands dy and x go through the random Hadamard transform first."""

    @staticmethod
    def forward(ctx, x, w, sr=None, rht=None):
        qx, sx = _q(x, E4M3)
        qw, sw = _q(w, E4M3)
        ctx.saved = (qx, sx, qw, sw, x.detach().clone())
        ctx.sr, ctx.rht = sr, rht
        return torch.from_numpy(gemm_nt(qx, qw, E4M3, E4M3, sx, sw).astype(np.float32))

    @staticmethod
    def backward(ctx, dy):
        qx, sx, qw, sw, x = ctx.saved
        if ctx.sr is None:
            qg, sg = _q(dy, E5M2)
        else:
            qg, s, _ = quantize_per_tensor_sr(dy.detach().contiguous().numpy(), E5M2, ctx.sr[0], ctx.sr[1])
            sg = Scale("tensor", s)
        dx = torch.from_numpy(gemm_nn(qg, qw, E5M2, E4M3, sg, sw).astype(np.float32))
        if ctx.rht is None:
            dw = torch.from_numpy(gemm_tn(qg, qx, E5M2, E4M3, sg, sx).astype(np.float32))
        else:
            hg, shg, _ = quantize_per_tensor_rht(dy.detach().contiguous().numpy(), E5M2, ctx.rht)
            hx, shx, _ = quantize_per_tensor_rht(x.contiguous().numpy(), E4M3, ctx.rht)
            dw = torch.from_numpy(gemm_tn(hg, hx, E5M2, E4M3, Scale("tensor", shg), Scale("tensor", shx))
                                  .astype(np.float32))
        return dx, dw, None, None


def _qr(t, fmt, axis, K):
    q, s = quantize_rowwise(t.detach().contiguous().numpy(), axis, fmt)
    return q, Scale.rowwise(s, K)


class OracleFP8MatmulRowwise(torch.autograd.Function):
    """The "rowwise" recipe: each GEMM input scaled per row along that GEMM's
    contraction (x, w per row for fprop; dy per row and w per column for
    dgrad; dy and x per column for wgrad).  gw_hp: the "rowwise_with_gw_hp"
    recipe, whose wgrad is not quantized: dw = dy^T x of the unquantized
    values, in fp64, rounded once to fp32."""

    @staticmethod
    def forward(ctx, x, w, gw_hp=False):
        M, K = x.shape
        N = w.shape[0]
        qx, sx = _qr(x, E4M3, 0, K)
        qw, sw = _qr(w, E4M3, 0, K)
        ctx.saved = (x.detach().clone(), w.detach().clone())
        ctx.gw_hp = gw_hp
        return torch.from_numpy(gemm_nt(qx, qw, E4M3, E4M3, sx, sw).astype(np.float32))

    @staticmethod
    def backward(ctx, dy):
        x, w = ctx.saved
        M, K = x.shape
        N = w.shape[0]
        qg0, sg0 = _qr(dy, E5M2, 0, N)
        qw1, sw1 = _qr(w, E4M3, 1, N)
        dx = torch.from_numpy(gemm_nn(qg0, qw1, E5M2, E4M3, sg0, sw1).astype(np.float32))
        if ctx.gw_hp:
            dw = torch.from_numpy((dy.detach().double().numpy().T @ x.double().numpy()).astype(np.float32))
        else:
            qg1, sg1 = _qr(dy, E5M2, 1, M)
            qx1, sx1 = _qr(x, E4M3, 1, M)
            dw = torch.from_numpy(gemm_tn(qg1, qx1, E5M2, E4M3, sg1, sx1).astype(np.float32))
        return dx, dw, None


def train_mlp(X, Y, W1, W2, fp8=True, steps=300, lr=3e-3, recipe="tensorwise", grad_sr_seed=None,
              wgrad_rht_seed=None):
    """The smoke-check [5] training run on the CPU: the stack [W1, W2] (relu
    between the two linears) fitted to Y by mean squared error under
    AdamW(lr), every matmul the oracle's FP8 matmul of `recipe` or plain
    fp32; returns the per-step losses."""
    weights = [w.detach().clone().requires_grad_() for w in (W1, W2)]
    opt = torch.optim.AdamW(weights, lr=lr)

    def fp8_mm(t):
        def mm(a, b, j):
            if recipe in ("rowwise", "rowwise_with_gw_hp"):
                return OracleFP8MatmulRowwise.apply(a, b, recipe == "rowwise_with_gw_hp")
            return OracleFP8Matmul.apply(a, b, None if grad_sr_seed is None else (grad_sr_seed, 2 * t + j),
                                         None if wgrad_rht_seed is None else wgrad_rht_seed + 2 * t + j)
        return mm

    losses = []
    for t in range(steps):
        mm = fp8_mm(t) if fp8 else (lambda a, b, j: a @ b.T)
        h = X
        for j, w in enumerate(weights):
            h = mm(torch.relu(h) if j else h, w, j)
        loss = torch.nn.functional.mse_loss(h, Y)
        opt.zero_grad(set_to_none=True)
        loss.backward()
        opt.step()
        losses.append(loss.item())
    return losses
