"""Simulated-FP8 training on the HIP path ("fp8_parity.py" lab page, class
FP8Matmul and smoke check [5]) against the oracle."""
import numpy as np
import pytest
import torch

import workloads
from oracle import fp8_train

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-3   # max |GPU - oracle| <= 1e-3 * max |oracle| for fp32 GEMM outputs


def _close(got, ref, what):
    got = got.detach().double().cpu()
    ref = ref.detach().double().cpu()
    assert got.shape == ref.shape, what
    err = (got - ref).abs().max().item()
    assert err <= TOL_F32 * ref.abs().max().item(), f"{what}: max |diff| {err} vs max |ref| {ref.abs().max().item()}"


@pytest.fixture(scope="module")
def training():
    from fp8_scaled_quantization_amax_amd import training
    return training


@pytest.fixture(scope="module")
def lab():
    return workloads.lab_mlp_inputs()


def test_fp8_matmul_one_step_matches_oracle(training, lab):
    """Forward output and both gradients of one FP8Matmul (the MLP's second
    layer at its initial weights) agree with the oracle's FP8Matmul."""
    dev = torch.device("cuda")
    h = torch.relu(lab["X"] @ lab["W1"].T)
    g = torch.randn(512, 16, generator=torch.Generator().manual_seed(5)) * 1e-3
    xo, wo = h.clone().requires_grad_(), lab["W2"].clone().requires_grad_()
    yo = fp8_train.OracleFP8Matmul.apply(xo, wo)
    yo.backward(g)
    xg, wg = h.to(dev).requires_grad_(), lab["W2"].to(dev).requires_grad_()
    yg = training.FP8Matmul.apply(xg, wg)
    yg.backward(g.to(dev))
    torch.cuda.synchronize()
    _close(yg, yo, "y")
    _close(xg.grad, xo.grad, "dx")
    _close(wg.grad, wo.grad, "dw")


def test_fp8_matmul_skips_unneeded_input_grad(training, lab):
    dev = torch.device("cuda")
    x = lab["X"].to(dev)
    w = lab["W1"].to(dev).requires_grad_()
    training.FP8Matmul.apply(x, w).sum().backward()
    assert w.grad is not None and x.grad is None
    assert torch.isfinite(w.grad).all()


def test_fp8_matmul_rejects_mismatched_shapes(training):
    dev = torch.device("cuda")
    with pytest.raises(ValueError):
        training.FP8Matmul.apply(torch.zeros(32, 16, device=dev), torch.zeros(16, 32, device=dev))


def test_lab_check5_training_parity(training, lab):
    """Check [5] on the GPU: 300 AdamW steps of the MLP with every matmul in FP8
    end within 10% of the fp32 run's final loss, and the loss curve follows
    the oracle's FP8 run."""
    dev = torch.device("cuda")
    X, Y, W1, W2 = (lab[k].to(dev) for k in ("X", "Y", "W1", "W2"))
    l8 = training.train_mlp(X, Y, W1, W2, fp8=True)
    l32 = training.train_mlp(X, Y, W1, W2, fp8=False)
    o8 = fp8_train.train_mlp(lab["X"], lab["Y"], lab["W1"], lab["W2"], fp8=True)
    gap = abs(l8[-1] - l32[-1]) / l32[-1]
    rel = np.abs(np.array(l8) - np.array(o8)) / np.array(o8)
    print(f"final loss fp32 {l32[-1]:.6f}, FP8 GPU {l8[-1]:.6f}, FP8 oracle {o8[-1]:.6f}; gap {100 * gap:.2f}%; "
          f"GPU vs oracle rel. deviation: step 0 {rel[0]:.2e}, steps <10 {rel[:10].max():.2e}, "
          f"<100 {rel[:100].max():.2e}, all {rel.max():.2e}", flush=True)
    assert gap < 0.10
    # Step 0 runs on identical weights.  The GPU's fp32 accumulation in layer 1
    # (within the GEMM tolerance of the exact product) can move relu(h)'s amax
    # by an ulp, or push an element across an FP8 rounding midpoint, so layer
    # 2's codes may differ in a few places.  The loss then agrees to the GEMM
    # tolerance, not bitwise.
    assert rel[0] <= TOL_F32
    # Later steps drift apart: AdamW's first updates are about lr * sign(grad),
    # and code flips compound.  So the curve gets a loose bound, not a parity
    # claim.  (Measured on MI355X: 1.7e-5 at step 0, 3e-4 over the first 10
    # steps, 1.1e-2 over all 300.)
    assert rel.max() < 0.05


def test_fp8_matmul_bf16_matches_oracle(training, lab):
    """bf16 activations and weights: the quantizer widens them exactly, so the
    codes are the oracle's on the fp32 copies; y, dx, dw come out in bf16 and
    agree within max |diff| <= 2^-7 max |oracle|."""
    dev = torch.device("cuda")
    h = torch.relu(lab["X"] @ lab["W1"].T).to(torch.bfloat16)
    w = lab["W2"].to(torch.bfloat16)
    g = (torch.randn(512, 16, generator=torch.Generator().manual_seed(6)) * 1e-3).to(torch.bfloat16)
    xo, wo = h.float().requires_grad_(), w.float().requires_grad_()
    yo = fp8_train.OracleFP8Matmul.apply(xo, wo)
    yo.backward(g.float())
    xg, wg = h.to(dev).requires_grad_(), w.to(dev).requires_grad_()
    yg = training.FP8Matmul.apply(xg, wg)
    yg.backward(g.to(dev))
    torch.cuda.synchronize()
    for got, ref, what in ((yg, yo, "y"), (xg.grad, xo.grad, "dx"), (wg.grad, wo.grad, "dw")):
        assert got.dtype == torch.bfloat16, what
        got, ref = got.detach().double().cpu(), ref.detach().double()
        err = (got - ref).abs().max().item()
        assert err <= 2.0 ** -7 * ref.abs().max().item(), f"{what}: {err}"


def test_fp8_matmul_rejects_mixed_dtypes(training):
    dev = torch.device("cuda")
    with pytest.raises(ValueError):
        training.FP8Matmul.apply(torch.zeros(32, 16, device=dev), torch.zeros(16, 16, device=dev, dtype=torch.bfloat16))


def test_rowwise_one_step_matches_oracle(training, lab):
    """The rowwise recipe's forward output and both gradients agree with the
    oracle's rowwise FP8 matmul (fp32 tolerance)."""
    dev = torch.device("cuda")
    h = torch.relu(lab["X"] @ lab["W1"].T)
    g = torch.randn(512, 16, generator=torch.Generator().manual_seed(7)) * 1e-3
    xo, wo = h.clone().requires_grad_(), lab["W2"].clone().requires_grad_()
    yo = fp8_train.OracleFP8MatmulRowwise.apply(xo, wo)
    yo.backward(g)
    xg, wg = h.to(dev).requires_grad_(), lab["W2"].to(dev).requires_grad_()
    yg = training.fp8_matmul(xg, wg, "rowwise")
    yg.backward(g.to(dev))
    torch.cuda.synchronize()
    _close(yg, yo, "y")
    _close(xg.grad, xo.grad, "dx")
    _close(wg.grad, wo.grad, "dw")


def test_rowwise_training_parity(training, lab):
    """Check [5]'s bound on the GPU with the rowwise recipe, and the loss curve
    against the oracle's rowwise run (step 0 to the GEMM tolerance, the curve
    within 5%, as for the tensorwise recipe)."""
    dev = torch.device("cuda")
    X, Y, W1, W2 = (lab[k].to(dev) for k in ("X", "Y", "W1", "W2"))
    l8 = training.train_mlp(X, Y, W1, W2, fp8=True, recipe="rowwise")
    l32 = training.train_mlp(X, Y, W1, W2, fp8=False)
    o8 = fp8_train.train_mlp(lab["X"], lab["Y"], lab["W1"], lab["W2"], fp8=True, recipe="rowwise")
    gap = abs(l8[-1] - l32[-1]) / l32[-1]
    rel = np.abs(np.array(l8) - np.array(o8)) / np.array(o8)
    print(f"rowwise: final loss fp32 {l32[-1]:.6f}, FP8 GPU {l8[-1]:.6f}, FP8 oracle {o8[-1]:.6f}; gap "
          f"{100 * gap:.2f}%; GPU vs oracle step 0 {rel[0]:.2e}, all {rel.max():.2e}", flush=True)
    assert gap < 0.10
    assert rel[0] <= TOL_F32
    assert rel.max() < 0.05


def test_rowwise_gw_hp_one_step_matches_oracle(training, lab):
    """The rowwise_with_gw_hp recipe (wgrad not quantized): forward output and
    both gradients agree with the oracle's (fp32 tolerance)."""
    dev = torch.device("cuda")
    h = torch.relu(lab["X"] @ lab["W1"].T)
    g = torch.randn(512, 16, generator=torch.Generator().manual_seed(8)) * 1e-3
    xo, wo = h.clone().requires_grad_(), lab["W2"].clone().requires_grad_()
    yo = fp8_train.OracleFP8MatmulRowwise.apply(xo, wo, True)
    yo.backward(g)
    xg, wg = h.to(dev).requires_grad_(), lab["W2"].to(dev).requires_grad_()
    yg = training.fp8_matmul(xg, wg, "rowwise_with_gw_hp")
    yg.backward(g.to(dev))
    torch.cuda.synchronize()
    _close(yg, yo, "y")
    _close(xg.grad, xo.grad, "dx")
    _close(wg.grad, wo.grad, "dw")


def test_rowwise_gw_hp_training_parity(training, lab):
    """Check [5]'s bound on the GPU with the rowwise_with_gw_hp recipe, and the
    loss curve against the oracle's run (step 0 to the GEMM tolerance, the
    curve within 5%)."""
    dev = torch.device("cuda")
    X, Y, W1, W2 = (lab[k].to(dev) for k in ("X", "Y", "W1", "W2"))
    l8 = training.train_mlp(X, Y, W1, W2, fp8=True, recipe="rowwise_with_gw_hp")
    l32 = training.train_mlp(X, Y, W1, W2, fp8=False)
    o8 = fp8_train.train_mlp(lab["X"], lab["Y"], lab["W1"], lab["W2"], fp8=True, recipe="rowwise_with_gw_hp")
    gap = abs(l8[-1] - l32[-1]) / l32[-1]
    rel = np.abs(np.array(l8) - np.array(o8)) / np.array(o8)
    print(f"rowwise_with_gw_hp: final loss fp32 {l32[-1]:.6f}, FP8 GPU {l8[-1]:.6f}, FP8 oracle {o8[-1]:.6f}; "
          f"gap {100 * gap:.2f}%; GPU vs oracle step 0 {rel[0]:.2e}, all {rel.max():.2e}", flush=True)
    assert gap < 0.10
    assert rel[0] <= TOL_F32
    assert rel.max() < 0.05


def test_sr_gradient_one_step_matches_oracle(training, lab):
    """Stochastically rounded output gradient (same seed and offset on both
    sides, so the same codes): forward output and both gradients agree with
    the oracle."""
    dev = torch.device("cuda")
    h = torch.relu(lab["X"] @ lab["W1"].T)
    g = torch.randn(512, 16, generator=torch.Generator().manual_seed(8)) * 1e-3
    xo, wo = h.clone().requires_grad_(), lab["W2"].clone().requires_grad_()
    yo = fp8_train.OracleFP8Matmul.apply(xo, wo, (99, 5))
    yo.backward(g)
    xg, wg = h.to(dev).requires_grad_(), lab["W2"].to(dev).requires_grad_()
    yg = training.fp8_matmul(xg, wg, sr=(99, 5))
    yg.backward(g.to(dev))
    torch.cuda.synchronize()
    _close(yg, yo, "y")
    _close(xg.grad, xo.grad, "dx")
    _close(wg.grad, wo.grad, "dw")


def test_sr_gradient_training_parity(training, lab):
    """Check [5]'s bound on the GPU with stochastically rounded gradients, and
    the loss curve against the oracle's run with the same seed."""
    dev = torch.device("cuda")
    X, Y, W1, W2 = (lab[k].to(dev) for k in ("X", "Y", "W1", "W2"))
    ls = training.train_mlp(X, Y, W1, W2, fp8=True, grad_sr_seed=1234)
    l32 = training.train_mlp(X, Y, W1, W2, fp8=False)
    os_ = fp8_train.train_mlp(lab["X"], lab["Y"], lab["W1"], lab["W2"], fp8=True, grad_sr_seed=1234)
    gap = abs(ls[-1] - l32[-1]) / l32[-1]
    rel = np.abs(np.array(ls) - np.array(os_)) / np.array(os_)
    print(f"SR gradients: final loss fp32 {l32[-1]:.6f}, FP8 GPU {ls[-1]:.6f}, FP8 oracle {os_[-1]:.6f}; gap "
          f"{100 * gap:.2f}%; GPU vs oracle step 0 {rel[0]:.2e}, all {rel.max():.2e}", flush=True)
    assert gap < 0.10
    assert rel[0] <= TOL_F32
    assert rel.max() < 0.05


def test_rht_wgrad_one_step_matches_oracle(training, lab):
    """Hadamard-transformed wgrad operands (same seed on both sides): forward
    output and both gradients agree with the oracle."""
    dev = torch.device("cuda")
    h = torch.relu(lab["X"] @ lab["W1"].T)
    g = torch.randn(512, 16, generator=torch.Generator().manual_seed(9)) * 1e-3
    xo, wo = h.clone().requires_grad_(), lab["W2"].clone().requires_grad_()
    yo = fp8_train.OracleFP8Matmul.apply(xo, wo, None, 321)
    yo.backward(g)
    xg, wg = h.to(dev).requires_grad_(), lab["W2"].to(dev).requires_grad_()
    yg = training.fp8_matmul(xg, wg, rht=321)
    yg.backward(g.to(dev))
    torch.cuda.synchronize()
    _close(yg, yo, "y")
    _close(xg.grad, xo.grad, "dx")
    _close(wg.grad, wo.grad, "dw")


def test_rht_wgrad_training_parity(training, lab):
    """Check [5]'s bound on the GPU with Hadamard-transformed wgrad operands,
    and the loss curve against the oracle's run with the same seeds."""
    dev = torch.device("cuda")
    X, Y, W1, W2 = (lab[k].to(dev) for k in ("X", "Y", "W1", "W2"))
    lh = training.train_mlp(X, Y, W1, W2, fp8=True, wgrad_rht_seed=500)
    l32 = training.train_mlp(X, Y, W1, W2, fp8=False)
    oh = fp8_train.train_mlp(lab["X"], lab["Y"], lab["W1"], lab["W2"], fp8=True, wgrad_rht_seed=500)
    gap = abs(lh[-1] - l32[-1]) / l32[-1]
    rel = np.abs(np.array(lh) - np.array(oh)) / np.array(oh)
    print(f"RHT wgrad: final loss fp32 {l32[-1]:.6f}, FP8 GPU {lh[-1]:.6f}, FP8 oracle {oh[-1]:.6f}; gap "
          f"{100 * gap:.2f}%; GPU vs oracle step 0 {rel[0]:.2e}, all {rel.max():.2e}", flush=True)
    assert gap < 0.10
    assert rel[0] <= TOL_F32
    assert rel.max() < 0.05
