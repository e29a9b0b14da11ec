"""Oracle pins for simulated-FP8 training ("fp8_parity.py" lab page, class
FP8Matmul and smoke check [5])."""
import pytest
import torch

import workloads
from oracle import fp8_train

E4M3_MAX, E5M2_MAX = 448.0, 57344.0


def _fake_quant(x, dtype, fmax):
    # the page's scaled_roundtrip written with torch's own float8 casts (an
    # independent library routine): s = max(amax / fmax, 1e-12), x / s cast and back
    s = (x.abs().max() / fmax).clamp_min(1e-12)
    return (x / s).to(dtype).float() * s


def test_one_step_matches_fake_quant_formulas():
    """Forward y = xq . wq^T, backward dx = gq . wq and dw = gq^T . xq, with xq,
    wq E4M3 and gq E5M2 -- a transposed operand or a dropped term in the
    oracle's backward fails here."""
    d = workloads.lab_mlp_inputs()
    x = torch.relu(d["X"] @ d["W1"].T).requires_grad_()
    w = d["W2"].clone().requires_grad_()
    y = fp8_train.OracleFP8Matmul.apply(x, w)
    g = torch.randn(y.shape, generator=torch.Generator().manual_seed(5)) * 1e-3
    y.backward(g)
    xq = _fake_quant(x.detach(), torch.float8_e4m3fn, E4M3_MAX)
    wq = _fake_quant(w.detach(), torch.float8_e4m3fn, E4M3_MAX)
    gq = _fake_quant(g, torch.float8_e5m2, E5M2_MAX)
    for got, ref in ((y.detach(), xq.double() @ wq.double().T), (x.grad, gq.double() @ wq.double()),
                     (w.grad, gq.double().T @ xq.double())):
        assert got.shape == ref.shape
        err = (got.double() - ref).abs().max().item()
        assert err <= 1e-6 * ref.abs().max().item(), (err, ref.abs().max().item())


@pytest.fixture(scope="module")
def losses():
    d = workloads.lab_mlp_inputs()
    l32 = fp8_train.train_mlp(d["X"], d["Y"], d["W1"], d["W2"], fp8=False)
    l8 = fp8_train.train_mlp(d["X"], d["Y"], d["W1"], d["W2"], fp8=True)
    return l32, l8


def test_lab_check5_final_loss_gap(losses):
    """Check [5]: after 300 AdamW steps (lr 3e-3) the simulated-FP8 final loss is
    within 10% of the fp32 one."""
    l32, l8 = losses
    assert len(l32) == len(l8) == 300
    assert abs(l8[-1] - l32[-1]) / l32[-1] < 0.10
    # both runs actually train (the loss falls by well over half)
    assert l32[-1] < 0.5 * l32[0] and l8[-1] < 0.5 * l8[0]


def test_first_step_loss_is_quantized_but_close(losses):
    """Step 0 sees the same weights: the FP8 loss differs from the fp32 one only
    by the quantization of X, W1, relu(X W1^T) and W2 (a few percent at most),
    and is not bitwise equal (the quantized path really ran)."""
    l32, l8 = losses
    assert l8[0] != l32[0]
    assert abs(l8[0] - l32[0]) / l32[0] < 0.05


def _fake_quant_rows(x, dtype, fmax, dim):
    # per-row (dim=1: max over each row) or per-column (dim=0) scaled round trip
    # with torch's float8 casts
    s = (x.abs().amax(dim=dim, keepdim=True) / fmax).clamp_min(1e-12)
    return (x / s).to(dtype).float() * s


def test_rowwise_one_step_matches_fake_quant_formulas():
    """The rowwise recipe: y = xq . wq^T with x and w scaled per row; dx = gq . wq'
    with dy per row and w per column; dw = gq'^T . xq' with dy and x per column."""
    d = workloads.lab_mlp_inputs()
    x = torch.relu(d["X"] @ d["W1"].T).requires_grad_()
    w = d["W2"].clone().requires_grad_()
    y = fp8_train.OracleFP8MatmulRowwise.apply(x, w)
    g = torch.randn(y.shape, generator=torch.Generator().manual_seed(5)) * 1e-3
    y.backward(g)
    e4, e5 = torch.float8_e4m3fn, torch.float8_e5m2
    xd, wd = x.detach(), w.detach()
    y_ref = _fake_quant_rows(xd, e4, E4M3_MAX, 1).double() @ _fake_quant_rows(wd, e4, E4M3_MAX, 1).double().T
    dx_ref = _fake_quant_rows(g, e5, E5M2_MAX, 1).double() @ _fake_quant_rows(wd, e4, E4M3_MAX, 0).double()
    dw_ref = _fake_quant_rows(g, e5, E5M2_MAX, 0).double().T @ _fake_quant_rows(xd, e4, E4M3_MAX, 0).double()
    for got, ref in ((y.detach(), y_ref), (x.grad, dx_ref), (w.grad, dw_ref)):
        assert got.shape == ref.shape
        err = (got.double() - ref).abs().max().item()
        assert err <= 1e-6 * ref.abs().max().item(), (err, ref.abs().max().item())


def test_rowwise_lab_check5_final_loss_gap():
    """Check [5]'s bound applied to the rowwise recipe."""
    d = workloads.lab_mlp_inputs()
    l32 = fp8_train.train_mlp(d["X"], d["Y"], d["W1"], d["W2"], fp8=False)
    lr = fp8_train.train_mlp(d["X"], d["Y"], d["W1"], d["W2"], fp8=True, recipe="rowwise")
    assert abs(lr[-1] - l32[-1]) / l32[-1] < 0.10
    assert lr[-1] < 0.5 * lr[0]


def test_rowwise_gw_hp_one_step():
    """The rowwise_with_gw_hp recipe: y and dx exactly as in the rowwise
    recipe, and dw equal to torch's own fp32 autograd gradient of x . w^T
    (the wgrad GEMM is not quantized)."""
    d = workloads.lab_mlp_inputs()
    x = torch.relu(d["X"] @ d["W1"].T)
    g = torch.randn(512, 16, generator=torch.Generator().manual_seed(5)) * 1e-3
    xr, wr = x.clone().requires_grad_(), d["W2"].clone().requires_grad_()
    yr = fp8_train.OracleFP8MatmulRowwise.apply(xr, wr)
    yr.backward(g)
    xh, wh = x.clone().requires_grad_(), d["W2"].clone().requires_grad_()
    yh = fp8_train.OracleFP8MatmulRowwise.apply(xh, wh, True)
    yh.backward(g)
    assert torch.equal(yh, yr) and torch.equal(xh.grad, xr.grad)
    xt, wt = x.clone().requires_grad_(), d["W2"].clone().requires_grad_()
    (xt @ wt.T).backward(g)
    err = (wh.grad.double() - wt.grad.double()).abs().max().item()
    assert err <= 1e-6 * wt.grad.abs().max().item(), err
    assert not torch.equal(wh.grad, wr.grad)   # the quantized wgrad differs


def test_rowwise_gw_hp_lab_check5_final_loss_gap():
    """Check [5]'s bound applied to the rowwise_with_gw_hp recipe."""
    d = workloads.lab_mlp_inputs()
    l32 = fp8_train.train_mlp(d["X"], d["Y"], d["W1"], d["W2"], fp8=False)
    lh = fp8_train.train_mlp(d["X"], d["Y"], d["W1"], d["W2"], fp8=True, recipe="rowwise_with_gw_hp")
    assert abs(lh[-1] - l32[-1]) / l32[-1] < 0.10
    assert lh[-1] < 0.5 * lh[0]


def test_sr_gradients_lab_check5_final_loss_gap():
    """Check [5]'s bound with stochastically rounded E5M2 gradients."""
    d = workloads.lab_mlp_inputs()
    l32 = fp8_train.train_mlp(d["X"], d["Y"], d["W1"], d["W2"], fp8=False)
    ls = fp8_train.train_mlp(d["X"], d["Y"], d["W1"], d["W2"], fp8=True, grad_sr_seed=1234)
    assert abs(ls[-1] - l32[-1]) / l32[-1] < 0.10
    assert ls[-1] < 0.5 * ls[0]


def test_rht_wgrad_lab_check5_final_loss_gap():
    """Check [5]'s bound with Hadamard-transformed wgrad operands."""
    d = workloads.lab_mlp_inputs()
    l32 = fp8_train.train_mlp(d["X"], d["Y"], d["W1"], d["W2"], fp8=False)
    lh = fp8_train.train_mlp(d["X"], d["Y"], d["W1"], d["W2"], fp8=True, wgrad_rht_seed=500)
    assert abs(lh[-1] - l32[-1]) / l32[-1] < 0.10
    assert lh[-1] < 0.5 * lh[0]
