"""The MFMA-loop measurement aid (the measured FP8 matrix-core ceiling that
bench.py reports beside the nominal peak): every MFMA of the loop ran, which
its exact output shows (E4M3 ones: each thread ends at 8 * 4 * 128 * iters)."""
import pytest
import torch

import fp8_scaled_quantization_amax_amd as fq
from gpu_util import announce, dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("blocks,iters", [(1, 1), (8, 37), (512, 4096)])
def test_mfma_loop_counts_every_mfma(blocks, iters):
    announce("mfma loop", blocks, iters)
    out = fq.fp8q_mfma_loop(blocks, iters, dev())
    torch.cuda.synchronize()
    assert out.numel() == blocks * 256
    assert torch.all(out == 4096.0 * iters)


def test_mfma_loop_random_operands_runs_and_repeats():
    """The random-operand loop: finite outputs, the same on a second run, and
    not the all-ones result (the operands really are the random codes)."""
    announce("mfma loop random")
    a = fq.fp8q_mfma_loop(64, 64, dev(), random_operands=True)
    b = fq.fp8q_mfma_loop(64, 64, dev(), random_operands=True)
    torch.cuda.synchronize()
    assert torch.isfinite(a).all() and torch.equal(a, b)
    assert not torch.all(a == 4096.0 * 64)
    assert a.unique().numel() > 1000
