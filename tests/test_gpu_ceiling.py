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
