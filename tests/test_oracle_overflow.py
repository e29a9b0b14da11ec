"""Pins of the oracle's overflow count (what FP8Q_COUNT_OVERFLOW reports for a
delayed-scaling cast) to facts fixed outside it.

- torch's float8 casts (the very routines the lab page's numerics run on,
  non-saturating: E4M3 overflows to NaN, E5M2 to +-Inf) decide overflow
  element by element on the fp32 quotient x / s, which torch computes with
  IEEE division; the count must equal the number of finite x they overflow.
- Closed-form thresholds from the formats' definitions: E4M3's maximum 448
  has mantissa 110, the next step would be 480 (111), so the midpoint 464
  ties to 448 and only values above it overflow; E5M2's maximum 57344 has
  mantissa 11, the next step is 2^16 (10 00), so the midpoint 61440 ties to
  the even 2^16 and overflows.
- The lab page's smoke check [3] scenario: a delayed scale from a quiet
  history and a spike step overflows exactly the spike's large elements.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads

E4M3, E5M2 = 0, 1
TORCH_FP8 = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}


def torch_count(x, s, fmt):
    """Overflowing finite elements by torch's own cast of x / s."""
    xt = torch.as_tensor(np.asarray(x, np.float32))
    v = (xt / torch.tensor(np.float32(s))).to(TORCH_FP8[fmt]).to(torch.float32)
    bad = torch.isnan(v) if fmt == E4M3 else torch.isinf(v)
    return int((bad & torch.isfinite(xt)).sum())


@pytest.mark.parametrize("fmt,edge,first_over", [(E4M3, 464.0, np.nextafter(np.float32(464.0), np.float32(1e9))),
                                                (E5M2, np.nextafter(np.float32(61440.0), np.float32(0)), 61440.0)])
def test_thresholds(fmt, edge, first_over):
    assert orc.overflow_count(np.array([edge, -edge], np.float32), 1.0, fmt) == 0
    assert orc.overflow_count(np.array([first_over, -first_over], np.float32), 1.0, fmt) == 2
    assert torch_count(np.array([edge, first_over], np.float32), 1.0, fmt) == 1


def test_non_finite_inputs_are_not_counted():
    x = np.array([np.inf, -np.inf, np.nan, 1e30, -1e30, 1.0], np.float32)
    for fmt in (E4M3, E5M2):
        # 1e30 / 1 overflows the format (finite input); Inf and NaN inputs do not count
        assert orc.overflow_count(x, 1.0, fmt) == 2
        assert torch_count(x, 1.0, fmt) == 2


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_matches_torch_cast_on_random_data(fmt, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(20000) * rng.choice([1, 10, 100], 20000)).astype(np.float32)
    fmax = 448.0 if fmt == E4M3 else 57344.0
    for s in (np.float32(3.0 * 10 / fmax), np.float32(50.0 / fmax), np.float32(1.0)):
        assert orc.overflow_count(x, s, fmt) == torch_count(x, s, fmt)


def test_bf16_inputs():
    x = workloads.normal((64, 96), 30.0, 5, torch.bfloat16)
    bits = workloads.bf16_bits(x)
    s = np.float32(1.0 / 16)
    assert orc.overflow_count(bits, s, E4M3) == torch_count(x.float().numpy(), s, E4M3)


def test_delayed_spike_scenario():
    """Check [3]'s setting: the history saw quiet steps, then a step with a
    spike; its delayed scale overflows the spike's elements and nothing else."""
    quiet = workloads.normal((128, 64), 1.0, 11, torch.float32).numpy()
    hist = np.zeros(16, np.float32)
    hist[0] = np.abs(quiet).max()
    s = np.float32(np.float32(hist.max()) / np.float32(448.0))
    spike = quiet.copy()
    spike[5, 7] = 40.0 * hist[0]
    spike[9, 1] = -25.0 * hist[0]
    assert orc.overflow_count(spike, s, E4M3) == 2
    assert orc.overflow_count(quiet, s, E4M3) == 0
    assert orc.overflow_count(spike, s, E4M3) == torch_count(spike, s, E4M3)
