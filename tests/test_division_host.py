"""The quantizers divide by the scale with a reciprocal and two FMA residual
corrections instead of a full IEEE division.  This CPU test compiles that very
helper (csrc/device_common.h, div_by_scale, and div_by_own_scale where its
caller guarantees a finite estimate) as host code and checks it against
the correctly rounded fp32 quotient: every bf16 input against 2000 scales,
every fp32 input against one scale, and every bf16 input against an infinite
scale (x / Inf: +-0 for finite x, NaN otherwise)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_division_matches_correctly_rounded_quotient():
    out = os.path.join(ROOT, "_build", "div_exact")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    subprocess.run(["/opt/rocm/bin/hipcc", "-O2", "-fopenmp", "-std=c++17",
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "fp8_scaled_quantization_amax_amd", "csrc"),
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    os.path.join(ROOT, "tests", "host", "div_exact.hip"), "-o", out],
                   check=True, capture_output=True)
    r = subprocess.run([out, "2000", "1"], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "bf16 x 2000 scales: 0 relevant mismatches" in r.stdout
    assert "all fp32 x 1 scales: 0 relevant mismatches" in r.stdout
    assert "bf16 x infinite scale: 0 mismatches" in r.stdout
