"""Calibration of the FP8 accumulation model of test_fp8_tolerance.py.

That CPU emulation adds, per 64-k matrix-core instruction, a normal error of
std ACC_SIGMA times the instruction's sum|products|. Here an FP8 GEMM on the
device's matrix cores (torch's scaled matrix product, K = 64: one 64-k
reduction per output) runs on random E4M3 operands, and its error against the
exact float64 product, relative to sum|products|, must stay inside what that
normal covers: median <= 0.674 sigma and 99th percentile <= 2.576 sigma.
"""
import numpy as np
import pytest
import torch

from test_fp8_tolerance import ACC_SIGMA

pytestmark = pytest.mark.gpu


def test_fp8_matrix_core_accumulation_within_the_emulated_model():
    if not hasattr(torch, "_scaled_mm"):
        pytest.skip("torch has no scaled matrix product")
    g = torch.Generator(device="cuda").manual_seed(0)
    M = N = 256
    K = 64
    a = (torch.randn(M, K, device="cuda", generator=g) * 3).to(torch.float8_e4m3fn)
    b = (torch.randn(N, K, device="cuda", generator=g) * 3).to(torch.float8_e4m3fn)
    one = torch.tensor(1.0, device="cuda")
    try:
        c = torch._scaled_mm(a, b.t(), scale_a=one, scale_b=one, out_dtype=torch.float32)
    except RuntimeError as e:
        pytest.skip(f"scaled matrix product unavailable: {e}")
    A = a.to(torch.float64).cpu().numpy()
    B = b.to(torch.float64).cpu().numpy()
    exact = A @ B.T
    rel = np.abs(c.double().cpu().numpy() - exact) / (np.abs(A) @ np.abs(B).T)
    med, p99 = float(np.median(rel)), float(np.percentile(rel, 99))
    print(f"FP8 accumulation error / sum|products|: median {med:.2e}, p99 {p99:.2e}, "
          f"max {rel.max():.2e} (model sigma {ACC_SIGMA:.0e})")
    assert med <= 0.674 * ACC_SIGMA, med
    assert p99 <= 2.576 * ACC_SIGMA, p99
