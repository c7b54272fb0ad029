"""The reading behind the router's products on the bf16 matrix cores: a
float32 value splits exactly into three bf16 terms, and a bf16 activation
times each term is exact in float32, so a float32-accumulated sum over the
three terms is a float32 product of the exact operands. CPU only; torch's
bfloat16 cast rounds to nearest even, like the device's conversion."""
import numpy as np
import pytest
import torch


def split3(v):
    """hi = bf16(v), mid = bf16(v - hi), lo = bf16(v - hi - mid), every
    difference taken in float32 (as on the device)."""
    v = torch.as_tensor(v, dtype=torch.float32)
    hi = v.to(torch.bfloat16).float()
    r1 = v - hi
    mid = r1.to(torch.bfloat16).float()
    r2 = r1 - mid
    lo = r2.to(torch.bfloat16).float()
    return hi, mid, lo, r1, r2


def _values(n, seed):
    rng = np.random.default_rng(seed)
    # many binades, both signs, plus router-like weights and logit gradients
    v = np.concatenate([
        rng.standard_normal(n) * np.exp2(rng.integers(-60, 60, n)),
        rng.normal(0.0, 0.02, n),
        rng.standard_normal(n) * 1e-4,
    ]).astype(np.float32)
    # values on and next to bf16 rounding ties: 8 significant bits plus a half
    # step, and the float32 neighbours of such ties
    base = (rng.integers(128, 256, n) * 2 + 1).astype(np.float64) * np.exp2(rng.integers(-40, 40, n) - 9)
    ties = base.astype(np.float32)
    up = np.nextafter(ties, np.float32(np.inf))
    dn = np.nextafter(ties, np.float32(-np.inf))
    return np.concatenate([v, ties, up, dn, -ties]).astype(np.float32)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_three_bf16_terms_sum_exactly(seed):
    v = _values(20000, seed)
    hi, mid, lo, r1, r2 = split3(v)
    # the two remainders are exact in float32 and lo holds the last one exactly
    assert torch.equal(lo, r2)
    exact = hi.double() + mid.double() + lo.double()
    assert torch.equal(exact, torch.as_tensor(v, dtype=torch.float64))
    # each term is a bf16 value and the terms shrink by at least 2^8 each
    for t in (hi, mid, lo):
        assert torch.equal(t.to(torch.bfloat16).float(), t)
    nz = mid != 0
    assert (mid[nz].abs() <= hi[nz].abs() * 2.0 ** -8).all()
    nz = lo != 0
    assert (lo[nz].abs() <= mid[nz].abs() * 2.0 ** -8).all()


def test_bf16_products_are_exact_in_float32():
    rng = np.random.default_rng(7)
    x = torch.as_tensor(rng.standard_normal(50000), dtype=torch.float32).to(torch.bfloat16).float()
    w = torch.as_tensor(_values(10000, 3)[:50000], dtype=torch.float32)
    hi, mid, lo, _, _ = split3(w)
    for t in (hi, mid, lo):
        p64 = x.double() * t.double()
        assert torch.equal((x * t).double(), p64)       # no rounding in float32
    # and the three products add up to x * w exactly (in float64)
    assert torch.equal(x.double() * hi.double() + x.double() * mid.double() + x.double() * lo.double(),
                       x.double() * w.double())


def test_a_plain_bf16_operand_would_not_do():
    """The split is needed: rounding the float32 operand to one bf16 term
    loses about 2^-9 of it, far above the router's 1e-5 parity bound."""
    w = torch.as_tensor(np.random.default_rng(4).normal(0, 0.02, 10000), dtype=torch.float32)
    hi = w.to(torch.bfloat16).float()
    rel = ((w - hi).abs() / w.abs()).max().item()
    assert rel > 1e-3
