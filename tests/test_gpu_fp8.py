"""FP8 (E4M3) quantization through the C-ABI against the oracle: codes and
scale exponents are integer results, so the comparison is bit-exact."""
import numpy as np
import pytest
import torch

import oracle as O
from moe_inputs import bf16_bits_to_f32, to_bf16_bits

pytestmark = pytest.mark.gpu


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _rows(rows, K, seed):
    """bf16 bit patterns: Gaussian rows spread over 2^-40 .. 2^40, plus rows
    that sit on the scale's boundaries and special values."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((rows, K)).astype(np.float32)
    v *= np.exp2(rng.integers(-40, 40, rows)).astype(np.float32)[:, None]
    bits = to_bf16_bits(v)
    specials = [
        np.zeros(K, np.float32),                                   # all zero -> e = 0
        np.full(K, -0.0, np.float32),                              # negative zeros -> 0x80
        np.linspace(-448, 448, K).astype(np.float32),              # amax exactly 448 -> e = 0
        np.linspace(-1.75, 1.0, K).astype(np.float32) * 2.0 ** 20, # amax = 1.75 * 2^20
        np.linspace(-1.0, 1.7578125, K).astype(np.float32),        # amax just above 1.75
        np.linspace(-3e38, 3e38, K).astype(np.float32),            # near the top of the range
        rng.standard_normal(K).astype(np.float32) * 2.0 ** -60,    # tiny values
    ]
    for i, s in enumerate(specials[: max(rows - 1, 0)]):
        bits[i] = to_bf16_bits(s)
    if rows > len(specials):
        # bf16 subnormals (exponent field 0)
        sub = rng.integers(1, 128, K).astype(np.uint16) | (rng.integers(0, 2, K).astype(np.uint16) << 15)
        bits[len(specials)] = sub
    return bits


@pytest.mark.parametrize("rows,K", [(9, 16), (33, 4096), (12, 208), (5, 14336), (4, 16400)])
def test_quantize_rows_bit_exact(rows, K):
    import mixture_experts_layer_28_amd as moe
    print(f"[case] quantize rows={rows} K={K}", flush=True)
    bits = _rows(rows, K, seed=rows * 7 + K)
    x = _dev_bf16(bits)
    codes = torch.empty(rows, K, dtype=torch.uint8, device="cuda")
    sexp = torch.empty(rows, dtype=torch.int32, device="cuda")
    moe.quantize_fp8(x, codes, sexp)
    torch.cuda.synchronize()
    ref_c, ref_e = O.quantize_rows_fp8(bf16_bits_to_f32(bits).astype(np.float64))
    got_c, got_e = codes.cpu().numpy(), sexp.cpu().numpy()
    assert (got_e == ref_e).all(), (np.nonzero(got_e != ref_e)[0], got_e, ref_e)
    bad = np.argwhere(got_c != ref_c)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:5].tolist()}"


def test_quantize_respects_device_row_bound():
    """Rows at or beyond *valid_rows are not written."""
    import mixture_experts_layer_28_amd as moe
    rows, K = 9, 64
    bits = _rows(rows, K, seed=3)
    x = _dev_bf16(bits)
    codes = torch.full((rows, K), 0xAB, dtype=torch.uint8, device="cuda")
    sexp = torch.full((rows,), -12345, dtype=torch.int32, device="cuda")
    valid = torch.tensor([5], dtype=torch.int32, device="cuda")
    moe.quantize_fp8(x, codes, sexp, valid_rows=valid)
    torch.cuda.synchronize()
    ref_c, ref_e = O.quantize_rows_fp8(bf16_bits_to_f32(bits).astype(np.float64))
    got_c, got_e = codes.cpu().numpy(), sexp.cpu().numpy()
    assert (got_c[:5] == ref_c[:5]).all() and (got_e[:5] == ref_e[:5]).all()
    assert (got_c[5:] == 0xAB).all() and (got_e[5:] == -12345).all()


@pytest.mark.parametrize("G,R,C", [(1, 16, 8), (3, 64, 72), (2, 208, 136), (8, 96, 200),
                                   (1, 2048, 64), (2, 1040, 24)])
def test_quantize_transposed_bit_exact(G, R, C):
    """moe_quantize_fp8_t of [G, R, C] equals the oracle's per-row
    quantization of the G transposes: partial 64-row and 64-column tiles,
    the unrolled column-max loop and its tail, special columns."""
    import mixture_experts_layer_28_amd as moe
    print(f"[case] quantize transposed G={G} R={R} C={C}", flush=True)
    # rows of the transposes carry the special patterns, so they become columns
    bt = _rows(G * C, R, seed=G * 131 + R * 7 + C).reshape(G, C, R)
    x = _dev_bf16(np.ascontiguousarray(bt.transpose(0, 2, 1)))
    codes = torch.empty(G, C, R, dtype=torch.uint8, device="cuda")
    sexp = torch.empty(G, C, dtype=torch.int32, device="cuda")
    moe.quantize_fp8_t(x, codes, sexp)
    torch.cuda.synchronize()
    ref_c, ref_e = O.quantize_rows_fp8(bf16_bits_to_f32(bt.reshape(G * C, R)).astype(np.float64))
    got_c, got_e = codes.cpu().numpy().reshape(G * C, R), sexp.cpu().numpy().reshape(G * C)
    assert (got_e == ref_e).all(), np.nonzero(got_e != ref_e)[0][:10]
    bad = np.argwhere(got_c != ref_c)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:5].tolist()}"


@pytest.mark.parametrize("G,R,C", [(1, 16, 16), (2, 80, 48), (3, 208, 208), (2, 64, 4096),
                                   (1, 96, 6160), (1, 96, 14336), (1, 48, 20000)])
def test_quantize_both_bit_exact(G, R, C):
    """moe_quantize_fp8_both: the row codes equal the oracle's per-row
    quantization of each matrix, and the transposed codes its per-row
    quantization of the transposes (every rows-per-pass variant, partial
    64-row blocks, special rows and columns)."""
    import mixture_experts_layer_28_amd as moe
    print(f"[case] quantize both G={G} R={R} C={C}", flush=True)
    rows = _rows(G * R, C, seed=G * 17 + R * 3 + C).reshape(G, R, C)
    # special patterns in columns too: overwrite a few columns with a transposed block
    colsp = _rows(min(C, 7), R, seed=C + 1).T
    rows[0, :, : colsp.shape[1]] = colsp
    x = _dev_bf16(np.ascontiguousarray(rows))
    codes = torch.empty(G, R, C, dtype=torch.uint8, device="cuda")
    sexp = torch.empty(G, R, dtype=torch.int32, device="cuda")
    codes_t = torch.empty(G, C, R, dtype=torch.uint8, device="cuda")
    sexp_t = torch.empty(G, C, dtype=torch.int32, device="cuda")
    ws = torch.empty(moe.quantize_fp8_both_ws((G, R, C)), dtype=torch.uint8, device="cuda")
    moe.quantize_fp8_both(x, codes, sexp, codes_t, sexp_t, ws)
    torch.cuda.synchronize()
    f = bf16_bits_to_f32(rows).astype(np.float64)
    rc, re_ = O.quantize_rows_fp8(f.reshape(G * R, C))
    tc, te = O.quantize_rows_fp8(np.ascontiguousarray(f.transpose(0, 2, 1)).reshape(G * C, R))
    assert (sexp.cpu().numpy().reshape(-1) == re_).all()
    assert (codes.cpu().numpy().reshape(G * R, C) == rc).all()
    assert (sexp_t.cpu().numpy().reshape(-1) == te).all()
    bad = np.argwhere(codes_t.cpu().numpy().reshape(G * C, R) != tc)
    assert bad.size == 0, f"{len(bad)} transposed codes differ, first {bad[:5].tolist()}"
