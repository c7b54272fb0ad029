"""Thin Python binding of libmoe (include/moe.h): the same entry points, with
torch tensors in place of raw device pointers. Argument marshalling only:
every step runs in the library's HIP kernels. PyTorch supplies device memory
and the current stream.

The library is required: importing works without it (so the package can be
inspected), but every call raises if libmoe.so is missing or was built for
another target. There is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libmoe.so")

ABI_VERSION = 7
MOE_F32, MOE_BF16 = 0, 1
MOE_SOFTMAX, MOE_SIGMOID = 0, 1
MOE_SWIGLU, MOE_GELU = 0, 1
MOE_FP8_E4M3, MOE_FP8_E5M2 = 0, 1
(MOE_OP_ROUTE, MOE_OP_AUX_STATS, MOE_OP_PERMUTE, MOE_OP_FFN_FWD, MOE_OP_FFN_BWD,
 MOE_OP_ROUTE_BWD, MOE_OP_FFN_FWD_FP8, MOE_OP_FFN_BWD_FP8, MOE_OP_FFN_FWD_FP8B,
 MOE_OP_FFN_BWD_FP8W, MOE_OP_FFN_BWD_FP8B, MOE_OP_FFN_BWD_FP8BW) = range(12)

# every symbol include/moe.h declares
EXPORTS = (
    "moe_route", "moe_aux_stats", "moe_bias_update", "moe_permute", "moe_grouped_ffn_fwd", "moe_combine",
    "moe_combine_bwd", "moe_grouped_ffn_bwd", "moe_route_bwd", "moe_permute_bwd",
    "moe_workspace_size", "moe_capacity", "moe_status_str", "moe_last_error", "moe_abi_version",
    "moe_profile_enable", "moe_profile_read", "moe_quantize_fp8", "moe_grouped_ffn_fwd_fp8",
    "moe_quantize_fp8_t", "moe_grouped_ffn_bwd_fp8", "moe_quantize_fp8_both",
    "moe_permute_noalloc", "moe_quantize_fp8_blocks", "moe_grouped_ffn_fwd_fp8b",
    "moe_grouped_ffn_bwd_fp8w", "moe_quantize_fp8_squares", "moe_grouped_ffn_bwd_fp8b",
    "moe_grouped_ffn_bwd_fp8bw",
)


class MoeDesc(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64), ("d", ctypes.c_int64), ("E", ctypes.c_int64),
        ("k", ctypes.c_int64), ("f", ctypes.c_int64), ("n_shared", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("score", ctypes.c_int32), ("act", ctypes.c_int32),
        ("gumbel_tau", ctypes.c_float), ("capacity", ctypes.c_int64),
        ("fp8_grad", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


class MoeError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: status {status} ({msg})")
        self.status = status


_lib = None
_P = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    """Load libmoe.so (once; MOE_LIBRARY names another build of it, such as
    the host-sanitized one). Raises if it is not built."""
    global _lib
    if _lib is None:
        path = os.environ.get("MOE_LIBRARY", LIB_PATH)
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m mixture_experts_layer_28_amd.build`")
        L = ctypes.CDLL(path)
        DP = ctypes.POINTER(MoeDesc)
        sig = {
            "moe_route": [DP] + [_P] * 10 + [ctypes.c_size_t, _P],
            "moe_aux_stats": [DP] + [_P] * 8 + [ctypes.c_size_t, _P],
            "moe_bias_update": [DP, _P, ctypes.c_float, _P, _P],
            "moe_permute": [DP] + [_P] * 8 + [ctypes.c_size_t, _P],
            "moe_permute_noalloc": [DP] + [_P] * 8,
            "moe_grouped_ffn_fwd": [DP] + [_P] * 14 + [ctypes.c_size_t, _P],
            "moe_quantize_fp8": [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _P, _P,
                                 ctypes.c_int64, _P, _P],
            "moe_grouped_ffn_fwd_fp8": [DP] + [_P] * 20 + [ctypes.c_size_t, _P],
            "moe_quantize_fp8_blocks": [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _P, _P,
                                        ctypes.c_int64, _P, _P],
            "moe_grouped_ffn_fwd_fp8b": [DP] + [_P] * 20 + [ctypes.c_size_t, _P],
            "moe_quantize_fp8_t": [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _P, _P, _P],
            "moe_quantize_fp8_both": [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _P, _P, _P, _P,
                                      _P, ctypes.c_size_t, _P],
            "moe_grouped_ffn_bwd_fp8": [DP] + [_P] * 24 + [ctypes.c_size_t, _P],
            "moe_grouped_ffn_bwd_fp8w": [DP] + [_P] * 24 + [ctypes.c_size_t, _P],
            "moe_quantize_fp8_squares": [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _P, _P, _P, _P,
                                         _P],
            "moe_grouped_ffn_bwd_fp8b": [DP] + [_P] * 24 + [ctypes.c_size_t, _P],
            "moe_grouped_ffn_bwd_fp8bw": [DP] + [_P] * 24 + [ctypes.c_size_t, _P],
            "moe_combine": [DP] + [_P] * 6,
            "moe_combine_bwd": [DP] + [_P] * 7,
            "moe_grouped_ffn_bwd": [DP] + [_P] * 20 + [ctypes.c_size_t, _P],
            "moe_route_bwd": [DP] + [_P] * 7 + [ctypes.c_float, _P, ctypes.c_float] + [_P] * 4
                             + [ctypes.c_size_t, _P],
            "moe_permute_bwd": [DP] + [_P] * 6,
            "moe_workspace_size": [DP, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)],
            "moe_capacity": [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                             ctypes.POINTER(ctypes.c_int64)],
            "moe_status_str": [ctypes.c_int],
            "moe_last_error": [],
            "moe_abi_version": [],
            "moe_profile_enable": [ctypes.c_int],
            "moe_profile_read": [ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                 ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                                 ctypes.POINTER(ctypes.c_int)],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_char_p if name in ("moe_status_str", "moe_last_error") else ctypes.c_int
        if L.moe_abi_version() != ABI_VERSION:
            raise RuntimeError("libmoe ABI version mismatch")
        _lib = L
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        raise MoeError(fn, status, lib().moe_last_error().decode())


def make_desc(T, d, E, k, f, n_shared=0, dtype="bf16", score="softmax", act="swiglu",
              capacity=None, gumbel_tau=0.0, fp8_grad="e4m3") -> MoeDesc:
    if fp8_grad not in ("e4m3", "e5m2"):
        raise ValueError(f"fp8_grad must be 'e4m3' or 'e5m2' (got {fp8_grad!r})")
    return MoeDesc(T=T, d=d, E=E, k=k, f=f, n_shared=n_shared,
                   fp8_grad=MOE_FP8_E5M2 if fp8_grad == "e5m2" else MOE_FP8_E4M3,
                   dtype=MOE_BF16 if dtype == "bf16" else MOE_F32,
                   score=MOE_SOFTMAX if score == "softmax" else MOE_SIGMOID,
                   act=MOE_SWIGLU if act == "swiglu" else MOE_GELU,
                   gumbel_tau=float(gumbel_tau or 0.0),
                   capacity=-1 if capacity is None else int(capacity))


def capacity(T: int, k: int, E: int, cf: Optional[float]) -> Optional[int]:
    """Per-expert capacity ceil(cf*T*k/E) as the library computes it (None = no limit)."""
    if cf is None:
        return None
    out = ctypes.c_int64()
    _check("moe_capacity", lib().moe_capacity(T, k, E, float(cf), ctypes.byref(out)))
    return int(out.value)


def workspace_size(desc: MoeDesc, op: int) -> int:
    out = ctypes.c_size_t()
    _check("moe_workspace_size", lib().moe_workspace_size(ctypes.byref(desc), op, ctypes.byref(out)))
    return int(out.value)


def profile_enable(on: bool = True):
    """Start (or stop) recording per-kernel timing events; drops unread records."""
    _check("moe_profile_enable", lib().moe_profile_enable(1 if on else 0))


def profile_read() -> list:
    """[(kernel name, total ms, launches)] since profile_enable(True); clears them."""
    cap = 64
    n = ctypes.c_int()
    names = (ctypes.c_char_p * cap)()
    ms = (ctypes.c_double * cap)()
    cnt = (ctypes.c_int * cap)()
    _check("moe_profile_read", lib().moe_profile_read(cap, ctypes.byref(n), names, ms, cnt))
    return [(names[i].decode(), float(ms[i]), int(cnt[i])) for i in range(min(n.value, cap))]


def _p(t):
    """Device pointer of a tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to libmoe must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    if t.numel() == 0:   # torch reports 0 for empty views; hand over their storage
        return t.untyped_storage().data_ptr() or None
    return t.data_ptr()


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ws(ws):
    if ws is None:
        return None, 0
    return ws.data_ptr(), ws.numel() * ws.element_size()


# ------------------------------------------------------------- entry points
def route(desc, x, w_r, logit_bias, sel_bias, topk_idx, gate, scores, lse=None, ws=None,
          stream=None, gumbel_u=None):
    wp, wn = _ws(ws)
    _check("moe_route", lib().moe_route(ctypes.byref(desc), _p(x), _p(w_r), _p(logit_bias),
                                        _p(sel_bias), _p(gumbel_u), _p(topk_idx), _p(gate),
                                        _p(scores), _p(lse), wp, wn, _stream(stream)))


def aux_stats(desc, scores, topk_idx, lse, counts, y, z, out3, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check("moe_aux_stats", lib().moe_aux_stats(ctypes.byref(desc), _p(scores), _p(topk_idx),
                                                _p(lse), _p(counts), _p(y), _p(z), _p(out3), wp,
                                                wn, _stream(stream)))


def bias_update(desc, counts, gamma, bias, stream=None):
    _check("moe_bias_update", lib().moe_bias_update(ctypes.byref(desc), _p(counts), float(gamma),
                                                    _p(bias), _stream(stream)))


def permute(desc, x, topk_idx, offsets, row_of, token_of, n_dropped, x_perm, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check("moe_permute", lib().moe_permute(ctypes.byref(desc), _p(x), _p(topk_idx), _p(offsets),
                                            _p(row_of), _p(token_of), _p(n_dropped), _p(x_perm),
                                            wp, wn, _stream(stream)))


def permute_noalloc(desc, x, topk_idx, offsets, row_of, token_of, n_dropped, x_perm, stream=None):
    """moe_permute without a workspace (the library's own device scratch)."""
    _check("moe_permute_noalloc", lib().moe_permute_noalloc(
        ctypes.byref(desc), _p(x), _p(topk_idx), _p(offsets), _p(row_of), _p(token_of),
        _p(n_dropped), _p(x_perm), _stream(stream)))


def grouped_ffn_fwd(desc, x_perm, offsets, x, w13, w2, sw13, sw2, save_pre, save_h, save_pre_s,
                    save_h_s, out, out_shared, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check("moe_grouped_ffn_fwd", lib().moe_grouped_ffn_fwd(
        ctypes.byref(desc), _p(x_perm), _p(offsets), _p(x), _p(w13), _p(w2), _p(sw13), _p(sw2),
        _p(save_pre), _p(save_h), _p(save_pre_s), _p(save_h_s), _p(out), _p(out_shared), wp, wn,
        _stream(stream)))


def quantize_fp8(src, codes, scale_exp, valid_rows=None, stream=None):
    """Per-row E4M3 quantization of a bf16 tensor [..., K] into codes (uint8,
    same shape) and scale exponents (int32, shape [...]); valid_rows: optional
    one-element int32 device tensor bounding the rows quantized."""
    K = src.shape[-1]
    rows = src.numel() // K if K else 0
    if codes.shape != src.shape or scale_exp.numel() != rows:
        raise ValueError("codes must match src's shape and scale_exp hold one entry per row")
    _check("moe_quantize_fp8", lib().moe_quantize_fp8(_p(src), rows, K, K, _p(valid_rows),
                                                      _p(codes), K, _p(scale_exp),
                                                      _stream(stream)))


def grouped_ffn_fwd_fp8(desc, xq_perm, sx_perm, offsets, xq, sx, w13q, s13, w2q, s2, sw13q, ss13,
                        sw2q, ss2, save_pre, save_h, save_pre_s, save_h_s, out, out_shared,
                        ws=None, stream=None):
    wp, wn = _ws(ws)
    _check("moe_grouped_ffn_fwd_fp8", lib().moe_grouped_ffn_fwd_fp8(
        ctypes.byref(desc), _p(xq_perm), _p(sx_perm), _p(offsets), _p(xq), _p(sx), _p(w13q),
        _p(s13), _p(w2q), _p(s2), _p(sw13q), _p(ss13), _p(sw2q), _p(ss2), _p(save_pre),
        _p(save_h), _p(save_pre_s), _p(save_h_s), _p(out), _p(out_shared), wp, wn,
        _stream(stream)))


def fp8_block_scale_bytes(rows: int, K: int) -> int:
    """Bytes of the block scales of a rows x K matrix: one byte per 32
    elements, four to a 32-bit word per 128, words 32-row interleaved (word w
    of row r at word (r // 32 * ceil(K / 128) + w) * 32 + r % 32)."""
    return 128 * ((K + 127) // 128) * ((rows + 31) // 32)


def quantize_fp8_blocks(src, codes, scales, valid_rows=None, stream=None):
    """Block-scaled E4M3 quantization of a bf16 tensor [..., K] (its rows)
    into codes (uint8, same shape) and e8m0 scale bytes (a uint8 tensor of
    fp8_block_scale_bytes(rows, K) elements, interleaved as described there)."""
    K = src.shape[-1]
    rows = src.numel() // K if K else 0
    if codes.shape != src.shape or scales.numel() != fp8_block_scale_bytes(rows, K):
        raise ValueError("codes must match src's shape and scales hold fp8_block_scale_bytes(rows, K)")
    _check("moe_quantize_fp8_blocks", lib().moe_quantize_fp8_blocks(
        _p(src), rows, K, K, _p(valid_rows), _p(codes), K, _p(scales), _stream(stream)))


def grouped_ffn_fwd_fp8b(desc, xq_perm, bx_perm, offsets, xq, bx, w13q, b13, w2q, b2, sw13q, sb13,
                         sw2q, sb2, save_pre, save_h, save_pre_s, save_h_s, out, out_shared,
                         ws=None, stream=None):
    wp, wn = _ws(ws)
    _check("moe_grouped_ffn_fwd_fp8b", lib().moe_grouped_ffn_fwd_fp8b(
        ctypes.byref(desc), _p(xq_perm), _p(bx_perm), _p(offsets), _p(xq), _p(bx), _p(w13q),
        _p(b13), _p(w2q), _p(b2), _p(sw13q), _p(sb13), _p(sw2q), _p(sb2), _p(save_pre),
        _p(save_h), _p(save_pre_s), _p(save_h_s), _p(out), _p(out_shared), wp, wn,
        _stream(stream)))


def quantize_fp8_t(src, codes, scale_exp, stream=None):
    """Per-column E4M3 quantization of bf16 matrices src [..., R, C] into the
    codes of their transposes ([..., C, R], uint8) and one exponent per
    column ([..., C], int32)."""
    R, C = src.shape[-2], src.shape[-1]
    G = src.numel() // (R * C) if R * C else 0
    if codes.shape != src.shape[:-2] + (C, R) or scale_exp.shape != src.shape[:-2] + (C,):
        raise ValueError("codes must be [..., C, R] and scale_exp [..., C] for src [..., R, C]")
    _check("moe_quantize_fp8_t", lib().moe_quantize_fp8_t(_p(src), G, R, C, _p(codes),
                                                          _p(scale_exp), _stream(stream)))


def quantize_fp8_both_ws(src_shape) -> int:
    """Workspace bytes of quantize_fp8_both for a bf16 tensor of shape [..., R, C]."""
    R, C = src_shape[-2], src_shape[-1]
    G = 1
    for n in src_shape[:-2]:
        G *= n
    return (G * ((R + 63) // 64) * C * 2 + 255) // 256 * 256


def quantize_fp8_both(src, codes, scale_exp, codes_t, scale_exp_t, ws, stream=None):
    """Rows and columns of bf16 matrices src [..., R, C] in one call (two reads
    of src): codes [..., R, C] with scale_exp [..., R], and the transposes'
    codes_t [..., C, R] with scale_exp_t [..., C]; ws: quantize_fp8_both_ws bytes."""
    R, C = src.shape[-2], src.shape[-1]
    G = src.numel() // (R * C) if R * C else 0
    lead = src.shape[:-2]
    if codes.shape != src.shape or scale_exp.shape != lead + (R,) or \
            codes_t.shape != lead + (C, R) or scale_exp_t.shape != lead + (C,):
        raise ValueError("codes [..., R, C], scale_exp [..., R], codes_t [..., C, R], scale_exp_t [..., C]")
    wp, wn = _ws(ws)
    _check("moe_quantize_fp8_both", lib().moe_quantize_fp8_both(
        _p(src), G, R, C, _p(codes), _p(scale_exp), _p(codes_t), _p(scale_exp_t), wp, wn,
        _stream(stream)))


def quantize_fp8_squares(src, codes, scales, codes_t, scales_t, stream=None):
    """Square-block E4M3 quantization of bf16 matrices src [..., R, C] (32 x
    32 squares, one exponent each) into both layouts from one read: codes
    [..., R, C] with scales (fp8_block_scale_bytes(G*R, C) uint8) and the
    transposes' codes_t [..., C, R] with scales_t (fp8_block_scale_bytes(G*C, R)),
    G the number of matrices. Either pair may be None (that layout is skipped)."""
    R, C = src.shape[-2], src.shape[-1]
    G = src.numel() // (R * C) if R * C else 0
    lead = src.shape[:-2]
    if (codes is None) != (scales is None) or (codes_t is None) != (scales_t is None):
        raise ValueError("codes and scales (and codes_t and scales_t) are given together")
    if codes is not None and (codes.shape != src.shape or
                              scales.numel() != fp8_block_scale_bytes(G * R, C)):
        raise ValueError("codes [..., R, C] and scales of fp8_block_scale_bytes(G*R, C) bytes")
    if codes_t is not None and (codes_t.shape != lead + (C, R) or
                                scales_t.numel() != fp8_block_scale_bytes(G * C, R)):
        raise ValueError("codes_t [..., C, R] and scales_t of fp8_block_scale_bytes(G*C, R) bytes")
    _check("moe_quantize_fp8_squares", lib().moe_quantize_fp8_squares(
        _p(src), G, R, C, _p(codes), _p(scales), _p(codes_t), _p(scales_t), _stream(stream)))


def grouped_ffn_bwd_fp8(desc, x_perm, offsets, x, w13q_t, s13_t, w2q_t, s2_t, sw13q_t, ss13_t,
                        sw2q_t, ss2_t, save_pre, save_h, save_pre_s, save_h_s, dout, dy, dx_perm,
                        dx_shared, dw13, dw2, dsw13, dsw2, ws=None, stream=None, fp8_wgrad=False,
                        block=False):
    """The FP8 backward (data gradients on FP8 operands); fp8_wgrad runs the
    weight gradients on token-axis block-scaled FP8 operands as well
    (moe_grouped_ffn_bwd_fp8w, workspace MOE_OP_FFN_BWD_FP8W). block: the
    data gradients on block scales against square-block weights, s13_t ..
    ss2_t being their scale bytes (moe_grouped_ffn_bwd_fp8b / _fp8bw,
    workspace MOE_OP_FFN_BWD_FP8B / MOE_OP_FFN_BWD_FP8BW)."""
    wp, wn = _ws(ws)
    name = "moe_grouped_ffn_bwd_fp8" + ("b" if block else "") + ("w" if fp8_wgrad else "")
    _check(name, getattr(lib(), name)(
        ctypes.byref(desc), _p(x_perm), _p(offsets), _p(x), _p(w13q_t), _p(s13_t), _p(w2q_t),
        _p(s2_t), _p(sw13q_t), _p(ss13_t), _p(sw2q_t), _p(ss2_t), _p(save_pre), _p(save_h),
        _p(save_pre_s), _p(save_h_s), _p(dout), _p(dy), _p(dx_perm), _p(dx_shared), _p(dw13),
        _p(dw2), _p(dsw13), _p(dsw2), wp, wn, _stream(stream)))


def combine(desc, out, out_shared, gate, row_of, y, stream=None):
    _check("moe_combine", lib().moe_combine(ctypes.byref(desc), _p(out), _p(out_shared), _p(gate),
                                            _p(row_of), _p(y), _stream(stream)))


def combine_bwd(desc, dy, out, gate, row_of, dgate, dout, stream=None):
    _check("moe_combine_bwd", lib().moe_combine_bwd(ctypes.byref(desc), _p(dy), _p(out), _p(gate),
                                                    _p(row_of), _p(dgate), _p(dout),
                                                    _stream(stream)))


def grouped_ffn_bwd(desc, x_perm, offsets, x, w13, w2, sw13, sw2, save_pre, save_h, save_pre_s,
                    save_h_s, dout, dy, dx_perm, dx_shared, dw13, dw2, dsw13, dsw2, ws=None,
                    stream=None):
    wp, wn = _ws(ws)
    _check("moe_grouped_ffn_bwd", lib().moe_grouped_ffn_bwd(
        ctypes.byref(desc), _p(x_perm), _p(offsets), _p(x), _p(w13), _p(w2), _p(sw13), _p(sw2),
        _p(save_pre), _p(save_h), _p(save_pre_s), _p(save_h_s), _p(dout), _p(dy), _p(dx_perm),
        _p(dx_shared), _p(dw13), _p(dw2), _p(dsw13), _p(dsw2), wp, wn, _stream(stream)))


def route_bwd(desc, x, w_r, scores, topk_idx, gate, dgate, y, aux_coef, lse, z_coef, dlogits,
              dx_router, dw_r, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check("moe_route_bwd", lib().moe_route_bwd(
        ctypes.byref(desc), _p(x), _p(w_r), _p(scores), _p(topk_idx), _p(gate), _p(dgate), _p(y),
        float(aux_coef), _p(lse), float(z_coef), _p(dlogits), _p(dx_router), _p(dw_r), wp, wn,
        _stream(stream)))


def permute_bwd(desc, dx_perm, row_of, dx_shared, dx_router, dx, stream=None):
    _check("moe_permute_bwd", lib().moe_permute_bwd(ctypes.byref(desc), _p(dx_perm), _p(row_of),
                                                    _p(dx_shared), _p(dx_router), _p(dx),
                                                    _stream(stream)))


from .layer import MoELayer  # noqa: E402,F401
