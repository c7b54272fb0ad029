"""One MoE layer's forward and backward as an ordered sequence of libmoe
calls on one stream. Buffers come from torch (device memory only); the
routed-row buffers are sized for the worst case T*k rows, so no call ever
waits on the device to learn how many rows were kept.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (MOE_OP_AUX_STATS, MOE_OP_FFN_BWD, MOE_OP_FFN_BWD_FP8, MOE_OP_FFN_BWD_FP8B, MOE_OP_FFN_BWD_FP8BW,
               MOE_OP_FFN_BWD_FP8W, MOE_OP_FFN_FWD, MOE_OP_FFN_FWD_FP8, MOE_OP_FFN_FWD_FP8B, MOE_OP_PERMUTE,
               MOE_OP_ROUTE, MOE_OP_ROUTE_BWD, aux_stats, bias_update, combine, combine_bwd,
               fp8_block_scale_bytes, grouped_ffn_bwd, grouped_ffn_bwd_fp8, grouped_ffn_fwd,
               grouped_ffn_fwd_fp8, grouped_ffn_fwd_fp8b, make_desc, permute, permute_bwd, quantize_fp8,
               quantize_fp8_blocks, quantize_fp8_both, quantize_fp8_both_ws, quantize_fp8_squares,
               quantize_fp8_t, route, route_bwd, workspace_size)


class MoELayer:
    """Buffers and call order of one layer.

    Weights/inputs are passed at call time (the layer owns no parameters):
    x [T,d], w_r [E,d] fp32, w13 [E,2f|f,d], w2 [E,d,f], optional shared
    sw13/sw2, optional logit_bias/sel_bias [E] fp32, dy [T,d].

    aux_coef weights the load-balance loss and z_coef the router z-loss in
    the router gradient; bias_gamma > 0 makes step() apply the aux-loss-free
    bias update to sel_bias (in place) from this batch's expert loads;
    gumbel_tau > 0 turns on the noisy gate, whose uniforms [T, E] fp32 the
    caller passes to forward() (inp["gumbel_u"] for step()).

    fp8_fwd runs both forward GEMMs on per-row E4M3 operands: every forward
    quantizes x_perm (and x for a shared expert) and the current weights,
    keeps the pre-activations and H in bf16, and the backward runs in bf16
    as usual. fp8_bwd runs the backward's two data-gradient GEMMs on E4M3
    operands as well: the weights are quantized per input channel (into their
    transposes) - by the forward in the same pass as its row quantization
    when both are FP8, else by the backward - and the library quantizes the
    upstream and pre-activation gradients per row; the weight gradients stay
    bf16. The transposed codes a forward made serve the next backward on the
    same weight tensors (weights do not change between the two).

    fp8_scale picks the scaling: "row" (one power-of-two scale per operand
    row), "block" (forward only: one per 32 elements along K of each row, e8m0
    bytes, on the block-scaled matrix instructions; the backward's FP8 GEMMs
    keep per-row scales and quantize the weight transposes themselves), or
    "square" (weights in 32 x 32 squares, one quantization per weight serving
    the forward and the data gradients, written in both layouts from one
    read; activations and gradients in blocks of 32 along K, forward and data
    gradients on the block-scaled instructions).

    fp8_wgrad (with fp8_bwd) runs the weight gradients on FP8 operands too:
    the library quantizes dO, H, dpre and x_perm along the token axis (one
    scale per 32 of an expert's tokens per column) into their transposes.
    fp8_grad picks the FP8 format of the backward's gradient operands (dO,
    dpre): "e4m3" or "e5m2" (weights and activations stay E4M3).
    """

    def __init__(self, T, d, E, k, f, n_shared=0, dtype="bf16", score="softmax", act="swiglu",
                 capacity: Optional[int] = None, aux_coef: float = 0.0, z_coef: float = 0.0,
                 bias_gamma: float = 0.0, gumbel_tau: float = 0.0, fp8_fwd: bool = False,
                 fp8_bwd: bool = False, fp8_scale: str = "row", fp8_wgrad: bool = False,
                 fp8_grad: str = "e4m3", device="cuda"):
        self.desc = make_desc(T, d, E, k, f, n_shared, dtype, score, act, capacity, gumbel_tau,
                              fp8_grad)
        self.T, self.d, self.E, self.k, self.f = T, d, E, k, f
        self.n_shared, self.aux_coef, self.z_coef = n_shared, aux_coef, z_coef
        self.bias_gamma = bias_gamma
        self.fp8_fwd, self.fp8_bwd = fp8_fwd, fp8_bwd
        if (fp8_fwd or fp8_bwd) and dtype != "bf16":
            raise ValueError("the FP8 GEMMs keep bf16 activations: dtype must be bf16")
        if fp8_scale not in ("row", "block", "square"):
            raise ValueError(f"fp8_scale must be 'row', 'block' or 'square' (got {fp8_scale!r})")
        self.fp8_square = fp8_scale == "square" and (fp8_fwd or fp8_bwd)
        self.fp8_block = fp8_fwd and fp8_scale in ("block", "square")
        if fp8_wgrad and not fp8_bwd:
            raise ValueError("fp8_wgrad runs with the FP8 data gradients: set fp8_bwd too")
        self.fp8_wgrad = fp8_wgrad
        dt = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.dt = dt
        P = 2 * f if act == "swiglu" else f
        R = T * k
        dev = torch.device(device)
        i32, f32 = torch.int32, torch.float32

        def z(*shape, dtype=dt):
            # never hand out a NULL pointer: zero-row buffers are views of one row
            full = (max(shape[0], 1),) + tuple(shape[1:])
            return torch.empty(*full, dtype=dtype, device=dev)[: shape[0]]

        # forward
        self.topk_idx = z(T, k, dtype=i32)
        self.gate = z(T, k, dtype=f32)
        self.scores = z(T, E, dtype=f32)
        self.lse = z(T, dtype=f32)
        self.counts = z(E, dtype=i32)
        self.y_frac = z(E, dtype=f32)
        self.z_mean = z(E, dtype=f32)
        self.aux_out = z(3, dtype=f32)
        self.offsets = z(E + 1, dtype=i32)
        self.row_of = z(T, k, dtype=i32)
        self.token_of = z(max(R, 1), dtype=i32)
        self.n_dropped = z(1, dtype=i32)
        self.x_perm = z(R, d)
        self.save_pre = z(R, P)
        self.save_h = z(R, f)
        self.out = z(R, d)
        self.save_pre_s = z(T, P) if n_shared else None
        self.save_h_s = z(T, f) if n_shared else None
        self.out_shared = z(T, d) if n_shared else None
        self.Y = z(T, d)
        # backward
        self.dgate = z(T, k, dtype=f32)
        self.dout = z(R, d)
        self.dx_perm = z(R, d)
        self.dx_shared = z(T, d) if n_shared else None
        self.dw13 = z(E, P, d)
        self.dw2 = z(E, d, f)
        self.dsw13 = z(1, P, d) if n_shared else None
        self.dsw2 = z(1, d, f) if n_shared else None
        self.dlogits = z(T, E, dtype=f32)
        self.dx_router = z(T, d, dtype=f32)
        self.dw_r = z(E, d, dtype=f32)
        self.dX = z(T, d)
        u8 = torch.uint8

        # per-row exponents (int32), or the block-scale array of the
        # [rows, K] matrix (bytes)
        # (rows: the operand's leading shape; K: its row length)
        def sc_blk(rows, K):
            n = 1
            for r in rows:
                n *= r
            return z(fp8_block_scale_bytes(n, K), dtype=u8)

        def sc_row(rows, K):
            return z(*rows, dtype=i32)
        # row layouts for the FP8 forward, transposes for the FP8 data gradients
        # (the square quantizer writes whichever of the two the layer runs)
        if fp8_fwd:
            sc = sc_blk if self.fp8_block else sc_row
            self.xq_perm, self.sx_perm = z(R, d, dtype=u8), sc((R,), d)
            self.w13q, self.s13 = z(E, P, d, dtype=u8), sc((E, P), d)
            self.w2q, self.s2 = z(E, d, f, dtype=u8), sc((E, d), f)
            sh = bool(n_shared)
            self.xq, self.sx = (z(T, d, dtype=u8), sc((T,), d)) if sh else (None, None)
            self.sw13q, self.ss13 = (z(1, P, d, dtype=u8), sc((1, P), d)) if sh else (None, None)
            self.sw2q, self.ss2 = (z(1, d, f, dtype=u8), sc((1, d), f)) if sh else (None, None)
        if fp8_bwd:
            sh = bool(n_shared)
            sct = sc_blk if self.fp8_square else sc_row
            self.w13q_t, self.s13_t = z(E, d, P, dtype=u8), sct((E, d), P)
            self.w2q_t, self.s2_t = z(E, f, d, dtype=u8), sct((E, f), d)
            self.sw13q_t, self.ss13_t = (z(1, d, P, dtype=u8), sct((1, d), P)) if sh else (None, None)
            self.sw2q_t, self.ss2_t = (z(1, f, d, dtype=u8), sct((1, f), d)) if sh else (None, None)
        if self.fp8_square:
            bwd_op = MOE_OP_FFN_BWD_FP8BW if fp8_wgrad else MOE_OP_FFN_BWD_FP8B
        else:
            bwd_op = MOE_OP_FFN_BWD_FP8W if fp8_wgrad else MOE_OP_FFN_BWD_FP8
        ops = [MOE_OP_ROUTE, MOE_OP_AUX_STATS, MOE_OP_PERMUTE, MOE_OP_FFN_FWD, MOE_OP_FFN_BWD,
               MOE_OP_ROUTE_BWD] + \
              ([MOE_OP_FFN_FWD_FP8B if self.fp8_block else MOE_OP_FFN_FWD_FP8] if fp8_fwd else []) + \
              ([bwd_op] if fp8_bwd else [])
        wsb = max(workspace_size(self.desc, op) for op in ops)
        if fp8_fwd and fp8_bwd and not self.fp8_square:   # both orientations from the forward's pass
            wsb = max(wsb, quantize_fp8_both_ws((E, P, d)), quantize_fp8_both_ws((E, d, f)))
        self._wt_from = None      # weights whose transposed codes the forward made
        self.ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)

    # ------------------------------------------------------------ stages
    def forward(self, x, w_r, w13, w2, sw13=None, sw2=None, logit_bias=None, sel_bias=None,
                gumbel_u=None):
        D = self.desc
        route(D, x, w_r, logit_bias, sel_bias, self.topk_idx, self.gate, self.scores, self.lse,
              self.ws, gumbel_u=gumbel_u)
        aux_stats(D, self.scores, self.topk_idx, self.lse, self.counts, self.y_frac, self.z_mean,
                  self.aux_out, self.ws)
        permute(D, x, self.topk_idx, self.offsets, self.row_of, self.token_of, self.n_dropped,
                self.x_perm, self.ws)
        if self.fp8_block:
            quantize_fp8_blocks(self.x_perm, self.xq_perm, self.sx_perm,
                                valid_rows=self.offsets[self.E:])
            if self.fp8_square:
                # both layouts from one read; the backward reuses the transposes
                self._quantize_squares(w13, w2, sw13, sw2)
            else:
                quantize_fp8_blocks(w13, self.w13q, self.s13)
                quantize_fp8_blocks(w2, self.w2q, self.s2)
            if self.n_shared:
                quantize_fp8_blocks(x, self.xq, self.sx)
                if not self.fp8_square:
                    quantize_fp8_blocks(sw13, self.sw13q, self.ss13)
                    quantize_fp8_blocks(sw2, self.sw2q, self.ss2)
            grouped_ffn_fwd_fp8b(D, self.xq_perm, self.sx_perm, self.offsets, self.xq, self.sx,
                                 self.w13q, self.s13, self.w2q, self.s2, self.sw13q, self.ss13,
                                 self.sw2q, self.ss2, self.save_pre, self.save_h, self.save_pre_s,
                                 self.save_h_s, self.out, self.out_shared, self.ws)
        elif self.fp8_fwd:
            quantize_fp8(self.x_perm, self.xq_perm, self.sx_perm, valid_rows=self.offsets[self.E:])
            if self.fp8_bwd:
                # rows for the forward and columns (transposes) for the backward in one pass
                quantize_fp8_both(w13, self.w13q, self.s13, self.w13q_t, self.s13_t, self.ws)
                quantize_fp8_both(w2, self.w2q, self.s2, self.w2q_t, self.s2_t, self.ws)
                self._wt_from = (w13.data_ptr(), w2.data_ptr())
            else:
                quantize_fp8(w13, self.w13q, self.s13)
                quantize_fp8(w2, self.w2q, self.s2)
            if self.n_shared:
                quantize_fp8(x, self.xq, self.sx)
                if self.fp8_bwd:
                    quantize_fp8_both(sw13, self.sw13q, self.ss13, self.sw13q_t, self.ss13_t, self.ws)
                    quantize_fp8_both(sw2, self.sw2q, self.ss2, self.sw2q_t, self.ss2_t, self.ws)
                else:
                    quantize_fp8(sw13, self.sw13q, self.ss13)
                    quantize_fp8(sw2, self.sw2q, self.ss2)
            grouped_ffn_fwd_fp8(D, self.xq_perm, self.sx_perm, self.offsets, self.xq, self.sx,
                                self.w13q, self.s13, self.w2q, self.s2, self.sw13q, self.ss13,
                                self.sw2q, self.ss2, self.save_pre, self.save_h, self.save_pre_s,
                                self.save_h_s, self.out, self.out_shared, self.ws)
        else:
            grouped_ffn_fwd(D, self.x_perm, self.offsets, x, w13, w2, sw13, sw2, self.save_pre,
                            self.save_h, self.save_pre_s, self.save_h_s, self.out,
                            self.out_shared, self.ws)
        combine(D, self.out, self.out_shared, self.gate, self.row_of, self.Y)
        return self.Y

    def _quantize_squares(self, w13, w2, sw13, sw2):
        """Square-block codes of the weights in the layouts this layer runs:
        rows for the FP8 forward, transposes for the FP8 data gradients."""
        def pair(codes, scales, on):
            return (getattr(self, codes), getattr(self, scales)) if on else (None, None)
        names = [(w13, "w13q", "s13"), (w2, "w2q", "s2")]
        if self.n_shared:
            names += [(sw13, "sw13q", "ss13"), (sw2, "sw2q", "ss2")]
        for w, c, sc in names:
            quantize_fp8_squares(w, *pair(c, sc, self.fp8_fwd), *pair(c + "_t", sc + "_t", self.fp8_bwd))
        self._wt_from = (w13.data_ptr(), w2.data_ptr())

    def backward(self, dy, x, w_r, w13, w2, sw13=None, sw2=None):
        D = self.desc
        combine_bwd(D, dy, self.out, self.gate, self.row_of, self.dgate, self.dout)
        if self.fp8_bwd and self.fp8_square:
            if self._wt_from != (w13.data_ptr(), w2.data_ptr()):
                self._quantize_squares(w13, w2, sw13, sw2)
            self._wt_from = None
            grouped_ffn_bwd_fp8(D, self.x_perm, self.offsets, x, self.w13q_t, self.s13_t,
                                self.w2q_t, self.s2_t, self.sw13q_t, self.ss13_t, self.sw2q_t,
                                self.ss2_t, self.save_pre, self.save_h, self.save_pre_s,
                                self.save_h_s, self.dout, dy, self.dx_perm, self.dx_shared,
                                self.dw13, self.dw2, self.dsw13, self.dsw2, self.ws,
                                fp8_wgrad=self.fp8_wgrad, block=True)
        elif self.fp8_bwd:
            # the forward already made the transposed codes of these weights
            # (FP8 forward); otherwise quantize them here
            if self._wt_from != (w13.data_ptr(), w2.data_ptr()):
                quantize_fp8_t(w13, self.w13q_t, self.s13_t)
                quantize_fp8_t(w2, self.w2q_t, self.s2_t)
                if self.n_shared:
                    quantize_fp8_t(sw13, self.sw13q_t, self.ss13_t)
                    quantize_fp8_t(sw2, self.sw2q_t, self.ss2_t)
            self._wt_from = None
            grouped_ffn_bwd_fp8(D, self.x_perm, self.offsets, x, self.w13q_t, self.s13_t,
                                self.w2q_t, self.s2_t, self.sw13q_t, self.ss13_t, self.sw2q_t,
                                self.ss2_t, self.save_pre, self.save_h, self.save_pre_s,
                                self.save_h_s, self.dout, dy, self.dx_perm, self.dx_shared,
                                self.dw13, self.dw2, self.dsw13, self.dsw2, self.ws,
                                fp8_wgrad=self.fp8_wgrad)
        else:
            grouped_ffn_bwd(D, self.x_perm, self.offsets, x, w13, w2, sw13, sw2, self.save_pre,
                            self.save_h, self.save_pre_s, self.save_h_s, self.dout, dy,
                            self.dx_perm, self.dx_shared, self.dw13, self.dw2, self.dsw13,
                            self.dsw2, self.ws)
        route_bwd(D, x, w_r, self.scores, self.topk_idx, self.gate, self.dgate, self.y_frac,
                  self.aux_coef, self.lse, self.z_coef, self.dlogits, self.dx_router, self.dw_r,
                  self.ws)
        permute_bwd(D, self.dx_perm, self.row_of, self.dx_shared, self.dx_router, self.dX)
        return self.dX

    def update_bias(self, sel_bias, gamma=None):
        """Aux-loss-free balancing: nudge sel_bias (in place) by the last forward's loads."""
        bias_update(self.desc, self.counts, self.bias_gamma if gamma is None else gamma, sel_bias)

    def step(self, inp: dict):
        """Forward then backward over one batch; inp holds the device tensors."""
        self.forward(inp["x"], inp["w_r"], inp["w13"], inp["w2"], inp.get("sw13"),
                     inp.get("sw2"), inp.get("logit_bias"), inp.get("sel_bias"),
                     inp.get("gumbel_u"))
        self.backward(inp["dy"], inp["x"], inp["w_r"], inp["w13"], inp["w2"], inp.get("sw13"),
                      inp.get("sw2"))
        if self.bias_gamma and inp.get("sel_bias") is not None:
            self.update_bias(inp["sel_bias"])
