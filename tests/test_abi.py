"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import mixture_experts_layer_28_amd as moe
import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(moe_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    names = _declared()
    assert len(names) == 29
    assert sorted(moe.EXPORTS) == names
    for n in names:
        assert hasattr(L, n), n
    assert L.moe_abi_version() == 7


# fake, aligned, non-null device addresses: validation must fail (or, for
# T = 0, succeed) before anything touches them
FAKE = 0x100000


def _status(fn, *args):
    return fn(*args)


def _desc(**kw):
    base = dict(T=64, d=64, E=8, k=2, f=64)
    base.update(kw)
    return moe.make_desc(**base)


def test_desc_validation():
    L = moe.lib()
    bad = [
        _desc(d=60), _desc(f=12), _desc(k=0), _desc(k=9), _desc(E=0), _desc(E=2000),
        _desc(T=-1), _desc(n_shared=2),
    ]
    for d in bad:
        out = ctypes.c_size_t()
        s = L.moe_workspace_size(ctypes.byref(d), 0, ctypes.byref(out))
        assert s in (1, 2), (d.d, d.f, d.k, d.E, d.T)
        assert L.moe_last_error().decode()
    d = _desc()
    d.dtype = 7
    assert L.moe_workspace_size(ctypes.byref(d), 0, ctypes.byref(ctypes.c_size_t())) == 1
    d = _desc(k=17, E=32)
    assert L.moe_workspace_size(ctypes.byref(d), 0, ctypes.byref(ctypes.c_size_t())) == 2


def test_null_and_misaligned_pointers_rejected():
    L = moe.lib()
    d = _desc()
    ws = moe.workspace_size(d, moe.MOE_OP_ROUTE)
    # x NULL
    s = L.moe_route(ctypes.byref(d), None, FAKE, None, None, None, FAKE, FAKE, FAKE, None, FAKE, ws,
                    None)
    assert s == 1 and "x is NULL" in L.moe_last_error().decode()
    # misaligned gate
    s = L.moe_route(ctypes.byref(d), FAKE, FAKE, None, None, None, FAKE, FAKE + 4, FAKE, None, FAKE, ws,
                    None)
    assert s == 1 and "aligned" in L.moe_last_error().decode()
    # workspace too small
    s = L.moe_route(ctypes.byref(d), FAKE, FAKE, None, None, None, FAKE, FAKE, FAKE, None, FAKE, ws - 1,
                    None)
    assert s == 3
    # combine without row_of
    s = L.moe_combine(ctypes.byref(d), FAKE, None, FAKE, None, FAKE, None)
    assert s == 1 and "row_of" in L.moe_last_error().decode()
    # shared expert requested but its weights missing
    ds = _desc(n_shared=1)
    s = L.moe_grouped_ffn_fwd(ctypes.byref(ds), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE,
                              FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None)
    assert s == 1 and "sw13" in L.moe_last_error().decode()
    # misaligned lse
    s = L.moe_route(ctypes.byref(d), FAKE, FAKE, None, None, None, FAKE, FAKE, FAKE, FAKE + 2, FAKE, ws,
                    None)
    assert s == 1 and "lse" in L.moe_last_error().decode()
    # bias update without a bias vector
    assert L.moe_bias_update(ctypes.byref(d), FAKE, 1e-3, None, None) == 1
    assert "bias" in L.moe_last_error().decode()
    assert L.moe_bias_update(ctypes.byref(d), FAKE, float("nan"), FAKE, None) == 1


def test_fp8_gradient_format_validation():
    """desc.fp8_grad takes E4M3 (0) or E5M2 (1); anything else fails desc
    validation before any HIP call."""
    L = moe.lib()
    for v, want in ((0, 0), (1, 0), (2, 1), (-1, 1)):
        d = _desc()
        d.fp8_grad = v
        out = ctypes.c_size_t()
        assert L.moe_workspace_size(ctypes.byref(d), moe.MOE_OP_FFN_BWD_FP8, ctypes.byref(out)) == want
    with pytest.raises(ValueError):
        moe.make_desc(64, 64, 8, 2, 64, fp8_grad="e3m4")
    assert moe.make_desc(64, 64, 8, 2, 64, fp8_grad="e5m2").fp8_grad == moe.MOE_FP8_E5M2
    # the struct layout the header declares: 6 int64, 3 int32, a float, an int64, 2 int32
    assert ctypes.sizeof(moe.MoeDesc) == 80 and moe.MoeDesc.fp8_grad.offset == 72


def test_noisy_gate_validation():
    L = moe.lib()
    ws = moe.workspace_size(_desc(), moe.MOE_OP_ROUTE)
    route = lambda d, u: L.moe_route(ctypes.byref(d), FAKE, FAKE, None, None, u, FAKE, FAKE, FAKE,
                                     None, FAKE, ws, None)
    # temperature set but no draws
    assert route(_desc(gumbel_tau=0.5), None) == 1 and "gumbel_u" in L.moe_last_error().decode()
    # draws without a temperature
    assert route(_desc(), FAKE) == 1 and "gumbel_tau" in L.moe_last_error().decode()
    # misaligned draws
    assert route(_desc(gumbel_tau=0.5), FAKE + 2) == 1
    # negative or non-finite temperature, and sigmoid scoring, are refused at the descriptor
    out = ctypes.c_size_t()
    for bad, code in ((_desc(gumbel_tau=-1.0), 1), (_desc(gumbel_tau=float("inf")), 1),
                      (_desc(gumbel_tau=1.0, score="sigmoid"), 2)):
        assert L.moe_workspace_size(ctypes.byref(bad), 0, ctypes.byref(out)) == code
    # a zero-token call with the noisy gate on is a no-op that touches nothing
    assert L.moe_route(ctypes.byref(_desc(T=0, gumbel_tau=0.5)), FAKE, FAKE, None, None, FAKE,
                       FAKE, FAKE, FAKE, None, None, 0, None) == 0


def test_z_loss_needs_softmax_scoring_and_lse():
    L = moe.lib()
    ws = moe.workspace_size(_desc(score="sigmoid"), moe.MOE_OP_ROUTE_BWD)
    args = [FAKE] * 6 + [None, 0.0]
    tail = [FAKE, FAKE, FAKE, FAKE if ws else None, ws, None]
    d = _desc(score="sigmoid")
    assert L.moe_route_bwd(ctypes.byref(d), *args, FAKE, 1e-3, *tail) == 2
    assert "softmax" in L.moe_last_error().decode()
    d = _desc()
    assert L.moe_route_bwd(ctypes.byref(d), *args, None, 1e-3, *tail) == 1
    assert "lse" in L.moe_last_error().decode()
    assert L.moe_route_bwd(ctypes.byref(d), *args, None, float("nan"), *tail) == 1


def test_zero_tokens_is_a_noop_without_touching_memory():
    L = moe.lib()
    d = _desc(T=0)
    assert L.moe_route(ctypes.byref(d), FAKE, FAKE, None, None, None, FAKE, FAKE, FAKE, FAKE, None, 0,
                       None) == 0
    assert L.moe_aux_stats(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0,
                           None) == 0
    assert L.moe_bias_update(ctypes.byref(d), FAKE, 1e-3, FAKE, None) == 0
    assert L.moe_permute(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 0
    assert L.moe_combine(ctypes.byref(d), FAKE, None, FAKE, FAKE, FAKE, None) == 0
    assert L.moe_combine_bwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 0
    assert L.moe_permute_bwd(ctypes.byref(d), FAKE, FAKE, None, None, FAKE, None) == 0


@pytest.mark.parametrize("T,k,E,cf", [(1024, 1, 8, 1.25), (8192, 2, 8, 1.25), (4096, 2, 8, 1.0),
                                      (1000, 3, 7, 1.1), (37, 2, 5, 0.33), (64, 2, 8, 0.0)])
def test_capacity_matches_oracle(T, k, E, cf):
    assert moe.capacity(T, k, E, cf) == O.capacity(T, k, E, cf)
    assert moe.capacity(T, k, E, None) is None


def test_workspace_sizes_cover_the_layer():
    d = moe.make_desc(8192, 4096, 8, 2, 14336, capacity=2560)
    sizes = [moe.workspace_size(d, op) for op in range(8)]
    # the FP8 forward keeps H's codes and exponents between its two GEMMs
    assert sizes[moe.MOE_OP_FFN_FWD_FP8] >= 8192 * 2 * 14336 + 8192 * 2 * 4
    # backward needs the [T*k, 2f] activation-gradient buffer
    assert sizes[moe.MOE_OP_FFN_BWD] >= 8192 * 2 * 2 * 14336 * 2
    assert sizes[moe.MOE_OP_ROUTE] >= 8192 * 8 * 4
    # the FP8 backward adds the codes and exponents of dO [T*k, d] and dpre [T*k, 2f]
    assert sizes[moe.MOE_OP_FFN_BWD_FP8] >= sizes[moe.MOE_OP_FFN_BWD] + 16384 * (4096 + 4) + \
        16384 * (2 * 14336 + 4)
    with pytest.raises(moe.MoeError):
        moe.workspace_size(d, 99)


def test_status_strings():
    L = moe.lib()
    assert L.moe_status_str(0) == b"ok"
    assert L.moe_status_str(3) == b"workspace too small"


def _header_params():
    text = open(HEADER).read()
    out = {}
    for m in re.finditer(r"^(?:int|const char\*)\s+(moe_\w+)\s*\(([^)]*)\)\s*;", text, re.M | re.S):
        params = [p.strip() for p in m.group(2).replace("\n", " ").split(",") if p.strip()]
        if params == ["void"]:
            params = []
        out[m.group(1)] = params
    return out


def _kind(param):
    if "*" in param:
        return "ptr"
    if param.startswith("size_t"):
        return "size_t"
    if param.startswith("float"):
        return "float"
    if param.startswith("double"):
        return "double"
    if param.startswith("int64_t"):
        return "int64"
    if param.startswith("int"):
        return "int"
    raise AssertionError(param)


def test_binding_signatures_match_header():
    L = moe.lib()
    ct = {ctypes.c_void_p: "ptr", ctypes.c_size_t: "size_t", ctypes.c_float: "float",
          ctypes.c_double: "double", ctypes.c_int64: "int64", ctypes.c_int: "int"}
    for name, params in _header_params().items():
        want = [_kind(p) for p in params]
        got = []
        for a in getattr(L, name).argtypes:
            got.append(ct.get(a, "ptr"))  # POINTER(...) types are pointers
        assert got == want, (name, got, want)


def test_permute_noalloc_validation():
    """The workspace-free permute checks its arguments as moe_permute does,
    before any HIP call (fake pointers are never touched); T = 0 is a no-op."""
    L = moe.lib()
    D = _desc()
    args = [FAKE] * 7
    for i in range(7):
        bad = list(args)
        bad[i] = None
        st = L.moe_permute_noalloc(ctypes.byref(D), *bad, None)
        assert st == 1, (i, st)                       # MOE_ERR_INVALID_ARG
        bad[i] = FAKE + 4
        assert L.moe_permute_noalloc(ctypes.byref(D), *bad, None) == 1
    Z = _desc(T=0)
    assert L.moe_permute_noalloc(ctypes.byref(Z), *args, None) == 0
    B = _desc(E=0)
    assert L.moe_permute_noalloc(ctypes.byref(B), *args, None) == 1


def test_fp8_quantize_validation():
    """Bad sizes, strides and pointers fail before any HIP call; rows = 0 is
    a successful no-op."""
    L = moe.lib()
    P = ctypes.c_void_p
    ok = dict(src=FAKE, rows=4, K=64, ld_src=64, valid=None, codes=FAKE, ld_q=64, sexp=FAKE)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.moe_quantize_fp8(P(a["src"]) if a["src"] else None, a["rows"], a["K"], a["ld_src"],
                                  P(a["valid"]) if a["valid"] else None,
                                  P(a["codes"]) if a["codes"] else None, a["ld_q"],
                                  P(a["sexp"]) if a["sexp"] else None, None)
    for bad in (dict(K=8), dict(K=72), dict(ld_src=32), dict(ld_src=68), dict(ld_q=72),
                dict(rows=-1), dict(src=0), dict(codes=FAKE + 8), dict(sexp=0),
                dict(valid=FAKE + 2)):
        assert call(**bad) == 1, bad
        assert L.moe_last_error().decode()
    assert call(rows=0) == 0


def test_fp8_forward_validation():
    L = moe.lib()
    P = ctypes.c_void_p
    ptrs = [P(FAKE)] * 19

    def call(d, ws_bytes=1 << 40):
        return L.moe_grouped_ffn_fwd_fp8(ctypes.byref(d), *ptrs, P(FAKE), ws_bytes, None)
    # fp32 layers and widths off the 16-grid are unsupported; too little workspace fails
    assert call(_desc(dtype="f32")) == 2
    assert call(_desc(d=72)) == 2 and call(_desc(f=72)) == 2
    assert call(_desc(), ws_bytes=16) == 3
    assert call(_desc(T=0)) == 0


def test_fp8_block_quantize_validation():
    """Bad sizes, strides and pointers fail before any HIP call; rows = 0 is
    a successful no-op."""
    L = moe.lib()
    P = ctypes.c_void_p
    ok = dict(src=FAKE, rows=4, K=80, ld_src=80, valid=None, codes=FAKE, ld_q=80, sc=FAKE)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        ptr = lambda v: P(v) if v else None   # noqa: E731
        return L.moe_quantize_fp8_blocks(ptr(a["src"]), a["rows"], a["K"], a["ld_src"],
                                         ptr(a["valid"]), ptr(a["codes"]), a["ld_q"], ptr(a["sc"]),
                                         None)
    for bad in (dict(K=8), dict(K=72), dict(ld_src=64), dict(ld_src=84), dict(ld_q=88),
                dict(rows=-1), dict(rows=1 << 31), dict(src=0), dict(codes=FAKE + 8),
                dict(sc=0), dict(sc=FAKE + 4), dict(valid=FAKE + 2),
                # 2^30 rows x 2 words: the scale array would reach 2^31 words
                dict(rows=1 << 30, K=256, ld_src=256, ld_q=256)):
        assert call(**bad) == 1, bad
        assert L.moe_last_error().decode()
    assert call(rows=0) == 0


def test_fp8_block_forward_validation():
    L = moe.lib()
    P = ctypes.c_void_p
    ptrs = [P(FAKE)] * 19

    def call(d, ws_bytes=1 << 40, p=ptrs):
        return L.moe_grouped_ffn_fwd_fp8b(ctypes.byref(d), *p, P(FAKE), ws_bytes, None)
    assert call(_desc(dtype="f32")) == 2
    assert call(_desc(d=72)) == 2 and call(_desc(f=72)) == 2
    assert call(_desc(T=0)) == 0
    # the workspace holds H's codes and block scales (128 bytes per 128 of f
    # and 32 rows: 4 groups of 32 rows x 2 words here)
    d = _desc(T=64, k=2, f=256)
    need = ctypes.c_size_t()
    assert L.moe_workspace_size(ctypes.byref(d), moe.MOE_OP_FFN_FWD_FP8B, ctypes.byref(need)) == 0
    row = ctypes.c_size_t()
    assert L.moe_workspace_size(ctypes.byref(d), moe.MOE_OP_FFN_FWD_FP8, ctypes.byref(row)) == 0
    assert need.value - row.value == 128 * 2 * 4 - 128 * 4
    assert call(d, ws_bytes=need.value - 1) == 3
    # a NULL or misaligned block-scale array is rejected
    for bad_v in (None, P(FAKE + 4)):
        bad = list(ptrs)
        bad[1] = bad_v
        assert call(_desc(), p=bad) == 1


def test_fp8_wgrad_backward_validation():
    """The FP8 weight-gradient backward validates like the FP8 backward, and
    its workspace adds the token-axis codes and scales of both operands."""
    L = moe.lib()
    P = ctypes.c_void_p
    ptrs = [P(FAKE)] * 23

    def call(d, ws_bytes=1 << 40):
        return L.moe_grouped_ffn_bwd_fp8w(ctypes.byref(d), *ptrs, P(FAKE), ws_bytes, None)
    assert call(_desc(dtype="f32")) == 2
    assert call(_desc(d=72)) == 2 and call(_desc(f=72)) == 2
    d = _desc(T=64, d=64, E=8, k=2, f=64)
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.moe_workspace_size(ctypes.byref(d), moe.MOE_OP_FFN_BWD_FP8, ctypes.byref(a)) == 0
    assert L.moe_workspace_size(ctypes.byref(d), moe.MOE_OP_FFN_BWD_FP8W, ctypes.byref(b)) == 0
    # Rp = 128 * (ceil(128 / 128) + 8) = 1152: codes 128 x Rp and 64 x Rp,
    # scales 128 * 9 per 32 rows, a 9-int k-step table, two bounds
    Rp = 1152
    extra = (128 * Rp) + (4 * 128 * 9) + (64 * Rp) + (2 * 128 * 9) + 256 + 256
    assert b.value - a.value == extra
    assert call(d, ws_bytes=b.value - 1) == 3
    bad = list(ptrs)
    bad[3] = None
    assert L.moe_grouped_ffn_bwd_fp8w(ctypes.byref(_desc()), *bad, P(FAKE), 1 << 40, None) == 1


def test_fp8_transposing_quantize_validation():
    """Bad shapes and pointers fail before any HIP call; G = 0 is a no-op."""
    L = moe.lib()
    P = ctypes.c_void_p
    ok = dict(src=FAKE, G=2, R=64, C=24, codes=FAKE, sexp=FAKE)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.moe_quantize_fp8_t(P(a["src"]) if a["src"] else None, a["G"], a["R"], a["C"],
                                    P(a["codes"]) if a["codes"] else None,
                                    P(a["sexp"]) if a["sexp"] else None, None)
    for bad in (dict(R=8), dict(R=72), dict(R=0), dict(C=4), dict(C=12), dict(G=-1),
                dict(G=70000), dict(src=0), dict(codes=FAKE + 8), dict(sexp=FAKE + 4)):
        assert call(**bad) == 1, bad
        assert L.moe_last_error().decode()
    assert call(G=0) == 0


def test_fp8_backward_validation():
    L = moe.lib()
    P = ctypes.c_void_p
    ptrs = [P(FAKE)] * 23

    def call(d, ws_bytes=1 << 40):
        return L.moe_grouped_ffn_bwd_fp8(ctypes.byref(d), *ptrs, P(FAKE), ws_bytes, None)
    assert call(_desc(dtype="f32")) == 2
    assert call(_desc(d=72)) == 2 and call(_desc(f=72)) == 2
    assert call(_desc(), ws_bytes=16) == 3
    # a NULL transposed weight is rejected
    bad = list(ptrs)
    bad[3] = None
    assert L.moe_grouped_ffn_bwd_fp8(ctypes.byref(_desc()), *bad, P(FAKE), 1 << 40, None) == 1


def test_fp8_quantize_both_validation():
    """Bad shapes, pointers and workspace fail before any HIP call."""
    L = moe.lib()
    P = ctypes.c_void_p
    ok = dict(src=FAKE, G=2, R=64, C=48, codes=FAKE, sexp=FAKE, codes_t=FAKE, sexp_t=FAKE,
              ws=FAKE, ws_bytes=1 << 20)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        ptr = lambda v: P(v) if v else None   # noqa: E731
        return L.moe_quantize_fp8_both(ptr(a["src"]), a["G"], a["R"], a["C"], ptr(a["codes"]),
                                       ptr(a["sexp"]), ptr(a["codes_t"]), ptr(a["sexp_t"]),
                                       ptr(a["ws"]), a["ws_bytes"], None)
    for bad in (dict(R=8), dict(R=72), dict(C=8), dict(C=40), dict(C=32784), dict(G=-1),
                dict(codes_t=0), dict(sexp_t=FAKE + 4), dict(ws=FAKE + 16)):
        assert call(**bad) == 1, bad
    # 2 * ceil(64 / 64) * 48 * 2 = 192 bytes -> 256 needed
    assert call(ws_bytes=255) == 3 and call(ws=0) == 3
    assert call(G=0) == 0


def test_fp8_square_quantize_validation():
    """Bad shapes and pointers fail before any HIP call; G = 0 is a no-op."""
    L = moe.lib()
    P = ctypes.c_void_p
    ok = dict(src=FAKE, G=2, R=64, C=48, codes=FAKE, sc=FAKE, codes_t=FAKE, sc_t=FAKE)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        ptr = lambda v: P(v) if v else None   # noqa: E731
        return L.moe_quantize_fp8_squares(ptr(a["src"]), a["G"], a["R"], a["C"], ptr(a["codes"]),
                                          ptr(a["sc"]), ptr(a["codes_t"]), ptr(a["sc_t"]), None)
    for bad in (dict(R=8), dict(R=72), dict(R=0), dict(C=8), dict(C=40), dict(C=1 << 23),
                dict(R=1 << 23), dict(G=-1), dict(G=70000), dict(src=0), dict(codes=FAKE + 8),
                dict(sc=0), dict(sc=FAKE + 4), dict(codes_t=0), dict(sc_t=FAKE + 2),
                # 2^15 matrices of 2^17 rows x 1 word: the row-layout scales reach 2^31 words
                dict(G=1 << 15, R=1 << 17, C=16),
                # a layout's codes and scales come together, and one layout at least
                dict(codes=0), dict(sc_t=0), dict(codes=0, sc=0, codes_t=0, sc_t=0)):
        assert call(**bad) == 1, bad
        assert L.moe_last_error().decode()
    assert call(G=0) == 0
    assert call(G=0, codes=0, sc=0) == 0 and call(G=0, codes_t=0, sc_t=0) == 0


@pytest.mark.parametrize("name,op", [("moe_grouped_ffn_bwd_fp8b", moe.MOE_OP_FFN_BWD_FP8B),
                                     ("moe_grouped_ffn_bwd_fp8bw", moe.MOE_OP_FFN_BWD_FP8BW)])
def test_fp8_block_backward_validation(name, op):
    """The block-scaled FP8 backward validates like the per-row one; its
    workspace holds block-scale bytes of dO and dpre in place of one int32
    per row, and the weight-gradient form adds the token-axis buffers of
    moe_grouped_ffn_bwd_fp8w and a second one for dO's token-axis codes
    (kept from the data gradients to dW2)."""
    L = moe.lib()
    P = ctypes.c_void_p
    ptrs = [P(FAKE)] * 23
    fn = getattr(L, name)

    def call(d, ws_bytes=1 << 40, p=ptrs):
        return fn(ctypes.byref(d), *p, P(FAKE), ws_bytes, None)
    assert call(_desc(dtype="f32")) == 2
    assert call(_desc(d=72)) == 2 and call(_desc(f=72)) == 2
    d = _desc(T=64, d=256, E=8, k=2, f=128)
    sz = {}
    for o in (moe.MOE_OP_FFN_BWD_FP8, moe.MOE_OP_FFN_BWD_FP8W, op):
        v = ctypes.c_size_t()
        assert L.moe_workspace_size(ctypes.byref(d), o, ctypes.byref(v)) == 0
        sz[o] = v.value
    al = lambda x: (x + 255) // 256 * 256   # noqa: E731
    R, P2 = 128, 256
    # block scales of [128, 256] and [128, 256]: 4 groups of 32 rows x 2 words x 128 bytes
    blk = al(moe.fp8_block_scale_bytes(R, 256)) + al(moe.fp8_block_scale_bytes(R, P2))
    row = al(4 * R) + al(4 * R)
    if op == moe.MOE_OP_FFN_BWD_FP8B:
        assert sz[op] - sz[moe.MOE_OP_FFN_BWD_FP8] == blk - row
    else:
        # plus dO's token-axis codes (d x Rp, Rp = 128 * (ceil(128 / 128) + 8)) and scales
        Rp = 1152
        assert sz[op] - sz[moe.MOE_OP_FFN_BWD_FP8W] == blk - row + al(256 * Rp) + \
            al(moe.fp8_block_scale_bytes(256, Rp))
    assert call(d, ws_bytes=sz[op] - 1) == 3
    # a NULL or misaligned transposed weight or scale array is rejected
    for i in (3, 4):
        for bad_v in (None, P(FAKE + 4)):
            bad = list(ptrs)
            bad[i] = bad_v
            assert call(_desc(), p=bad) == 1
