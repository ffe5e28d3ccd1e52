"""CPU oracle for the block-quantized weight matmul -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of `bench.py` may import
this package.  The product path (the HIP library and its binding) never calls it.

This is a ctypes wrapper over `qg_oracle.c` (plain C, built with gcc), which holds every piece
of arithmetic: the format decoders, the f16 / bf16 conversions, the f64 GEMM, the row scaling,
the routing plan, the combine, the MoE chain and its error-bound components.  The wrapper only
marshals numpy arrays (and builds the per-expert pointer tables the chain takes).  Each function's
definition and its sources are stated in `qg_oracle.c`.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

FMT = {"q4": 0, "q4a": 1, "q8": 2, "q8a": 3, "q8a16": 4}
XT = {"f32": 0, "f16": 1, "bf16": 2, "f64": 3}

_p = C.c_void_p
_i = C.c_int
_sz = C.c_size_t


def default_threads() -> int:
    """Host threads for the oracle: the CPU share this process is meant to use (OMP_NUM_THREADS when
    set, else the core count), at most 16."""
    n = os.environ.get("OMP_NUM_THREADS")
    n = int(n) if n and n.isdigit() else (os.cpu_count() or 1)
    return max(1, min(n, 16))


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = C.CDLL(_LIB_PATH)
        L.orc_f16_value.restype = C.c_double
        L.orc_f16_value.argtypes = [C.c_uint16]
        L.orc_bf16_value.restype = C.c_double
        L.orc_bf16_value.argtypes = [C.c_uint16]
        L.orc_f32_to_f16.restype = C.c_uint16
        L.orc_f32_to_f16.argtypes = [C.c_float]
        L.orc_f32_to_bf16.restype = C.c_uint16
        L.orc_f32_to_bf16.argtypes = [C.c_float]
        L.orc_weight_exact.restype = C.c_double
        L.orc_weight_exact.argtypes = [_i, _p, _p, _p, _i, _i, _i, _i, _i]
        L.orc_weight_f32.restype = C.c_float
        L.orc_weight_f32.argtypes = [_i, _p, _p, _p, _i, _i, _i, _i, _i]
        L.orc_dequant_tile.restype = None
        L.orc_dequant_tile.argtypes = [_i, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _p]
        L.orc_gguf_weight_f32.restype = C.c_float
        L.orc_gguf_weight_f32.argtypes = [_i, _p, _i, _i, _i]
        L.orc_gguf_dequant.restype = None
        L.orc_gguf_dequant.argtypes = [_i, _p, _i, _i, _p]
        L.orc_gguf_repack.restype = None
        L.orc_gguf_repack.argtypes = [_i, _p, _i, _i, _p, _p]
        L.orc_gguf_repack_q8a.restype = None
        L.orc_gguf_repack_q8a.argtypes = [_i, _p, _i, _i, _p, _p, _p]
        L.orc_gguf_repack_q8a16.restype = None
        L.orc_gguf_repack_q8a16.argtypes = [_i, _p, _i, _i, _p, _p, _p]
        L.orc_gemm.restype = _i
        L.orc_gemm.argtypes = [_i, _p, _p, _p, _i, _i, _i, _p, _i, _i, _p, _i, _p, _i, _p, _p, _i]
        L.orc_x_half.restype = None
        L.orc_x_half.argtypes = [_p, _i, _p, _i, _p, _p]
        L.orc_x_half_guard.restype = None
        L.orc_q8f_fields.restype = None
        L.orc_q8f_fields.argtypes = [_p, _i, _i, _i, _p, _p]
        L.orc_q8f_gemm.restype = None
        L.orc_col_scale.restype = None
        L.orc_col_scale.argtypes = [_p, _i, _i, _i, _p, _i, _p]
        L.orc_q8f_gemm.argtypes = [_p, _i, _i, _i, _p, _i, _i, _p, _p]
        L.orc_x_half_guard.argtypes = [_p, _i, _i, _p, _i, _i, _p, _p]
        L.orc_swiglu.restype = None
        L.orc_swiglu.argtypes = [_p, _p, _sz, _p]
        L.orc_moe_plan.restype = _i
        L.orc_moe_plan.argtypes = [_p, _i, _i, _i, _p, _p, _p, _p, _p]
        L.orc_moe_combine.restype = None
        L.orc_moe_combine.argtypes = [_p, _i, _p, _p, _i, _i, _p, _p]
        L.orc_moe_ffn.restype = _i
        L.orc_moe_ffn.argtypes = [_i, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _p, _i, _i, _p, _p, _p, _p, _p, _p,
                                  _p, _p, _p, _p, _i]
        for name in ("orc_f16_values", "orc_bf16_values"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [_p, _sz, _p]
        for name in ("orc_f32_to_f16_array", "orc_f32_to_bf16_array"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [_p, _sz, _p]
        L.orc_dequant_exact.restype = None
        L.orc_dequant_exact.argtypes = [_i, _p, _p, _p, _i, _i, _i, _p]
        L.orc_conv_stats.restype = None
        L.orc_conv_stats.argtypes = [_p, _i, _i, _i, C.c_double, _p]
        L.orc_conv_gather.restype = None
        L.orc_conv_gather.argtypes = [_p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _i, _p, _i, _p, _p]
        L.orc_conv2d.restype = _i
        L.orc_conv2d.argtypes = [_i, _p, _p, _p, _i, _i, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _i, _p, _i, _p,
                                 _i, _p, _p, _i]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _weights(fmt, codes, scales, offsets):
    if fmt == "q8":
        return _c(codes, np.int8), _c(scales, np.float32), None
    if fmt in ("q8a", "q8a16"):
        return _c(codes, np.int8), _c(scales, np.float32), _c(offsets, np.float32)
    return _c(codes, np.uint8), _c(scales, np.uint16), (_c(offsets, np.uint16) if fmt == "q4a" else None)


# ---- 16-bit float definitions ------------------------------------------------------------------
def f16_values(bits) -> np.ndarray:
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, np.float64)
    lib().orc_f16_values(_ptr(b), b.size, _ptr(out))
    return out


def bf16_values(bits) -> np.ndarray:
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, np.float64)
    lib().orc_bf16_values(_ptr(b), b.size, _ptr(out))
    return out


def f32_to_f16(x) -> np.ndarray:
    a = _c(x, np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().orc_f32_to_f16_array(_ptr(a), a.size, _ptr(out))
    return out


def f32_to_bf16(x) -> np.ndarray:
    a = _c(x, np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().orc_f32_to_bf16_array(_ptr(a), a.size, _ptr(out))
    return out


# ---- dequantization ----------------------------------------------------------------------------
def weight_exact(fmt, codes, scales, offsets, group, N, K, n, k) -> float:
    c, s, o = _weights(fmt, codes, scales, offsets)
    return lib().orc_weight_exact(FMT[fmt], _ptr(c), _ptr(s), _ptr(o), group, N, K, n, k)


def dequant_exact(fmt, codes, scales, offsets, group, N, K) -> np.ndarray:
    """Whole matrix of exact weight values, f64 [N, K]."""
    c, s, o = _weights(fmt, codes, scales, offsets)
    out = np.empty((N, K), np.float64)
    lib().orc_dequant_exact(FMT[fmt], _ptr(c), _ptr(s), _ptr(o), group, N, K, _ptr(out))
    return out


def dequant_tile(fmt, codes, scales, offsets, group, N, K, n0, k0, rows, cols, staged) -> np.ndarray:
    """The staged tile [rows, cols]: f32 values, or f16 / bf16 bits (uint16)."""
    c, s, o = _weights(fmt, codes, scales, offsets)
    out = np.empty((rows, cols), np.float32 if staged == "f32" else np.uint16)
    lib().orc_dequant_tile(FMT[fmt], _ptr(c), _ptr(s), _ptr(o), group, N, K, n0, k0, rows, cols, XT[staged],
                           _ptr(out))
    return out


# ---- GEMM --------------------------------------------------------------------------------------
def gemm(fmt, codes, scales, offsets, group, N, K, X, xtype, T, ns=None, ts=None, threads=None):
    """(Y, S, threads_used): Y[t][n] = sum_k x*v32 and S = sum_k |x*v32| in f64, over the selected
    rows ns (default all N) and tokens ts (default all T); arrays [len(ts), len(ns)]."""
    c, s, o = _weights(fmt, codes, scales, offsets)
    xdt = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "f64": np.float64}[xtype]
    if xtype == "f16" and np.asarray(X).dtype == np.float16:
        X = np.asarray(X).view(np.uint16)
    x = _c(X, xdt)
    nsa = None if ns is None else _c(ns, np.int32)
    tsa = None if ts is None else _c(ts, np.int32)
    nn = N if nsa is None else nsa.size
    nt = T if tsa is None else tsa.size
    Y = np.empty((nt, nn), np.float64)
    S = np.empty((nt, nn), np.float64)
    if threads is None:
        threads = default_threads()
    used = lib().orc_gemm(FMT[fmt], _ptr(c), _ptr(s), _ptr(o), group, N, K, _ptr(x), XT[xtype], T,
                          _ptr(nsa), nn, _ptr(tsa), nt, _ptr(Y), _ptr(S), int(threads))
    return Y, S, used


# ---- MoE pieces --------------------------------------------------------------------------------
def x_half(X, K, src=None, R=None):
    """(xh f16 bits [R, K], rs f32 [R]) of the per-row power-of-two scaling of f32 rows."""
    x = _c(X, np.float32)
    srca = None if src is None else _c(src, np.int32)
    if R is None:
        R = srca.size if srca is not None else x.size // K
    xh = np.empty((R, K), np.uint16)
    rs = np.empty(R, np.float32)
    lib().orc_x_half(_ptr(x), K, _ptr(srca), R, _ptr(xh), _ptr(rs))
    return xh, rs


def q8f_fields(blob, N, K, has_col):
    """(rs f64 [N], col f64 [K]) of a q8_2f (has_col) or q8_row tensor blob (int8 codes [N][K], then
    the f16 row scales, then the f16 column field)."""
    b = _c(blob, np.uint8)
    rs = np.empty(N, np.float64)
    col = np.empty(K, np.float64)
    lib().orc_q8f_fields(_ptr(b), int(bool(has_col)), N, K, _ptr(rs), _ptr(col))
    return rs, col


def q8f_gemm(blob, N, K, has_col, X, xtype, T):
    """(Y, S) f64 [T, N] of the q8_2f / q8_row matmul: w = q col[k] rs[n]."""
    b = _c(blob, np.uint8)
    xdt = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "f64": np.float64}[xtype]
    if xtype == "f16" and np.asarray(X).dtype == np.float16:
        X = np.asarray(X).view(np.uint16)
    x = _c(X, xdt)
    Y = np.empty((T, N), np.float64)
    S = np.empty((T, N), np.float64)
    lib().orc_q8f_gemm(_ptr(b), int(bool(has_col)), N, K, _ptr(x), XT[xtype], T, _ptr(Y), _ptr(S))
    return Y, S


def col_scale(X, xtype, T, K, col, out_type):
    """X times the column field, the f32 product rounded to out_type ("f32" -> float32, "f16" /
    "bf16" -> uint16 bits), [T, K]."""
    xdt = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16}[xtype]
    if xtype == "f16" and np.asarray(X).dtype == np.float16:
        X = np.asarray(X).view(np.uint16)
    x = _c(X, xdt)
    c = _c(col, np.float32)
    out = np.empty((T, K), np.float32 if out_type == "f32" else np.uint16)
    lib().orc_col_scale(_ptr(x), XT[xtype], T, K, _ptr(c), XT[out_type], _ptr(out))
    return out


def x_half_guard(X, K, shift, src=None, R=None, x_rows=None):
    """(xh f16 bits [R, K], rs f32 [R]) of the fixed power-of-two range guard: x * 2^-shift to f16."""
    x = _c(X, np.float32)
    srca = None if src is None else _c(src, np.int32)
    if x_rows is None:
        x_rows = x.size // K
    if R is None:
        R = srca.size if srca is not None else x_rows
    xh = np.empty((R, K), np.uint16)
    rs = np.empty(R, np.float32)
    lib().orc_x_half_guard(_ptr(x), x_rows, K, _ptr(srca), R, int(shift), _ptr(xh), _ptr(rs))
    return xh, rs


def swiglu(G, U) -> np.ndarray:
    g = _c(G, np.float64)
    u = _c(U, np.float64)
    out = np.empty(g.shape, np.float64)
    lib().orc_swiglu(_ptr(g), _ptr(u), g.size, _ptr(out))
    return out


def moe_plan(logits, T, E, k) -> dict:
    lg = _c(logits, np.float32)
    seg_off = np.empty(E + 1, np.int32)
    row_src = np.empty(T * k, np.int32)
    slot_row = np.empty(T * k, np.int32)
    slot_w = np.empty(T * k, np.float64)
    slot_e = np.empty(T * k, np.int32)
    R = lib().orc_moe_plan(_ptr(lg), T, E, k, _ptr(seg_off), _ptr(row_src), _ptr(slot_row), _ptr(slot_w),
                           _ptr(slot_e))
    return {"R": R, "seg_off": seg_off, "row_src": row_src, "slot_row": slot_row, "slot_w": slot_w,
            "slot_expert": slot_e}


def moe_combine(O, H, slot_row, slot_w, T, k):
    """(y [T, H], b [T, H]) with y = sum_j w_j O[row_j] and b = sum_j |w_j O[row_j]| in f64."""
    o = _c(O, np.float64)
    sr = _c(slot_row, np.int32)
    sw = _c(slot_w, np.float64)
    y = np.empty((T, H), np.float64)
    b = np.empty((T, H), np.float64)
    lib().orc_moe_combine(_ptr(o), H, _ptr(sr), _ptr(sw), T, k, _ptr(y), _ptr(b))
    return y, b


def moe_ffn(m: dict, plan: dict, fmt: str = "q4", group: int = 64, threads=None) -> dict:
    """The MoE expert block in f64, orc_moe_ffn of qg_oracle.c (definition and bound there).

    m: E, H, I, T, X f32 [T*H], gu_codes / gu_scales [E][...] (fused [2I][H] per expert: gate rows
    first), dn_codes / dn_scales [E][...] ([H][I]), and gu_offsets / dn_offsets for Q4A.  plan: the
    oracle's routing plan.  Returns y [T][H], the bound components b_dn and b_gu [T][H], and the
    stage values GU [R][2I], A [R][I], O [R][H]."""
    E, H, I, T = m["E"], m["H"], m["I"], m["T"]
    k = len(plan["slot_w"]) // T
    keep = []

    def table(codes, scales, offs):
        arr_c, arr_s, arr_o = (_p * E)(), (_p * E)(), (_p * E)()
        for e in range(E):
            c, s, o = _weights(fmt, codes[e], scales[e], None if offs is None else offs[e])
            keep.extend([c, s, o])
            arr_c[e], arr_s[e], arr_o[e] = _ptr(c), _ptr(s), _ptr(o)
        return arr_c, arr_s, (arr_o if fmt == "q4a" else None)

    gc, gs, go = table(m["gu_codes"], m["gu_scales"], m.get("gu_offsets"))
    dc, ds, do = table(m["dn_codes"], m["dn_scales"], m.get("dn_offsets"))
    X = _c(np.asarray(m["X"]).reshape(T, H), np.float32)
    seg = _c(plan["seg_off"], np.int32)
    src = _c(plan["row_src"], np.int32)
    sr = _c(plan["slot_row"], np.int32)
    sw = _c(plan["slot_w"], np.float64)
    R = int(seg[E])
    y = np.empty((T, H), np.float64)
    bdn = np.empty((T, H), np.float64)
    bgu = np.empty((T, H), np.float64)
    GU = np.empty((R, 2 * I), np.float64)
    A = np.empty((R, I), np.float64)
    O = np.empty((R, H), np.float64)
    if threads is None:
        threads = default_threads()
    got = lib().orc_moe_ffn(FMT[fmt], gc, gs, go, dc, ds, do, group, E, H, I, _ptr(X), T, k, _ptr(seg), _ptr(src),
                            _ptr(sr), _ptr(sw), _ptr(y), _ptr(bdn), _ptr(bgu), _ptr(GU), _ptr(A), _ptr(O),
                            int(threads))
    if got != R:
        raise ValueError("orc_moe_ffn: a gathered row names a token outside X")
    return {"y": y, "b_dn": bdn, "b_gu": bgu, "GU": GU, "A": A, "O": O}


# ---- GGUF blocks with in-block scales (GGML type ids) -------------------------------------------
GGUF = {"q4_0": 2, "q4_1": 3, "q5_0": 6, "q5_1": 7, "q8_0": 8, "q4_k": 12, "q5_k": 13, "q6_k": 14, "q3_k": 11,
        "q2_k": 10}
# bytes per 32 elements (Q4_K: 144 per 256, Q5_K: 176 per 256)
GGUF_BLOCK_BYTES = {"q4_0": 18, "q4_1": 20, "q5_0": 22, "q5_1": 24, "q8_0": 34, "q4_k": 18, "q5_k": 22}
# bytes per 256-element super-block of the K-quants with a scale per 16 elements
GGUF_SUPER_BYTES = {"q6_k": 210, "q3_k": 110, "q2_k": 84}


def gguf_dequant(gtype, src, N, K) -> np.ndarray:
    """f32 [N, K]: every element decoded from the GGUF bytes, as the pages' loaders evaluate it."""
    b = _c(src, np.uint8)
    out = np.empty((N, K), np.float32)
    lib().orc_gguf_dequant(GGUF[gtype], _ptr(b), N, K, _ptr(out))
    return out


def gguf_repack(gtype, src, N, K) -> tuple:
    """(codes, scales) of the split layout: Q4_0 -> uint8 [N*K/2], f16 bits uint16 [N*K/32];
    Q8_0 -> int8 [N*K], f32 [N*K/32]."""
    b = _c(src, np.uint8)
    if gtype == "q4_0":
        codes = np.empty(N * K // 2, np.uint8)
        scales = np.empty(N * K // 32, np.uint16)
    else:
        codes = np.empty(N * K, np.uint8)
        scales = np.empty(N * K // 32, np.float32)
    lib().orc_gguf_repack(GGUF[gtype], _ptr(b), N, K, _ptr(codes), _ptr(scales))
    return (codes if gtype == "q4_0" else codes.view(np.int8)), scales


def gguf_repack_q8a(gtype, src, N, K) -> tuple:
    """(codes int8 [N*K], scales f32 [N*K/32], offsets f32 [N*K/32]) of the Q8A layout for the
    affine types Q4_1, Q5_0, Q5_1, Q4_K and Q5_K."""
    b = _c(src, np.uint8)
    codes = np.empty(N * K, np.int8)
    scales = np.empty(N * K // 32, np.float32)
    offs = np.empty(N * K // 32, np.float32)
    lib().orc_gguf_repack_q8a(GGUF[gtype], _ptr(b), N, K, _ptr(codes), _ptr(scales), _ptr(offs))
    return codes, scales, offs


def gguf_repack_q8a16(gtype, src, N, K, with_offsets=True) -> tuple:
    """(codes int8 [N*K], scales f32 [N*K/16], offsets f32 [N*K/16] or None) of the Q8A16 layout for
    the K-quants with a scale per 16 elements (Q6_K, Q3_K, Q2_K); with_offsets=False (Q6_K, Q3_K)
    gives the offset-free layout."""
    b = _c(src, np.uint8)
    codes = np.empty(N * K, np.int8)
    scales = np.empty(N * K // 16, np.float32)
    offs = np.empty(N * K // 16, np.float32) if with_offsets else None
    lib().orc_gguf_repack_q8a16(GGUF[gtype], _ptr(b), N, K, _ptr(codes), _ptr(scales), _ptr(offs))
    return codes, scales, offs


# ---- convolution (implicit GEMM over the same weights) -----------------------------------------
NORM = {None: 0, "none": 0, "group": 1, "layer": 2}


def conv_out_size(H, W, ksz, stride):
    """(oh, ow) with pad = ksz // 2."""
    pad = ksz // 2
    return (H + 2 * pad - ksz) // stride + 1, (W + 2 * pad - ksz) // stride + 1


def conv_stats(X, npix, cin, groups, eps) -> np.ndarray:
    """f64 [n][2] (mean, rstd): groups > 0 -> per group of cin / groups channels over all pixels;
    groups == 0 -> per pixel over its cin channels."""
    x = _c(X, np.float32)
    n = groups if groups > 0 else npix
    out = np.empty((n, 2), np.float64)
    lib().orc_conv_stats(_ptr(x), npix, cin, groups, float(eps), _ptr(out))
    return out


def conv_gather(X, H, W, cin, ksz, stride, norm=None, groups=0, stats=None, gb=None, silu=False, ps=None):
    """(A, M) f64 [len(ps)][ksz*ksz*cin]: the implicit GEMM's gathered input rows and their error
    magnitudes (see orc_conv_gather)."""
    x = _c(X, np.float32)
    oh, ow = conv_out_size(H, W, ksz, stride)
    psa = _c(np.arange(oh * ow) if ps is None else ps, np.int32)
    K = ksz * ksz * cin
    A = np.empty((psa.size, K), np.float64)
    M = np.empty((psa.size, K), np.float64)
    cpg = cin // groups if groups else 1
    lib().orc_conv_gather(_ptr(x), H, W, cin, ksz, stride, NORM[norm], cpg, _ptr(_c(stats, np.float32)),
                          _ptr(_c(gb, np.float32)), int(bool(silu)), _ptr(psa), psa.size, _ptr(A), _ptr(M))
    return A, M


def conv2d(fmt, codes, scales, offsets, group, n_out, X, H, W, cin, ksz, stride, norm=None, groups=0, stats=None,
           gb=None, silu=False, ps=None, os_=None, threads=None):
    """(Y, S) f64 [len(ps)][len(os)] (all output pixels / channels by default): Y[p][o] = the
    convolution of the (normalised, activated) image with weight row o; S the error magnitude
    sum_k M |v32|.  stats: f32 [n][2] (mean, rstd) as the convolution uses them."""
    c, s, o = _weights(fmt, codes, scales, offsets)
    x = _c(X, np.float32)
    oh, ow = conv_out_size(H, W, ksz, stride)
    psa = None if ps is None else _c(ps, np.int32)
    osa = None if os_ is None else _c(os_, np.int32)
    np_ = oh * ow if psa is None else psa.size
    no = n_out if osa is None else osa.size
    Y = np.empty((np_, no), np.float64)
    S = np.empty((np_, no), np.float64)
    cpg = cin // groups if groups else 1
    if threads is None:
        threads = default_threads()
    lib().orc_conv2d(FMT[fmt], _ptr(c), _ptr(s), _ptr(o), group, n_out, _ptr(x), H, W, cin, ksz, stride, NORM[norm],
                     cpg, _ptr(_c(stats, np.float32)), _ptr(_c(gb, np.float32)), int(bool(silu)), _ptr(psa),
                     0 if psa is None else psa.size, _ptr(osa), 0 if osa is None else osa.size, _ptr(Y), _ptr(S),
                     int(threads))
    return Y, S
