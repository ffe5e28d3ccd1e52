"""Python binding of libqgemm.so, the block-quantized weight matmul for MI355X (gfx950).

The functions below carry the names of the C entry points declared in include/qgemm.h and only
marshal arguments: torch tensors become device pointers, dtypes become the activation-type enum,
the current torch stream is passed as the hipStream_t, and a non-zero status raises QGError.
Every step of the computation runs in the library's HIP kernels.  There is no fallback: if the
library is not built, loading raises.

Host-side helpers for the packed layout (pack_q4 / pack_q4_blocks, expert tables) live here too;
they only move bytes.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemm.so")

QG_OK, QG_EINVAL, QG_EALIGN, QG_ESHAPE, QG_EUNSUPPORTED, QG_ELAUNCH, QG_EPLAN, QG_EWORKSPACE, QG_ESCRATCH = range(9)
QG_NOALLOC_SCRATCH_BYTES = 16 << 20
QG_X_F32, QG_X_F16, QG_X_BF16 = 0, 1, 2
QG_EXACT, QG_FAST, QG_FAST_WEXACT = 0, 1, 2
QG_FMT_Q4, QG_FMT_Q4A, QG_FMT_Q8, QG_FMT_Q8A, QG_FMT_Q8A16 = 0, 1, 2, 3, 4

FMT = {"q4": QG_FMT_Q4, "q4a": QG_FMT_Q4A, "q8": QG_FMT_Q8, "q8a": QG_FMT_Q8A, "q8a16": QG_FMT_Q8A16}
MODE = {"exact": QG_EXACT, "fast": QG_FAST, "fast_wexact": QG_FAST_WEXACT}

# exported symbols of include/qgemm.h, in declaration order
SYMBOLS = [
    "qg_strerror", "qg_abi_version",
    "qgemm_q4", "qgemm_q4a", "qgemm_q8", "qgemm_q8a", "qgemm_q8a16", "qgemm_batch",
    "qgemv_q4", "qgemv_q4a", "qgemv_q8", "qgemv_q8a", "qgemv_q8a16",
    "qg_dequant_dump", "qg_repack_gguf", "qg_repack_gguf_q8a", "qg_repack_gguf_q8a16", "qg_repack_q8f", "qg_col_scale", "qg_conv_stats",
    "qg_conv2d",
    "qg_moe_plan_host", "qg_moe_plan", "qg_x_half", "qg_x_half_guard", "qgemm_moe_grouped", "qg_swiglu", "qg_moe_combine",
    "qg_moe_ffn_workspace", "qg_moe_ffn", "qg_moe_ffn_noalloc",
]


class QGError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


_lib = None
_p, _i, _sz = C.c_void_p, C.c_int, C.c_size_t


def lib() -> C.CDLL:
    """The loaded libqgemm.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                              f"g.build()'` (or block_quantized_weight_affine_amd/build.py)")
        L = C.CDLL(LIB_PATH)
        L.qg_strerror.restype = C.c_char_p
        L.qg_strerror.argtypes = [_i]
        L.qg_abi_version.restype = _i
        L.qg_abi_version.argtypes = []
        sig_dense = [_p, _p, _p, _i, _p, _i, _i, _i, _i, _p]
        L.qgemm_q4.argtypes = sig_dense
        L.qgemm_q8.argtypes = sig_dense
        L.qgemm_q4a.argtypes = [_p, _p, _p, _i, _p, _i, _p, _i, _i, _i, _i, _p]
        sig_gemv = [_p, _p, _p, _i, _p, _i, _i, _i, _p]
        L.qgemv_q4.argtypes = sig_gemv
        L.qgemv_q8.argtypes = sig_gemv
        L.qgemv_q4a.argtypes = [_p, _p, _p, _i, _p, _i, _p, _i, _i, _i, _p]
        L.qgemm_q8a.argtypes = [_p, _p, _p, _p, _i, _p, _i, _i, _i, _i, _p]
        L.qgemv_q8a.argtypes = [_p, _p, _p, _p, _i, _p, _i, _i, _i, _p]
        L.qg_repack_gguf_q8a.argtypes = [_i, _p, _i, _i, _p, _p, _p, _p]
        L.qgemm_q8a16.argtypes = [_p, _p, _p, _p, _i, _p, _i, _i, _i, _i, _p]
        L.qgemv_q8a16.argtypes = [_p, _p, _p, _p, _i, _p, _i, _i, _i, _p]
        L.qg_repack_gguf_q8a16.argtypes = [_i, _p, _i, _i, _p, _p, _p, _p]
        L.qg_repack_q8f.argtypes = [_p, _i, _i, _i, _p, _p, _p]
        L.qg_col_scale.argtypes = [_p, _i, _i, _i, _p, _p, _i, _p]
        L.qg_conv_stats.argtypes = [_p, _i, _i, _i, C.c_float, _p, _p]
        L.qg_conv2d.argtypes = [_i, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _p, _p, _i, _p, _i, _p]
        L.qg_dequant_dump.argtypes = [_i, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _p, _p]
        L.qg_moe_plan_host.argtypes = [_p, _i, _i, _i, _p, _p, _p, _p, _p]
        L.qg_repack_gguf.argtypes = [_i, _p, _i, _i, _p, _p, _p]
        L.qgemm_batch.argtypes = [_i, _i, _p, _i, _p, _i, _i, _i, _i, _p]
        L.qg_moe_plan.argtypes = [_p, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p]
        L.qg_x_half.argtypes = [_p, _i, _p, _i, _i, _p, _p, _p]
        L.qg_x_half_guard.argtypes = [_p, _i, _p, _i, _i, _i, _p, _p, _p]
        L.qgemm_moe_grouped.argtypes = [_i, _p, _i, _p, _p, _i, _p, _i, _p, _p, _i, _i, _i, _i, _i, _p]
        L.qg_swiglu.argtypes = [_p, _i, _i, _p, _i, _p, _p]
        L.qg_moe_combine.argtypes = [_p, _i, _p, _p, _p, _i, _i, _i, _i, _p]
        L.qg_moe_ffn_workspace.restype = _sz
        L.qg_moe_ffn_workspace.argtypes = [_i, _i, _i, _i, _i]
        L.qg_moe_ffn.argtypes = [_i, _p, _p, _i, _i, _i, _i, _p, _i, _i, _p, _p, _p, _p, _p, _i, _i, _p, _sz, _p]
        L.qg_moe_ffn_noalloc.argtypes = [_i, _p, _p, _i, _i, _i, _i, _p, _i, _i, _p, _p, _p, _p, _p, _i, _i, _p]
        for name in SYMBOLS:
            if name not in ("qg_strerror", "qg_abi_version", "qg_moe_ffn_workspace"):
                getattr(L, name).restype = _i
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().qg_strerror(int(status)).decode()


def abi_version() -> int:
    return lib().qg_abi_version()


# ---- marshalling helpers ------------------------------------------------------------------------
def _ptr(t):
    """Device (or host) address of a torch tensor / numpy array / int; None for None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _xt(t) -> int:
    import torch
    return {torch.float32: QG_X_F32, torch.float16: QG_X_F16, torch.bfloat16: QG_X_BF16}[t.dtype]


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != QG_OK:
        raise QGError(status, where)


def _mode(mode):
    return MODE[mode] if isinstance(mode, str) else int(mode)


# ---- dense matmuls ------------------------------------------------------------------------------
def qgemm_q4(codes, scales, X, Y, N, K, T, mode="exact", xt=None, stream=None):
    _check(lib().qgemm_q4(_ptr(codes), _ptr(scales), _ptr(X), _xt(X) if xt is None else xt, _ptr(Y), N, K, T,
                          _mode(mode), _stream(stream)), "qgemm_q4")


def qgemm_q4a(codes, scales, offsets, group, X, Y, N, K, T, mode="exact", xt=None, stream=None):
    _check(lib().qgemm_q4a(_ptr(codes), _ptr(scales), _ptr(offsets), group, _ptr(X), _xt(X) if xt is None else xt,
                           _ptr(Y), N, K, T, _mode(mode), _stream(stream)), "qgemm_q4a")


def qgemm_q8(codes, scales, X, Y, N, K, T, mode="exact", xt=None, stream=None):
    _check(lib().qgemm_q8(_ptr(codes), _ptr(scales), _ptr(X), _xt(X) if xt is None else xt, _ptr(Y), N, K, T,
                          _mode(mode), _stream(stream)), "qgemm_q8")


def qgemm_q8a(codes, scales, offsets, X, Y, N, K, T, mode="exact", xt=None, stream=None):
    _check(lib().qgemm_q8a(_ptr(codes), _ptr(scales), _ptr(offsets), _ptr(X), _xt(X) if xt is None else xt,
                           _ptr(Y), N, K, T, _mode(mode), _stream(stream)), "qgemm_q8a")


def qgemv_q4(codes, scales, X, Y, N, K, T, xt=None, stream=None):
    _check(lib().qgemv_q4(_ptr(codes), _ptr(scales), _ptr(X), _xt(X) if xt is None else xt, _ptr(Y), N, K, T,
                          _stream(stream)), "qgemv_q4")


def qgemv_q4a(codes, scales, offsets, group, X, Y, N, K, T, xt=None, stream=None):
    _check(lib().qgemv_q4a(_ptr(codes), _ptr(scales), _ptr(offsets), group, _ptr(X), _xt(X) if xt is None else xt,
                           _ptr(Y), N, K, T, _stream(stream)), "qgemv_q4a")


def qgemv_q8(codes, scales, X, Y, N, K, T, xt=None, stream=None):
    _check(lib().qgemv_q8(_ptr(codes), _ptr(scales), _ptr(X), _xt(X) if xt is None else xt, _ptr(Y), N, K, T,
                          _stream(stream)), "qgemv_q8")


def qgemm_q8a16(codes, scales, offsets, X, Y, N, K, T, mode="exact", xt=None, stream=None):
    _check(lib().qgemm_q8a16(_ptr(codes), _ptr(scales), _ptr(offsets), _ptr(X), _xt(X) if xt is None else xt,
                             _ptr(Y), N, K, T, _mode(mode), _stream(stream)), "qgemm_q8a16")


def qgemv_q8a16(codes, scales, offsets, X, Y, N, K, T, xt=None, stream=None):
    _check(lib().qgemv_q8a16(_ptr(codes), _ptr(scales), _ptr(offsets), _ptr(X), _xt(X) if xt is None else xt,
                             _ptr(Y), N, K, T, _stream(stream)), "qgemv_q8a16")


def qgemv_q8a(codes, scales, offsets, X, Y, N, K, T, xt=None, stream=None):
    _check(lib().qgemv_q8a(_ptr(codes), _ptr(scales), _ptr(offsets), _ptr(X), _xt(X) if xt is None else xt,
                           _ptr(Y), N, K, T, _stream(stream)), "qgemv_q8a")


def qgemm(fmt, codes, scales, offsets, group, X, Y, N, K, T, mode="exact", stream=None):
    """Dispatch by format name: 'q4' | 'q4a' | 'q8' | 'q8a' | 'q8a16'."""
    if fmt == "q8a16":
        return qgemm_q8a16(codes, scales, offsets, X, Y, N, K, T, mode, stream=stream)
    if fmt == "q4":
        return qgemm_q4(codes, scales, X, Y, N, K, T, mode, stream=stream)
    if fmt == "q4a":
        return qgemm_q4a(codes, scales, offsets, group, X, Y, N, K, T, mode, stream=stream)
    if fmt == "q8a":
        return qgemm_q8a(codes, scales, offsets, X, Y, N, K, T, mode, stream=stream)
    return qgemm_q8(codes, scales, X, Y, N, K, T, mode, stream=stream)


def qgemv(fmt, codes, scales, offsets, group, X, Y, N, K, T, stream=None):
    if fmt == "q8a16":
        return qgemv_q8a16(codes, scales, offsets, X, Y, N, K, T, stream=stream)
    if fmt == "q4":
        return qgemv_q4(codes, scales, X, Y, N, K, T, stream=stream)
    if fmt == "q4a":
        return qgemv_q4a(codes, scales, offsets, group, X, Y, N, K, T, stream=stream)
    if fmt == "q8a":
        return qgemv_q8a(codes, scales, offsets, X, Y, N, K, T, stream=stream)
    return qgemv_q8(codes, scales, X, Y, N, K, T, stream=stream)


def qg_dequant_dump(fmt, codes, scales, offsets, group, N, K, n0, k0, rows, cols, staged, out, stream=None):
    _check(lib().qg_dequant_dump(FMT[fmt] if isinstance(fmt, str) else fmt, _ptr(codes), _ptr(scales),
                                 _ptr(offsets), group, N, K, n0, k0, rows, cols, staged, _ptr(out),
                                 _stream(stream)), "qg_dequant_dump")


class QgJob(C.Structure):
    """qg_job of qgemm.h: one weight matrix of a batched call."""
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("offsets", C.c_void_p), ("Y", C.c_void_p),
                ("N", C.c_int)]


def job_array(jobs):
    """Host array of qg_job from (codes, scales, offsets-or-None, Y, N) tuples of device tensors."""
    arr = (QgJob * len(jobs))()
    for i, (c, s, o, y, n) in enumerate(jobs):
        arr[i] = QgJob(_ptr(c), _ptr(s), _ptr(o), _ptr(y), int(n))
    return arr


def qgemm_batch(fmt, group, jobs, X, K, T, mode="exact", xt=None, stream=None):
    """jobs: list of (codes, scales, offsets-or-None, Y, N) sharing X [T][K]."""
    arr = job_array(jobs)
    _check(lib().qgemm_batch(FMT[fmt] if isinstance(fmt, str) else fmt, group, C.cast(arr, C.c_void_p), len(jobs),
                             _ptr(X), _xt(X) if xt is None else xt, K, T, _mode(mode), _stream(stream)), "qgemm_batch")


QG_GGUF_Q4_0, QG_GGUF_Q4_1, QG_GGUF_Q5_0, QG_GGUF_Q5_1, QG_GGUF_Q8_0, QG_GGUF_Q4_K, QG_GGUF_Q5_K = 2, 3, 6, 7, 8, 12, 13
QG_GGUF_Q2_K, QG_GGUF_Q3_K, QG_GGUF_Q6_K = 10, 11, 14
GGUF = {"q4_0": QG_GGUF_Q4_0, "q4_1": QG_GGUF_Q4_1, "q5_0": QG_GGUF_Q5_0, "q5_1": QG_GGUF_Q5_1,
        "q8_0": QG_GGUF_Q8_0, "q4_k": QG_GGUF_Q4_K, "q5_k": QG_GGUF_Q5_K, "q2_k": QG_GGUF_Q2_K,
        "q3_k": QG_GGUF_Q3_K, "q6_k": QG_GGUF_Q6_K}


def qg_repack_gguf(gtype, src, N, K, codes, scales, stream=None):
    """GGUF Q4_0 / Q8_0 blocks (device uint8 tensor) -> this library's codes and scales (device)."""
    _check(lib().qg_repack_gguf(GGUF[gtype] if isinstance(gtype, str) else gtype, _ptr(src), N, K, _ptr(codes),
                                _ptr(scales), _stream(stream)), "qg_repack_gguf")


def qg_repack_gguf_q8a(gtype, src, N, K, codes, scales, offsets, stream=None):
    """GGUF Q4_1 / Q5_0 / Q5_1 / Q4_K / Q5_K blocks (device uint8 tensor) -> Q8A codes (int8 [N*K]), f32
    scales and f32 offsets ([N*K/32]), all device tensors."""
    _check(lib().qg_repack_gguf_q8a(GGUF[gtype] if isinstance(gtype, str) else gtype, _ptr(src), N, K,
                                    _ptr(codes), _ptr(scales), _ptr(offsets), _stream(stream)),
           "qg_repack_gguf_q8a")


def qg_repack_q8f(blob, N, K, has_col, scales, col=None, stream=None):
    """q8_2f (has_col) / q8_row tensor blob (device uint8: int8 codes [N][K], f16 row scales, f16 column
    field) -> f32 Q8 block scales [N*K/32] and the f32 column field [K]; the blob is the Q8 codes."""
    _check(lib().qg_repack_q8f(_ptr(blob), N, K, int(bool(has_col)), _ptr(scales), _ptr(col), _stream(stream)),
           "qg_repack_q8f")


def qg_col_scale(X, T, K, col, Xs, stream=None):
    """Xs = X * col[k] (types from the tensors' dtypes)."""
    _check(lib().qg_col_scale(_ptr(X), _xt(X), T, K, _ptr(col), _ptr(Xs), _xt(Xs), _stream(stream)), "qg_col_scale")


# ---- convolution ------------------------------------------------------------------------------------
CONV_NORM = {None: 0, "none": 0, "group": 1, "layer": 2}


def conv_out_size(H, W, ksize, stride):
    """(oh, ow) of qg_conv2d: pad = ksize // 2."""
    pad = ksize // 2
    return (H + 2 * pad - ksize) // stride + 1, (W + 2 * pad - ksize) // stride + 1


def qg_conv_stats(X, npix, cin, groups, eps, stats, stream=None):
    """(mean, rstd) f32 pairs of the image X [npix][cin] into stats (device): per group of
    cin / groups channels (groups > 0) or per pixel (groups == 0)."""
    _check(lib().qg_conv_stats(_ptr(X), npix, cin, groups, float(eps), _ptr(stats), _stream(stream)),
           "qg_conv_stats")


def qg_conv2d(fmt, codes, scales, X, H, W, cin, ksize, stride, n_out, Y, norm=None, groups=0, stats=None,
              gamma_beta=None, silu=False, mode="exact", stream=None):
    """Implicit-GEMM convolution of the image X [H][W][cin] (f32) with the quantized weight matrix
    [n_out][ksize * ksize * cin] into Y [oh * ow][n_out] (device tensors)."""
    _check(lib().qg_conv2d(FMT[fmt] if isinstance(fmt, str) else fmt, _ptr(codes), _ptr(scales), _ptr(X), H, W, cin,
                           ksize, stride, n_out, CONV_NORM[norm] if not isinstance(norm, int) else norm, groups,
                           _ptr(stats), _ptr(gamma_beta), int(bool(silu)), _ptr(Y), _mode(mode), _stream(stream)),
           "qg_conv2d")


# ---- MoE ----------------------------------------------------------------------------------------
def qg_moe_plan_host(logits: np.ndarray, T: int, E: int, k: int) -> dict:
    """Routing plan on the host (numpy in, numpy out)."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    seg_off = np.empty(E + 1, np.int32)
    row_src = np.empty(T * k, np.int32)
    slot_row = np.empty(T * k, np.int32)
    slot_w = np.empty(T * k, np.float32)
    slot_e = np.empty(T * k, np.int32)
    _check(lib().qg_moe_plan_host(_ptr(lg), T, E, k, _ptr(seg_off), _ptr(row_src), _ptr(slot_row), _ptr(slot_w),
                                  _ptr(slot_e)), "qg_moe_plan_host")
    return {"seg_off": seg_off, "row_src": row_src, "slot_row": slot_row, "slot_w": slot_w, "slot_expert": slot_e}


def qg_moe_plan(logits, T, E, k, seg_off, row_src, slot_row, slot_w, slot_expert=None, status=None, stream=None):
    """Routing plan on the device: every argument a device tensor (int32 / float32) or None."""
    _check(lib().qg_moe_plan(_ptr(logits), T, E, k, _ptr(seg_off), _ptr(row_src), _ptr(slot_row), _ptr(slot_w),
                             _ptr(slot_expert), _ptr(status), _stream(stream)), "qg_moe_plan")


def qg_x_half(X, x_rows, row_src, R, K, Xh, rs, stream=None):
    _check(lib().qg_x_half(_ptr(X), x_rows, _ptr(row_src), R, K, _ptr(Xh), _ptr(rs), _stream(stream)), "qg_x_half")


def qg_x_half_guard(X, x_rows, row_src, R, K, shift, Xh, rs=None, stream=None):
    _check(lib().qg_x_half_guard(_ptr(X), x_rows, _ptr(row_src), R, K, int(shift), _ptr(Xh), _ptr(rs), _stream(stream)),
           "qg_x_half_guard")


def qgemm_moe_grouped(fmt, experts, group, seg_off, row_src, x_rows, X, rs, Y, N, K, R, E, mode="exact", xt=None,
                      stream=None):
    _check(lib().qgemm_moe_grouped(FMT[fmt] if isinstance(fmt, str) else fmt, _ptr(experts), group, _ptr(seg_off),
                                   _ptr(row_src), x_rows, _ptr(X), _xt(X) if xt is None else xt, _ptr(rs), _ptr(Y),
                                   N, K, R, E, _mode(mode), _stream(stream)), "qgemm_moe_grouped")


def qg_swiglu(GU, R, I, A, at, rs=None, stream=None):
    _check(lib().qg_swiglu(_ptr(GU), R, I, _ptr(A), at, _ptr(rs), _stream(stream)), "qg_swiglu")


def qg_moe_combine(O, R, slot_row, slot_w, Y, H, T, k, accumulate=0, stream=None):
    _check(lib().qg_moe_combine(_ptr(O), R, _ptr(slot_row), _ptr(slot_w), _ptr(Y), H, T, k, int(accumulate),
                                _stream(stream)), "qg_moe_combine")


def qg_moe_ffn_workspace(H, I, T, k, mode="exact") -> int:
    return int(lib().qg_moe_ffn_workspace(H, I, T, k, _mode(mode)))


def qg_moe_ffn(fmt, gate_up, down, group, E, H, I, X, T, k, seg_off, row_src, slot_row, slot_w, Y, accumulate,
               mode, workspace, ws_bytes, stream=None):
    _check(lib().qg_moe_ffn(FMT[fmt] if isinstance(fmt, str) else fmt, _ptr(gate_up), _ptr(down), group, E, H, I,
                            _ptr(X), T, k, _ptr(seg_off), _ptr(row_src), _ptr(slot_row), _ptr(slot_w), _ptr(Y),
                            int(accumulate), _mode(mode), _ptr(workspace), int(ws_bytes), _stream(stream)),
           "qg_moe_ffn")


def qg_moe_ffn_noalloc(fmt, gate_up, down, group, E, H, I, X, T, k, seg_off, row_src, slot_row, slot_w, Y,
                       accumulate, mode, stream=None):
    _check(lib().qg_moe_ffn_noalloc(FMT[fmt] if isinstance(fmt, str) else fmt, _ptr(gate_up), _ptr(down), group, E, H,
                                    I, _ptr(X), T, k, _ptr(seg_off), _ptr(row_src), _ptr(slot_row), _ptr(slot_w),
                                    _ptr(Y), int(accumulate), _mode(mode), _stream(stream)),
           "qg_moe_ffn_noalloc")


# ---- host layout helpers (byte movement only) ----------------------------------------------------
def pack_q4(nibbles: np.ndarray) -> np.ndarray:
    """Nibble matrix [N][K] (values 0..15, element order) -> packed Q4 codes uint8 [N][K/2] in the
    block layout: byte j of block b holds element 32b+j (low nibble) and 32b+16+j (high nibble)."""
    nb = np.asarray(nibbles, dtype=np.uint8)
    N, K = nb.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    if nb.max(initial=0) > 15:
        raise ValueError("nibbles must be in 0..15")
    b = nb.reshape(N, K // 32, 32)
    return (b[:, :, :16] | (b[:, :, 16:] << 4)).reshape(N, K // 2)


def unpack_q4(codes: np.ndarray, N: int, K: int) -> np.ndarray:
    """Inverse of pack_q4: packed codes -> nibble matrix [N][K]."""
    c = np.asarray(codes, dtype=np.uint8).reshape(N, K // 32, 16)
    return np.concatenate([c & 15, c >> 4], axis=2).reshape(N, K)


def expert_table(experts, device="cuda"):
    """Device array of qg_expert {codes, scales, offsets} (three 64-bit pointers each) for a list of
    (codes, scales, offsets-or-None) device tensors."""
    import torch
    rows = [[_ptr(c), _ptr(s), _ptr(o) if o is not None else 0] for (c, s, o) in experts]
    host = torch.tensor(np.array(rows, dtype=np.uint64).view(np.int64), dtype=torch.int64)
    return host.to(device)


def qg_repack_gguf_q8a16(gtype, src, N, K, codes, scales, offsets, stream=None):
    """GGUF Q6_K / Q3_K / Q2_K super-blocks (device uint8 tensor) -> Q8A16 codes (int8 [N*K]), f32 scales
    and f32 offsets ([N*K/16]; None for the offset-free Q6_K / Q3_K layout), all device tensors."""
    _check(lib().qg_repack_gguf_q8a16(GGUF[gtype] if isinstance(gtype, str) else gtype, _ptr(src), N, K,
                                      _ptr(codes), _ptr(scales), _ptr(offsets), _stream(stream)),
           "qg_repack_gguf_q8a16")
