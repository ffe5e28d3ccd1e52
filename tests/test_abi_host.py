"""CPU checks of the C ABI: the library loads, exports every function include/qgemm.h declares,
rejects bad arguments with the documented codes before any HIP call, and its host routing planner
and packing helpers agree with the oracle.  Nothing here launches a kernel."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import block_quantized_weight_affine_amd as qg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "qgemm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^\s*(?:const\s+char\s*\*|int|qg_status|size_t)\s+(\w+)\s*\(", src, flags=re.M)


def test_exports_every_declared_symbol():
    L = qg.lib()
    names = _declared()
    assert set(names) == set(qg.SYMBOLS), (names, qg.SYMBOLS)
    for n in names:
        assert hasattr(L, n), n
    assert qg.abi_version() == 1
    for s in range(9):
        assert qg.strerror(s)


# fake, never-dereferenced addresses: validation runs entirely on the host
A16 = 0x10000
A16b = 0x20000
A16c = 0x30000
A16d = 0x40000


def _q4(**kw):
    a = dict(codes=A16, scales=A16b, X=A16c, xt=qg.QG_X_F32, Y=A16d, N=256, K=512, T=16, mode=qg.QG_EXACT)
    a.update(kw)
    return qg.lib().qgemm_q4(a["codes"], a["scales"], a["X"], a["xt"], a["Y"], a["N"], a["K"], a["T"], a["mode"], None)


def test_dense_validation_codes():
    assert _q4(K=48) == qg.QG_ESHAPE            # K % 32
    assert _q4(K=16) == qg.QG_ESHAPE
    assert _q4(N=0) == qg.QG_ESHAPE
    assert _q4(T=-1) == qg.QG_ESHAPE
    assert _q4(codes=None) == qg.QG_EINVAL
    assert _q4(Y=None) == qg.QG_EINVAL
    assert _q4(xt=7) == qg.QG_EINVAL
    assert _q4(mode=5) == qg.QG_EINVAL
    assert _q4(codes=A16 + 8) == qg.QG_EALIGN
    assert _q4(X=A16c + 4) == qg.QG_EALIGN
    assert _q4(scales=A16b + 1) == qg.QG_EALIGN
    assert _q4(T=0) == qg.QG_OK                 # nothing to do, nothing launched
    assert _q4(T=0, codes=None) == qg.QG_OK
    assert _q4(T=16, mode=qg.QG_FAST, xt=qg.QG_X_F32) == qg.QG_EUNSUPPORTED
    L = qg.lib()
    # affine: group must be a multiple of 32 dividing K, offsets required
    assert L.qgemm_q4a(A16, A16b, A16, 48, A16c, 0, A16d, 256, 512, 16, 0, None) == qg.QG_ESHAPE
    assert L.qgemm_q4a(A16, A16b, A16, 96, A16c, 0, A16d, 256, 512, 16, 0, None) == qg.QG_ESHAPE
    assert L.qgemm_q4a(A16, A16b, None, 64, A16c, 0, A16d, 256, 512, 16, 0, None) == qg.QG_EINVAL
    # q8 scales are f32: 4-byte alignment
    assert L.qgemm_q8(A16, A16b + 2, A16c, 0, A16d, 256, 512, 16, 0, None) == qg.QG_EALIGN
    # the W-exact fast mode: Q4 and Q8 codes with f16 X only; not for grouped matmuls or the block
    assert L.qgemm_q4a(A16, A16b, A16, 64, A16c, 1, A16d, 256, 512, 16, qg.QG_FAST_WEXACT, None) == \
        qg.QG_EUNSUPPORTED
    assert L.qgemm_q8(A16, A16b, A16c, 0, A16d, 256, 512, 16, qg.QG_FAST_WEXACT, None) == qg.QG_EUNSUPPORTED
    assert L.qgemm_q8(A16, A16b, A16c, 2, A16d, 256, 512, 16, qg.QG_FAST_WEXACT, None) == qg.QG_EUNSUPPORTED
    assert L.qgemm_q4(A16, A16b, A16c, 1, A16d, 256, 512, 0, qg.QG_FAST_WEXACT, None) == qg.QG_OK
    assert L.qgemm_q4(A16, A16b, A16c, 1, A16d, 256, 512, 16, 3, None) == qg.QG_EINVAL
    assert L.qgemm_moe_grouped(0, A16, 64, A16b, None, 8, A16c, 1, None, A16d, 256, 512, 8, 4,
                               qg.QG_FAST_WEXACT, None) == qg.QG_EUNSUPPORTED
    # GEMV takes at most 8 rows
    assert L.qgemv_q8(A16, A16b, A16c, 0, A16d, 256, 512, 9, None) == qg.QG_ESHAPE
    assert L.qgemv_q4(A16, A16b, A16c, 0, A16d, 256, 512, 0, None) == qg.QG_OK


def test_dump_and_moe_validation_codes():
    L = qg.lib()
    # dump: tile must be inside the matrix, block aligned
    assert L.qg_dequant_dump(0, A16, A16b, None, 64, 64, 128, 0, 16, 4, 32, 0, A16c, None) == qg.QG_ESHAPE
    assert L.qg_dequant_dump(0, A16, A16b, None, 64, 64, 128, 60, 0, 8, 32, 0, A16c, None) == qg.QG_ESHAPE
    assert L.qg_dequant_dump(0, A16, A16b, None, 64, 64, 128, 0, 96, 1, 64, 0, A16c, None) == qg.QG_ESHAPE
    assert L.qg_dequant_dump(3, A16, A16b, None, 64, 64, 128, 0, 0, 1, 32, 0, A16c, None) == qg.QG_EINVAL
    # grouped: fast mode with f32 X only where the expert-row kernel scales the rows itself (K <= 2048
    # for Q4 / Q4A, 1024 for Q8); E >= 1
    assert L.qgemm_moe_grouped(0, A16, 64, A16b, None, 8, A16c, 0, None, A16d, 256, 2080, 8, 4, 1, None) == \
        qg.QG_EUNSUPPORTED
    assert L.qgemm_moe_grouped(2, A16, 64, A16b, None, 8, A16c, 0, None, A16d, 256, 1056, 8, 4, 1, None) == \
        qg.QG_EUNSUPPORTED
    assert L.qgemm_moe_grouped(0, A16, 64, A16b, None, 8, A16c, 0, None, A16d, 256, 512, 0, 4, 1, None) == qg.QG_OK
    assert L.qgemm_moe_grouped(0, A16, 64, A16b, None, 8, A16c, 1, None, A16d, 256, 512, 8, 0, 1, None) == \
        qg.QG_ESHAPE
    assert L.qgemm_moe_grouped(0, None, 64, A16b, None, 8, A16c, 1, None, A16d, 256, 512, 8, 4, 1, None) == \
        qg.QG_EINVAL
    assert L.qgemm_moe_grouped(0, A16 + 4, 64, A16b, None, 8, A16c, 1, None, A16d, 256, 512, 8, 4, 1, None) == \
        qg.QG_EALIGN
    assert L.qgemm_moe_grouped(0, A16, 64, A16b, None, 8, A16c, 1, None, A16d, 256, 512, 0, 4, 1, None) == qg.QG_OK
    assert L.qg_swiglu(A16, 4, 12, A16b, 0, None, None) == qg.QG_ESHAPE
    assert L.qg_swiglu(A16, 4, 16, A16b, 2, None, None) == qg.QG_EUNSUPPORTED
    assert L.qg_swiglu(A16, 4, 16, A16b, 1, None, None) == qg.QG_EINVAL
    assert L.qg_moe_combine(A16, 8, A16b, A16c, A16d, 6, 2, 2, 0, None) == qg.QG_ESHAPE
    assert L.qg_moe_combine(A16, 8, A16b, A16c, A16d + 8, 8, 2, 2, 0, None) == qg.QG_EALIGN
    assert L.qg_x_half(A16, 4, None, 4, 12, A16b, A16c, None) == qg.QG_ESHAPE
    assert L.qg_x_half_guard(A16, 4, None, 4, 16, 15, A16b, A16c, None) == qg.QG_EINVAL
    assert L.qg_x_half_guard(A16, 4, None, 4, 16, -1, A16b, A16c, None) == qg.QG_EINVAL
    assert L.qg_x_half_guard(A16, 4, None, 4, 12, 4, A16b, A16c, None) == qg.QG_ESHAPE
    assert L.qg_x_half_guard(A16, 4, None, 4, 16, 4, A16b + 8, None, None) == qg.QG_EALIGN
    assert L.qg_x_half_guard(None, 4, None, 4, 16, 4, A16b, None, None) == qg.QG_EINVAL
    assert L.qg_x_half_guard(None, 4, None, 0, 16, 4, None, None, None) == qg.QG_OK
    ws = qg.qg_moe_ffn_workspace(2048, 1536, 32, 8, "fast")
    assert ws >= 256 * (3072 * 4 + 2048 * 4 + 2048 * 2 + 1536 * 2)
    assert L.qg_moe_ffn(0, A16, A16b, 64, 128, 2048, 1536, A16c, 32, 8, A16d, A16d, A16d, A16d, A16d, 0, 1,
                        0x100000, ws - 1, None) == qg.QG_EWORKSPACE
    assert L.qg_moe_ffn(0, A16, A16b, 64, 128, 2048, 1536, A16c, 32, 8, A16d, A16d, A16d, A16d, A16d, 0, 1,
                        0x100010, ws, None) == qg.QG_EALIGN
    assert L.qg_moe_ffn(0, A16, A16b, 64, 128, 2048, 1536, A16c, 32, 8, A16d, A16d, A16d, A16d, A16d, 0,
                        qg.QG_FAST_WEXACT, 0x100000, ws, None) == qg.QG_EUNSUPPORTED


def test_batch_validation_codes():
    """qgemm_batch validates every job (with the dense entry points' codes) before any launch."""
    L = qg.lib()

    def call(jobs, J=None, T=1, mode=qg.QG_EXACT, xt=qg.QG_X_F32, K=256):
        arr = qg.job_array(jobs) if jobs is not None else None
        ptr = None if arr is None else __import__("ctypes").cast(arr, __import__("ctypes").c_void_p)
        return L.qgemm_batch(qg.QG_FMT_Q4, 64, ptr, len(jobs) if J is None else J, A16c, xt, K, T, mode, None)

    good = (A16, A16b, None, A16d, 64)
    assert call(None, J=1) == qg.QG_EINVAL
    assert call([good], J=0) == qg.QG_ESHAPE
    assert call([good] * 65) == qg.QG_ESHAPE
    assert call([good, (A16, A16b, None, A16d, 0)]) == qg.QG_ESHAPE            # N = 0 in job 1
    assert call([good, good, (A16 + 8, A16b, None, A16d, 64)]) == qg.QG_EALIGN  # codes of job 2
    assert call([good, (None, A16b, None, A16d, 64)]) == qg.QG_EINVAL
    assert call([good], K=48) == qg.QG_ESHAPE
    assert call([good], T=16, mode=qg.QG_FAST) == qg.QG_EUNSUPPORTED          # f32 X in fast mode, T > 8
    assert call([good], T=0) == qg.QG_OK                                        # nothing to do


def test_repack_gguf_validation_codes():
    """qg_repack_gguf checks type, sizes, pointers and alignment on the host, before any HIP call."""
    L = qg.lib()

    def call(t=qg.QG_GGUF_Q4_0, src=A16, N=8, K=256, codes=A16b, scales=A16c):
        return L.qg_repack_gguf(t, src, N, K, codes, scales, None)

    assert call(t=3) == qg.QG_EINVAL
    assert call(N=0) == qg.QG_ESHAPE
    assert call(K=48) == qg.QG_ESHAPE
    assert call(K=0) == qg.QG_ESHAPE
    assert call(src=None) == qg.QG_EINVAL
    assert call(scales=None) == qg.QG_EINVAL
    assert call(src=A16 + 1) == qg.QG_EALIGN
    assert call(codes=A16b + 8) == qg.QG_EALIGN
    assert call(t=qg.QG_GGUF_Q8_0, scales=A16c + 2) == qg.QG_EALIGN


def test_q8f_validation_codes():
    """q8_2f / q8_row repack and the column-field step: sizes, pointers and alignment are checked
    before any launch (no GPU needed for a rejected call)."""
    L = qg.lib()
    assert L.qg_repack_q8f(A16, 64, 48, 1, A16b, A16c, None) == qg.QG_ESHAPE
    assert L.qg_repack_q8f(A16, 0, 64, 1, A16b, A16c, None) == qg.QG_ESHAPE
    assert L.qg_repack_q8f(None, 64, 64, 1, A16b, A16c, None) == qg.QG_EINVAL
    assert L.qg_repack_q8f(A16, 64, 64, 1, A16b, None, None) == qg.QG_EINVAL
    assert L.qg_repack_q8f(A16 + 8, 64, 64, 0, A16b, None, None) == qg.QG_EALIGN
    assert L.qg_repack_q8f(A16, 64, 64, 1, A16b, A16c + 4, None) == qg.QG_EALIGN
    assert L.qg_col_scale(A16, 0, 4, 12, A16b, A16c, 1, None) == qg.QG_ESHAPE
    assert L.qg_col_scale(A16, 3, 4, 16, A16b, A16c, 1, None) == qg.QG_EINVAL
    assert L.qg_col_scale(A16, 0, 4, 16, A16b, A16c, 5, None) == qg.QG_EINVAL
    assert L.qg_col_scale(A16, 0, 4, 16, A16b + 4, A16c, 1, None) == qg.QG_EALIGN
    assert L.qg_col_scale(A16, 0, 4, 16, None, A16c, 1, None) == qg.QG_EINVAL
    assert L.qg_col_scale(None, 0, 0, 16, None, None, 1, None) == qg.QG_OK


def test_q8a_validation_codes():
    """Q8A: offsets required and 4-byte aligned (f32), W-exact unsupported, no grouped or expert-block
    calls; the GGUF -> Q8A repack checks type, sizes, pointers and alignment."""
    L = qg.lib()

    def gemm(codes=A16, scales=A16b, offs=A16, xt=qg.QG_X_F32, T=16, mode=qg.QG_EXACT):
        return L.qgemm_q8a(codes, scales, offs, A16c, xt, A16d, 256, 512, T, mode, None)

    assert gemm(offs=None) == qg.QG_EINVAL
    assert gemm(offs=A16 + 2) == qg.QG_EALIGN
    assert gemm(scales=A16b + 2) == qg.QG_EALIGN
    assert gemm(codes=A16 + 4) == qg.QG_EALIGN
    assert gemm(T=0, offs=None) == qg.QG_OK
    assert gemm(xt=qg.QG_X_F16, mode=qg.QG_FAST_WEXACT) == qg.QG_EUNSUPPORTED
    assert gemm(xt=qg.QG_X_F32, mode=qg.QG_FAST) == qg.QG_EUNSUPPORTED
    assert L.qgemv_q8a(A16, A16b, A16, A16c, 0, A16d, 256, 512, 9, None) == qg.QG_ESHAPE
    assert L.qgemv_q8a(A16, A16b, None, A16c, 0, A16d, 256, 512, 1, None) == qg.QG_EINVAL
    assert L.qg_dequant_dump(qg.QG_FMT_Q8A, A16, A16b, A16 + 2, 64, 64, 256, 0, 0, 8, 64, 0, A16c, None) == \
        qg.QG_EALIGN
    assert L.qg_dequant_dump(qg.QG_FMT_Q8A, A16, A16b, None, 64, 64, 256, 0, 0, 8, 64, 0, A16c, None) == \
        qg.QG_EINVAL
    assert L.qgemm_moe_grouped(qg.QG_FMT_Q8A, A16, 64, A16b, None, 8, A16c, 0, None, A16d, 256, 512, 8, 4,
                               qg.QG_EXACT, None) == qg.QG_EUNSUPPORTED
    assert L.qg_moe_ffn(qg.QG_FMT_Q8A, A16, A16b, 64, 4, 256, 256, A16c, 2, 2, A16, A16, A16, A16, A16d, 0,
                        qg.QG_EXACT, A16, 0x1000000, None) == qg.QG_EUNSUPPORTED

    def rep(t=qg.QG_GGUF_Q4_K, src=A16, N=8, K=512, codes=A16b, scales=A16c, offs=A16d):
        return L.qg_repack_gguf_q8a(t, src, N, K, codes, scales, offs, None)

    assert rep(t=qg.QG_GGUF_Q4_0) == qg.QG_EINVAL     # not an affine type
    assert rep(t=qg.QG_GGUF_Q8_0) == qg.QG_EINVAL
    assert rep(t=5) == qg.QG_EINVAL
    assert rep(K=288) == qg.QG_ESHAPE                 # Q4_K needs K % 256 == 0
    assert rep(t=qg.QG_GGUF_Q5_K, K=288) == qg.QG_ESHAPE
    assert rep(N=0) == qg.QG_ESHAPE
    assert rep(t=qg.QG_GGUF_Q4_1, K=48) == qg.QG_ESHAPE
    assert rep(offs=None) == qg.QG_EINVAL
    assert rep(src=None) == qg.QG_EINVAL
    assert rep(src=A16 + 1) == qg.QG_EALIGN
    assert rep(codes=A16b + 8) == qg.QG_EALIGN
    assert rep(scales=A16c + 2) == qg.QG_EALIGN
    assert rep(offs=A16d + 2) == qg.QG_EALIGN


def test_q8a16_validation_codes():
    """Q8A16: offsets optional but aligned, W-exact unsupported, no batched, grouped or convolution call;
    the GGUF -> Q8A16 repack checks type, sizes (K % 256), pointers and alignment."""
    L = qg.lib()

    def gemm(codes=A16, scales=A16b, offs=A16, xt=qg.QG_X_F32, T=16, mode=qg.QG_EXACT):
        return L.qgemm_q8a16(codes, scales, offs, A16c, xt, A16d, 256, 512, T, mode, None)

    # offsets are optional (NULL: no offset term); only present ones are checked
    assert gemm(offs=A16 + 2) == qg.QG_EALIGN
    assert gemm(offs=None, scales=A16b + 2) == qg.QG_EALIGN
    assert gemm(scales=A16b + 2) == qg.QG_EALIGN
    assert gemm(codes=A16 + 4) == qg.QG_EALIGN
    assert gemm(T=0, offs=None) == qg.QG_OK
    assert gemm(xt=qg.QG_X_F16, mode=qg.QG_FAST_WEXACT) == qg.QG_EUNSUPPORTED
    assert L.qgemv_q8a16(A16, A16b, A16, A16c, 0, A16d, 256, 512, 9, None) == qg.QG_ESHAPE
    assert L.qgemv_q8a16(A16, None, None, A16c, 0, A16d, 256, 512, 1, None) == qg.QG_EINVAL
    jobs = qg.job_array([(A16, A16b, A16, A16d, 64)])
    assert L.qgemm_batch(qg.QG_FMT_Q8A16, 64, C.cast(jobs, C.c_void_p), 1, A16c, 0, 512, 2, qg.QG_EXACT,
                         None) == qg.QG_EUNSUPPORTED
    assert L.qg_dequant_dump(qg.QG_FMT_Q8A16, A16, A16b, A16 + 2, 64, 64, 256, 0, 0, 8, 64, 1, A16c, None) == \
        qg.QG_EALIGN
    assert L.qgemm_moe_grouped(qg.QG_FMT_Q8A16, A16, 64, A16b, None, 8, A16c, 0, None, A16d, 256, 512, 8, 4,
                               qg.QG_EXACT, None) == qg.QG_EUNSUPPORTED
    assert L.qg_conv2d(qg.QG_FMT_Q8A16, A16, A16b, A16c, 8, 8, 32, 3, 1, 64, 0, 0, None, None, 0, A16d,
                       qg.QG_EXACT, None) == qg.QG_EUNSUPPORTED

    def rep(t=qg.QG_GGUF_Q6_K, src=A16, N=8, K=512, codes=A16b, scales=A16c, offs=A16d):
        return L.qg_repack_gguf_q8a16(t, src, N, K, codes, scales, offs, None)

    assert rep(t=qg.QG_GGUF_Q4_K) == qg.QG_EINVAL     # a 32-element-scale type
    assert rep(t=qg.QG_GGUF_Q8_0) == qg.QG_EINVAL
    assert rep(t=9) == qg.QG_EINVAL
    assert rep(K=288) == qg.QG_ESHAPE                 # K % 256 == 0
    assert rep(t=qg.QG_GGUF_Q2_K, K=128) == qg.QG_ESHAPE
    assert rep(N=0) == qg.QG_ESHAPE
    assert rep(t=qg.QG_GGUF_Q2_K, offs=None) == qg.QG_EINVAL    # Q2_K has real offsets
    assert rep(src=None) == qg.QG_EINVAL
    assert rep(src=A16 + 1) == qg.QG_EALIGN
    assert rep(codes=A16b + 8) == qg.QG_EALIGN
    assert rep(scales=A16c + 2) == qg.QG_EALIGN
    assert rep(offs=None, scales=A16c + 2) == qg.QG_EALIGN
    assert rep(t=qg.QG_GGUF_Q3_K, offs=A16d + 2) == qg.QG_EALIGN


def test_conv_validation_codes():
    """qg_conv2d / qg_conv_stats check formats, modes, shapes, pointers and alignment on the host."""
    L = qg.lib()

    def conv(fmt=qg.QG_FMT_Q4, codes=A16, scales=A16b, X=A16c, H=8, W=8, cin=64, k=3, stride=1, n_out=32,
             norm=0, groups=0, stats=None, gb=None, silu=0, Y=A16d, mode=qg.QG_EXACT):
        return L.qg_conv2d(fmt, codes, scales, X, H, W, cin, k, stride, n_out, norm, groups, stats, gb, silu, Y,
                           mode, None)

    assert conv(fmt=qg.QG_FMT_Q4A) == qg.QG_EUNSUPPORTED      # no affine convolution
    assert conv(fmt=qg.QG_FMT_Q8A) == qg.QG_EUNSUPPORTED
    assert conv(fmt=9) == qg.QG_EINVAL
    assert conv(mode=qg.QG_FAST) == qg.QG_EUNSUPPORTED
    assert conv(cin=48) == qg.QG_ESHAPE
    assert conv(cin=0) == qg.QG_ESHAPE
    assert conv(k=0) == qg.QG_ESHAPE
    assert conv(stride=0) == qg.QG_ESHAPE
    assert conv(n_out=0) == qg.QG_ESHAPE
    assert conv(H=0) == qg.QG_ESHAPE
    assert conv(norm=1, groups=3, stats=A16, gb=A16) == qg.QG_ESHAPE   # groups must divide cin
    assert conv(norm=1, groups=0, stats=A16, gb=A16) == qg.QG_ESHAPE
    assert conv(norm=3) == qg.QG_EINVAL
    assert conv(silu=1) == qg.QG_EINVAL                        # SiLU only with a normalisation
    assert conv(norm=2, stats=None, gb=A16) == qg.QG_EINVAL
    assert conv(norm=2, stats=A16, gb=None) == qg.QG_EINVAL
    assert conv(codes=None) == qg.QG_EINVAL
    assert conv(X=A16c + 4) == qg.QG_EALIGN
    assert conv(codes=A16 + 8) == qg.QG_EALIGN
    assert conv(norm=2, stats=A16 + 2, gb=A16) == qg.QG_EALIGN
    assert conv(fmt=qg.QG_FMT_Q8, scales=A16b + 2) == qg.QG_EALIGN

    def stats(X=A16, npix=64, cin=64, groups=8, eps=1e-5, out=A16b):
        return L.qg_conv_stats(X, npix, cin, groups, eps, out, None)

    assert stats(groups=3) == qg.QG_ESHAPE
    assert stats(npix=0) == qg.QG_ESHAPE
    assert stats(groups=-1) == qg.QG_ESHAPE
    assert stats(eps=-1.0) == qg.QG_EINVAL
    assert stats(eps=float("nan")) == qg.QG_EINVAL
    assert stats(X=None) == qg.QG_EINVAL
    assert stats(out=A16b + 2) == qg.QG_EALIGN


def test_device_plan_validation_codes():
    """qg_moe_plan checks its sizes and pointers on the host, before any HIP call."""
    L = qg.lib()

    def call(T=32, E=128, k=8, logits=A16, seg=A16b, rsrc=A16c, srow=A16d, sw=0x50000, se=None, st=None):
        return L.qg_moe_plan(logits, T, E, k, seg, rsrc, srow, sw, se, st, None)

    assert call(T=0) == qg.QG_ESHAPE
    assert call(E=0) == qg.QG_ESHAPE
    assert call(E=1025, k=8) == qg.QG_ESHAPE          # at most 1024 experts
    assert call(k=0) == qg.QG_ESHAPE
    assert call(E=8, k=9) == qg.QG_ESHAPE             # k <= E
    assert call(E=128, k=33) == qg.QG_ESHAPE          # k <= 32
    assert call(T=2049, k=8) == qg.QG_ESHAPE          # T * k <= 16384
    assert call(T=8192, k=2, E=8, logits=None) == qg.QG_EINVAL   # 16384 slots pass the size check
    assert call(logits=None) == qg.QG_EINVAL
    assert call(sw=None) == qg.QG_EINVAL
    assert call(srow=A16d + 2) == qg.QG_EALIGN
    assert call(st=0x60001) == qg.QG_EALIGN


def test_plan_host_matches_oracle(orc):
    import synth
    for (T, E, k, seed) in [(32, 128, 8, 1004), (75, 8, 2, 7), (5, 16, 16, 3)]:
        lg = synth.normal_as(seed, synth.STREAM_LOGITS, T * E, 0.0, 1.0, "f32").reshape(T, E)
        if T == 5:
            lg[1, :] = 0.25                 # all tied: experts in index order
            lg[2, 3] = lg[2, 9] = 5.0        # a tie at the top
        ours = qg.qg_moe_plan_host(lg, T, E, k)
        ref = orc.moe_plan(lg, T, E, k)
        for key in ("seg_off", "row_src", "slot_row", "slot_expert"):
            assert np.array_equal(ours[key], ref[key]), key
        assert np.allclose(ours["slot_w"], ref["slot_w"], rtol=2e-7, atol=1e-12)
    bad = np.zeros((2, 4), np.float32)
    bad[1, 2] = np.nan
    with pytest.raises(qg.QGError) as e:
        qg.qg_moe_plan_host(bad, 2, 4, 2)
    assert e.value.status == qg.QG_EPLAN


def test_pack_q4_round_trip_against_oracle(orc):
    rng = np.random.default_rng(2)
    N, K = 7, 96
    nib = rng.integers(0, 16, (N, K)).astype(np.uint8)
    codes = qg.pack_q4(nib)
    assert codes.shape == (N, K // 2)
    assert np.array_equal(qg.unpack_q4(codes, N, K), nib)
    scales = np.full(N * K // 32, 0x3C00, np.uint16)     # scale 1.0: weight = nibble - 8
    W = orc.dequant_exact("q4", codes.reshape(-1), scales, None, 64, N, K)
    assert np.array_equal(W, nib.astype(np.float64) - 8.0)
    with pytest.raises(ValueError):
        qg.pack_q4(np.full((1, 32), 16, np.uint8))


def test_noalloc_ffn_validation_codes():
    """The no-allocation expert block checks everything before any HIP call: a call whose
    intermediates exceed the fixed scratch, bad shapes, null and misaligned pointers."""
    L = qg.lib()
    args = [0, A16, A16b, 64, 128, 2048, 1536, A16c, 32, 8, A16d, A16d, A16d, A16d, A16d, 0, 0, None]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return L.qg_moe_ffn_noalloc(*a)
    assert qg.qg_moe_ffn_workspace(2048, 1536, 32, 8, "exact") <= qg.QG_NOALLOC_SCRATCH_BYTES
    assert qg.qg_moe_ffn_workspace(2048, 1536, 32, 8, "fast") <= qg.QG_NOALLOC_SCRATCH_BYTES
    # 4096 tokens x top 8: 32768 routed rows need ~870 MB of intermediates
    assert call(a8=4096) == qg.QG_ESCRATCH
    # exact mode at H 2048, I 1536: 26 624 bytes per routed row, 630 rows, so 78 tokens at top 8
    assert qg.qg_moe_ffn_workspace(2048, 1536, 78, 8, "exact") <= qg.QG_NOALLOC_SCRATCH_BYTES
    assert call(a8=79, a16=0) == qg.QG_ESCRATCH
    assert call(a9=129) == qg.QG_ESHAPE                    # k > E
    assert call(a5=2050) == qg.QG_ESHAPE                   # H % 32
    assert call(a0=5) == qg.QG_EINVAL
    assert call(a14=None) == qg.QG_EINVAL
    assert call(a14=A16d + 4) == qg.QG_EALIGN              # Y: the combine's 16-byte rows
    assert call(a7=A16c + 8) == qg.QG_EALIGN
    assert call(a8=0) == qg.QG_OK                          # T = 0: nothing to do, no HIP call
    # the workspace entry point applies the same checks first
    assert L.qg_moe_ffn(0, A16, A16b, 64, 128, 2048, 1536, A16c, 32, 8, A16d, A16d, A16d, A16d, A16d + 4, 0, 1,
                        0x100000, 1 << 30, None) == qg.QG_EALIGN
