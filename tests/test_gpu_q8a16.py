"""Q8A16 (int8 codes, f32 scale and f32 offset per 16-element block; w = fl(fl(q d) + m)) on the GPU, and
the GGUF K-quants that map onto it (Q6_K, Q3_K, Q2_K):

  * the device repack GGUF -> Q8A16 against the oracle's repack, bit for bit (the oracle's repack is
    pinned on the CPU to decode every element, zeros' signs included, as its direct GGUF decoder);
  * the f32 staged tile of the exact kernel's decode against the oracle's direct GGUF decode, bit for
    bit;
  * qgemm_q8a16 / qgemv_q8a16 on seeded fields against the oracle's f64 GEMM within tau * S of the
    mode, over every kernel the dispatcher picks (T = 1 streaming GEMV, T <= 8 K-split GEMV, the
    plain GEMV past the K-split limits, the exact MFMA tiles of both sizes -- in both modes);
  * matmuls through device-repacked GGUF weights against the oracle's GEMM over its own repack."""
import numpy as np
import pytest
import torch

import block_quantized_weight_affine_amd as qg
import synth
from helpers import TAU, check_tol, dev, sample_idx

pytestmark = pytest.mark.gpu

SBB = {"q6_k": 210, "q3_k": 110, "q2_k": 84}


def _gguf_bytes(gtype, N, K, seed):
    """Random super-block bytes; the f16 fields drawn from seeded uniforms (both signs, a few
    subnormal)."""
    nb = N * K // 256
    rng = np.random.default_rng(seed)
    src = rng.integers(0, 256, nb * SBB[gtype]).astype(np.uint8).reshape(nb, SBB[gtype])
    d = synth.f16_uniform(seed, 1, nb, -0.05, 0.05)
    d[::97] = 0x0003
    at = {"q6_k": 208, "q3_k": 108, "q2_k": 80}[gtype]
    src[:, at], src[:, at + 1] = d & 0xFF, d >> 8
    if gtype == "q2_k":
        m = synth.f16_uniform(seed, 2, nb, -0.05, 0.05)
        src[:, 82], src[:, 83] = m & 0xFF, m >> 8
    return src.reshape(-1)


def _repack_dev(gtype, src, N, K, with_offsets=True):
    codes = torch.empty(N * K, dtype=torch.int8, device="cuda")
    scales = torch.empty(N * K // 16, dtype=torch.float32, device="cuda")
    offs = torch.empty(N * K // 16, dtype=torch.float32, device="cuda") if with_offsets else None
    print(f"repack q8a16 {gtype} N={N} K={K}", flush=True)
    qg.qg_repack_gguf_q8a16(gtype, dev(src), N, K, codes, scales, offs)
    torch.cuda.synchronize()
    return codes, scales, offs


@pytest.mark.parametrize("gtype", ["q6_k", "q3_k", "q2_k"])
@pytest.mark.parametrize("NK", [(64, 512), (3, 256), (517, 1024)])
def test_repack_q8a16_bit_exact(orc, gtype, NK):
    N, K = NK
    src = _gguf_bytes(gtype, N, K, 61 + N)
    codes, scales, offs = _repack_dev(gtype, src, N, K)
    rc, rs, ro = orc.gguf_repack_q8a16(gtype, src, N, K)
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(offs.cpu().numpy().view(np.uint32), ro.view(np.uint32))


@pytest.mark.parametrize("gtype", ["q6_k", "q3_k", "q2_k"])
def test_q8a16_staged_tile_equals_gguf_decode(orc, gtype):
    """The exact kernels' decode of the repacked weights (qg_dequant_dump, f32) is the pages' value of
    every element, bit for bit; the fast kernels' f16 / bf16 staging is its nearest-even rounding, bit
    for bit against the oracle's."""
    N, K = 37, 768
    src = _gguf_bytes(gtype, N, K, 71)
    codes, scales, offs = _repack_dev(gtype, src, N, K)
    out = torch.empty((N, K), dtype=torch.float32, device="cuda")
    qg.qg_dequant_dump("q8a16", codes, scales, offs, 64, N, K, 0, 0, N, K, qg.QG_X_F32, out)
    torch.cuda.synchronize()
    ref = orc.gguf_dequant(gtype, src, N, K)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    rc, rs, ro = orc.gguf_repack_q8a16(gtype, src, N, K)
    for staged, code in (("f16", qg.QG_X_F16), ("bf16", qg.QG_X_BF16)):
        o16 = torch.empty((N, K), dtype=torch.int16, device="cuda")
        qg.qg_dequant_dump("q8a16", codes, scales, offs, 64, N, K, 0, 0, N, K, code, o16)
        torch.cuda.synchronize()
        r16 = orc.dequant_tile("q8a16", rc, rs, ro, 64, N, K, 0, 0, N, K, staged)
        assert np.array_equal(o16.cpu().numpy().view(np.uint16), r16), staged


def _fields(N, K, T, xt, seed):
    """Q8A16 fields: codes from the dense Q8 generator, scales of both signs and offsets per 16 k."""
    w = synth.make_dense("q8", N, K, T, xt, 1.0, seed)
    rng = np.random.default_rng(seed)
    sc = (rng.uniform(0.002, 0.01, N * K // 16) * rng.choice([-1.0, 1.0], N * K // 16)).astype(np.float32)
    of = rng.normal(0.0, 0.2, N * K // 16).astype(np.float32)
    return w["codes"], sc, of, w["X"]


def _xdev(X, xt):
    t = dev(X)
    return t.view(torch.float16) if xt == "f16" else t.view(torch.bfloat16) if xt == "bf16" else t


def _run(c, s, o, X, N, K, T, mode, xt, gemv=False):
    Y = torch.full((T + 2, N), float("nan"), device="cuda")
    if gemv:
        qg.qgemv_q8a16(c, s, o, _xdev(X, xt), Y, N, K, T)
    else:
        qg.qgemm_q8a16(c, s, o, _xdev(X, xt), Y, N, K, T, mode)
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    assert np.all(np.isnan(y[T:])), "rows at or beyond T were written"
    return y[:T]


CASES = [
    # N, K, T, mode, xt: the T = 1 streaming GEMV, the K-split GEMV, the plain GEMV past the K-split
    # limits (T = 1 and T = 6), the exact MFMA tiles in both modes (ragged N / T, K % 64 == 32)
    (200, 256, 1, "exact", "f32"),
    (200, 4096, 1, "exact", "bf16"),
    (333, 1056, 5, "exact", "f16"),
    (70, 16640, 1, "exact", "f32"),
    (70, 9216, 6, "exact", "f32"),
    (390, 1056, 37, "exact", "f32"),
    (390, 1056, 37, "fast", "bf16"),
    (96, 160, 9, "fast", "f16"),
    (200, 256, 40, "fast", "f32"),
]


# fast-mode tile sizes: 256 x 256, 128 x 256 and 128 x 128 (the dispatcher's workgroup-count rule)
BIG = [(4096, 256, 3328), (4096, 256, 1664), (1024, 128, 3200)]


@pytest.mark.parametrize("NKT", BIG, ids=lambda c: "-".join(map(str, c)))
def test_q8a16_fast_large_tiles_sampled(orc, NKT):
    N, K, T = NKT
    codes, sc, of, X = _fields(N, K, T, "f16", 2800 + T)
    print(f"q8a16 fast {NKT}", flush=True)
    y = _run(dev(codes), dev(sc), dev(of), X, N, K, T, "fast", "f16")
    ns, ts = sample_idx(N, 96, 3), sample_idx(T, 40, 4)
    Yr, S, _ = orc.gemm("q8a16", codes, sc, of, 64, N, K, X, "f16", T, ns=ns, ts=ts)
    check_tol(y[np.ix_(ts, ns)], Yr, S, TAU["fast"], f"q8a16 fast {NKT}")
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_q8a16_matmul_matches_oracle(orc, case):
    N, K, T, mode, xt = case
    codes, sc, of, X = _fields(N, K, T, xt, 2500 + N + K + T)
    c, s, o = dev(codes), dev(sc), dev(of)
    print(f"q8a16 {case}", flush=True)
    y = _run(c, s, o, X, N, K, T, mode, xt)
    Yr, S, _ = orc.gemm("q8a16", codes, sc, of, 64, N, K, X, xt, T)
    check_tol(y, Yr, S, TAU[mode], f"q8a16 {case}")
    if T <= 8:
        yv = _run(c, s, o, X, N, K, T, mode, xt, gemv=True)
        assert np.array_equal(yv.view(np.uint32), y.view(np.uint32)), "qgemv_q8a16 differs from qgemm_q8a16"


def test_q8a16_exact_64_row_tiles_sampled(orc):
    """N 4096, T 2048: the exact kernel's 64-row tiles; sampled outputs."""
    N, K, T = 4096, 128, 2048
    codes, sc, of, X = _fields(N, K, T, "f32", 2700)
    print("q8a16 64-row tiles", flush=True)
    y = _run(dev(codes), dev(sc), dev(of), X, N, K, T, "exact", "f32")
    ns, ts = sample_idx(N, 96, 5), sample_idx(T, 40, 6)
    Yr, S, _ = orc.gemm("q8a16", codes, sc, of, 64, N, K, X, "f32", T, ns=ns, ts=ts)
    check_tol(y[np.ix_(ts, ns)], Yr, S, TAU["exact"], "q8a16 64-row tiles")
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("gtype", ["q6_k", "q3_k", "q2_k"])
@pytest.mark.parametrize("case", [("exact", 1, "f32"), ("exact", 3, "bf16"), ("exact", 40, "f32"),
                                  ("fast", 96, "f16")], ids=lambda c: f"{c[0]}-T{c[1]}-{c[2]}")
def test_matmul_through_repacked_kquant(orc, gtype, case):
    mode, T, xt = case
    N, K = 160, 512
    src = _gguf_bytes(gtype, N, K, 81)
    codes, scales, offs = _repack_dev(gtype, src, N, K)
    X = synth.normal_as(83, synth.STREAM_X, T * K, 0.0, 1.0, xt)
    Y = torch.full((T, N), float("nan"), device="cuda")
    qg.qgemm_q8a16(codes, scales, offs, _xdev(X, xt), Y, N, K, T, mode)
    torch.cuda.synchronize()
    rc, rs, ro = orc.gguf_repack_q8a16(gtype, src, N, K)
    Yr, S, _ = orc.gemm("q8a16", rc, rs, ro, 64, N, K, X, xt, T)
    check_tol(Y.cpu().numpy(), Yr, S, TAU[mode], f"{gtype} {mode} T={T}")


def test_q6_k_decode_full_size_sampled(orc):
    """A 4096 x 4096 Q6_K matrix repacked on the device, then the T = 1 decode GEMV, at sampled outputs."""
    N, K = 4096, 4096
    src = _gguf_bytes("q6_k", N, K, 87)
    codes, scales, offs = _repack_dev("q6_k", src, N, K)
    X = synth.normal_as(89, synth.STREAM_X, K, 0.0, 1.0, "f32")
    Y = torch.full((1, N), float("nan"), device="cuda")
    qg.qgemv_q8a16(codes, scales, offs, dev(X), Y, N, K, 1)
    torch.cuda.synchronize()
    rc, rs, ro = orc.gguf_repack_q8a16("q6_k", src, N, K)
    ns = sample_idx(N, 256, 9)
    Yr, S, _ = orc.gemm("q8a16", rc, rs, ro, 64, N, K, X, "f32", 1, ns=ns)
    check_tol(Y.cpu().numpy()[:, ns], Yr, S, TAU["exact"], "q6_k decode")


def test_q8a16_refused_where_not_built():
    """The batched, grouped and 16-bit-staged paths refuse Q8A16 before launching anything."""
    N, K, T = 64, 256, 3
    c = torch.zeros(N * K, dtype=torch.int8, device="cuda")
    s = torch.zeros(N * K // 16, dtype=torch.float32, device="cuda")
    X = torch.zeros((T, K), dtype=torch.float32, device="cuda")
    Y = torch.zeros((T, N), dtype=torch.float32, device="cuda")
    with pytest.raises(RuntimeError):
        qg.qgemm_batch("q8a16", 64, [(c, s, s, Y, N)], X, K, T)
    with pytest.raises(RuntimeError):
        qg.qgemm_q8a16(c, s, s, X.half(), Y, N, K, T, "fast_wexact")


@pytest.mark.parametrize("gtype", ["q6_k", "q3_k"])
def test_offset_free_layout(orc, gtype):
    """Q6_K / Q3_K repacked without offsets: codes and scales as the oracle's, the staged tile equal to
    the in-block decode bit for bit, and matmuls (T = 1 streaming GEMV, T = 3 K-split GEMV, T = 40
    exact tiles, T = 96 fast) against the oracle's offset-free GEMM; the T = 1 result equals the one
    with the explicit -0 offsets bit for bit."""
    N, K = 96, 1024
    src = _gguf_bytes(gtype, N, K, 91)
    codes, scales, none = _repack_dev(gtype, src, N, K, with_offsets=False)
    assert none is None
    rc, rs, _ = orc.gguf_repack_q8a16(gtype, src, N, K, with_offsets=False)
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    out = torch.empty((N, K), dtype=torch.float32, device="cuda")
    qg.qg_dequant_dump("q8a16", codes, scales, None, 64, N, K, 0, 0, N, K, qg.QG_X_F32, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), orc.gguf_dequant(gtype, src, N, K).view(np.uint32))
    for mode, T, xt in (("exact", 1, "f32"), ("exact", 3, "f16"), ("exact", 40, "f32"), ("fast", 96, "bf16")):
        X = synth.normal_as(93 + T, synth.STREAM_X, T * K, 0.0, 1.0, xt)
        Y = torch.full((T, N), float("nan"), device="cuda")
        print(f"offset-free {gtype} {mode} T={T}", flush=True)
        qg.qgemm_q8a16(codes, scales, None, _xdev(X, xt), Y, N, K, T, mode)
        torch.cuda.synchronize()
        Yr, S, _ = orc.gemm("q8a16", rc, rs, None, 64, N, K, X, xt, T)
        check_tol(Y.cpu().numpy(), Yr, S, TAU[mode], f"offset-free {gtype} {mode} T={T}")
        if T == 1:
            c2, s2, o2 = _repack_dev(gtype, src, N, K)
            Y2 = torch.full((T, N), float("nan"), device="cuda")
            qg.qgemv_q8a16(c2, s2, o2, _xdev(X, xt), Y2, N, K, T)
            torch.cuda.synchronize()
            assert np.array_equal(Y.cpu().numpy().view(np.uint32), Y2.cpu().numpy().view(np.uint32))
