"""Q8A (int8 codes, f32 scale and f32 offset per 32-k block; w = fl(fl(q d) + m)) on the GPU, and the
affine GGUF types that map onto it (Q4_1, Q5_0, Q5_1, Q4_K, Q5_K):

  * the device repack GGUF -> Q8A against the oracle's repack, bit for bit (the oracle's repack is
    pinned on the CPU to decode every element as the oracle's direct GGUF decoder does);
  * the staged tiles of every mode against the oracle's, bit for bit;
  * qgemm_q8a / qgemv_q8a / qgemm_batch on seeded Q8A fields against the oracle's f64 GEMM, within
    tau * S of the mode, over every kernel the dispatcher picks (T = 1 streaming GEMV, T <= 8 GEMV,
    exact MFMA tiles, fast MFMA tiles of each size);
  * matmuls through device-repacked GGUF weights against the oracle's GEMM over its own repack."""
import numpy as np
import pytest
import torch

import block_quantized_weight_affine_amd as qg
import synth
from helpers import TAU, check_tol, dev, sample_idx

pytestmark = pytest.mark.gpu

BB = {"q4_1": 20, "q5_0": 22, "q5_1": 24, "q4_k": 144, "q5_k": 176}
STAGED = {"f32": qg.QG_X_F32, "f16": qg.QG_X_F16, "bf16": qg.QG_X_BF16}


def _gguf_bytes(gtype, N, K, seed):
    """Random field bytes; the f16 fields drawn from seeded uniforms (both signs, a few subnormal)."""
    per = 256 if gtype in ("q4_k", "q5_k") else 32
    nb = N * K // per
    rng = np.random.default_rng(seed)
    src = rng.integers(0, 256, nb * BB[gtype]).astype(np.uint8).reshape(nb, BB[gtype])
    d = synth.f16_uniform(seed, 1, nb, -0.05, 0.05)
    d[::97] = 0x0003
    src[:, 0], src[:, 1] = d & 0xFF, d >> 8
    if gtype in ("q4_1", "q5_1", "q4_k", "q5_k"):
        m = synth.f16_uniform(seed, 2, nb, -0.5, 0.5)
        src[:, 2], src[:, 3] = m & 0xFF, m >> 8
    return src.reshape(-1)


def _repack_dev(gtype, src, N, K):
    codes = torch.empty(N * K, dtype=torch.int8, device="cuda")
    scales = torch.empty(N * K // 32, dtype=torch.float32, device="cuda")
    offs = torch.empty(N * K // 32, dtype=torch.float32, device="cuda")
    print(f"repack q8a {gtype} N={N} K={K}", flush=True)
    qg.qg_repack_gguf_q8a(gtype, dev(src), N, K, codes, scales, offs)
    torch.cuda.synchronize()
    return codes, scales, offs


@pytest.mark.parametrize("gtype", ["q4_1", "q5_0", "q5_1", "q4_k", "q5_k"])
@pytest.mark.parametrize("NK", [(64, 512), (3, 256), (517, 1024)])
def test_repack_q8a_bit_exact(orc, gtype, NK):
    N, K = NK
    src = _gguf_bytes(gtype, N, K, 31 + N)
    codes, scales, offs = _repack_dev(gtype, src, N, K)
    rc, rs, ro = orc.gguf_repack_q8a(gtype, src, N, K)
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(offs.cpu().numpy().view(np.uint32), ro.view(np.uint32))


def _xdev(X, xt):
    t = dev(X)
    return t.view(torch.float16) if xt == "f16" else t.view(torch.bfloat16) if xt == "bf16" else t


def _run(w, N, K, T, mode, xt, gemv=False):
    codes, scales, offs = dev(w["codes"]), dev(w["scales"]), dev(w["offsets"])
    X = _xdev(w["X"], xt)
    Y = torch.full((T + 2, N), float("nan"), device="cuda")
    if gemv:
        qg.qgemv_q8a(codes, scales, offs, X, Y, N, K, T)
    else:
        qg.qgemm_q8a(codes, scales, offs, X, Y, N, K, T, mode)
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    assert np.all(np.isnan(y[T:])), "rows at or beyond T were written"
    return y[:T]


CASES = [
    # N, K, T, mode, xt: the T = 1 streaming GEMV, the T <= 8 GEMV, the exact MFMA tiles, the fast
    # decoded tiles (ragged N / T, K % 64 == 32)
    (200, 224, 1, "exact", "f32"),
    (200, 4096, 1, "exact", "bf16"),
    (333, 1056, 5, "exact", "f16"),
    (390, 1056, 37, "exact", "f32"),
    (390, 1056, 37, "exact", "bf16"),
    (520, 1024, 130, "fast", "f16"),
    (96, 160, 9, "fast", "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_q8a_matmul_matches_oracle(orc, case):
    N, K, T, mode, xt = case
    w = synth.make_dense("q8a", N, K, T, xt, 1.0, 2100 + N + K + T)
    print(f"q8a {case}", flush=True)
    y = _run(w, N, K, T, mode, xt)
    Yr, S, _ = orc.gemm("q8a", w["codes"], w["scales"], w["offsets"], 64, N, K, w["X"], xt, T)
    check_tol(y, Yr, S, TAU[mode], f"q8a {case}")
    if T <= 8:
        yv = _run(w, N, K, T, mode, xt, gemv=True)
        assert np.array_equal(yv.view(np.uint32), y.view(np.uint32)), "qgemv_q8a differs from qgemm_q8a"


# fast-mode tile sizes: 256 x 256, 128 x 256 and 128 x 128 (the dispatcher's workgroup-count rule)
BIG = [(4096, 256, 3328), (4096, 256, 1664), (1024, 128, 3200)]


@pytest.mark.parametrize("NKT", BIG, ids=lambda c: "-".join(map(str, c)))
def test_q8a_fast_large_tiles_sampled(orc, NKT):
    N, K, T = NKT
    w = synth.make_dense("q8a", N, K, T, "f16", 1.0, 2300 + T)
    print(f"q8a fast {NKT}", flush=True)
    y = _run(w, N, K, T, "fast", "f16")
    ns, ts = sample_idx(N, 96, 3), sample_idx(T, 40, 4)
    Yr, S, _ = orc.gemm("q8a", w["codes"], w["scales"], w["offsets"], 64, N, K, w["X"], "f16", T, ns=ns, ts=ts)
    check_tol(y[np.ix_(ts, ns)], Yr, S, TAU["fast"], f"q8a fast {NKT}")
    assert np.all(np.isfinite(y))


def test_q8a_dump_extreme_fields(orc):
    """Scales and offsets at f32 extremes (subnormal, zero of both signs, negative, large) and offsets
    that cancel the product exactly: the staged values of every mode bit for bit."""
    N, K = 16, 128
    codes = np.resize(np.arange(-128, 128, dtype=np.int16).astype(np.int8), N * K)
    sc = np.array([1e-45, 2.0 ** -126, 0.0, -0.0, -3.5, 1.0, 0.125, 6.0e4, 1e30, -2.0 ** -20], np.float32)
    of = np.array([-0.0, 0.0, 16.0, -1e-40, 3.0e38, -7.25, 0.5, -1.0, 1e-3, 2.0 ** 20], np.float32)
    scales = np.resize(sc, N * K // 32)
    offs = np.resize(of, N * K // 32)
    offs[8] = 128.0 * scales[8]          # block 8 starts at code -128: -128 d + 128 d = +0
    for staged in ("f32", "f16", "bf16"):
        out = torch.empty((N, K), dtype=torch.float32 if staged == "f32" else torch.int16, device="cuda")
        qg.qg_dequant_dump("q8a", dev(codes), dev(scales), dev(offs), 64, N, K, 0, 0, N, K, STAGED[staged], out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        ref = orc.dequant_tile("q8a", codes, scales, offs, 64, N, K, 0, 0, N, K, staged)
        if staged == "f32":
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), staged
        else:
            assert np.array_equal(got.view(np.uint16), ref), staged


@pytest.mark.parametrize("gtype", ["q4_1", "q5_0", "q5_1", "q4_k", "q5_k"])
@pytest.mark.parametrize("case", [("exact", 1, "f32"), ("exact", 40, "f32"), ("fast", 96, "f16")],
                         ids=lambda c: f"{c[0]}-T{c[1]}-{c[2]}")
def test_matmul_through_repacked_gguf(orc, gtype, case):
    mode, T, xt = case
    N, K = 160, 512
    src = _gguf_bytes(gtype, N, K, 41)
    codes, scales, offs = _repack_dev(gtype, src, N, K)
    X = synth.normal_as(43, synth.STREAM_X, T * K, 0.0, 1.0, xt)
    Y = torch.full((T, N), float("nan"), device="cuda")
    qg.qgemm_q8a(codes, scales, offs, _xdev(X, xt), Y, N, K, T, mode)
    torch.cuda.synchronize()
    rc, rs, ro = orc.gguf_repack_q8a(gtype, src, N, K)
    Yr, S, _ = orc.gemm("q8a", rc, rs, ro, 64, N, K, X, xt, T)
    check_tol(Y.cpu().numpy(), Yr, S, TAU[mode], f"{gtype} {mode} T={T}")


def test_q4_k_decode_full_size_sampled(orc):
    """A 4096 x 4096 Q4_K matrix repacked on the device, then the T = 1 decode GEMV, at sampled outputs."""
    N, K = 4096, 4096
    src = _gguf_bytes("q4_k", N, K, 47)
    codes, scales, offs = _repack_dev("q4_k", src, N, K)
    X = synth.normal_as(53, synth.STREAM_X, K, 0.0, 1.0, "f32")
    Y = torch.full((1, N), float("nan"), device="cuda")
    qg.qgemv_q8a(codes, scales, offs, dev(X), Y, N, K, 1)
    torch.cuda.synchronize()
    rc, rs, ro = orc.gguf_repack_q8a("q4_k", src, N, K)
    ns = sample_idx(N, 256, 7)
    Yr, S, _ = orc.gemm("q8a", rc, rs, ro, 64, N, K, X, "f32", 1, ns=ns)
    check_tol(Y.cpu().numpy()[:, ns], Yr, S, TAU["exact"], "q4_k decode")


@pytest.mark.parametrize("T", [1, 3])
def test_q8a_batch(orc, T):
    """Three Q8A matrices sharing X through qgemm_batch (T = 1: one streaming-GEMV launch)."""
    K = 768
    Ns = [256, 96, 520]
    ws = [synth.make_dense("q8a", n, K, T, "f32", 1.0, 2500 + n) for n in Ns]
    X = ws[0]["X"]
    keep, jobs = [], []
    for w, n in zip(ws, Ns):
        c, s, o = dev(w["codes"]), dev(w["scales"]), dev(w["offsets"])
        y = torch.full((T, n), float("nan"), device="cuda")
        keep.append((c, s, o, y))
        jobs.append((c, s, o, y, n))
    print(f"q8a batch T={T}", flush=True)
    qg.qgemm_batch("q8a", 64, jobs, dev(X), K, T)
    torch.cuda.synchronize()
    for (c, s, o, y), w, n in zip(keep, ws, Ns):
        Yr, S, _ = orc.gemm("q8a", w["codes"], w["scales"], w["offsets"], 64, n, K, X, "f32", T)
        check_tol(y.cpu().numpy(), Yr, S, TAU["exact"], f"batch N={n}")
