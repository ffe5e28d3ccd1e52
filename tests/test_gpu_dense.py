"""Dense matmul parity: GEMV (T <= 8), exact (f32 MFMA) and fast (f16 / bf16 MFMA) tile kernels
against the f64 oracle, at tile-spanning sizes with ragged tails and at the workloads' full sizes
(sampled outputs), plus edge cases."""
import numpy as np
import pytest
import torch

import block_quantized_weight_affine_amd as qg
import synth
from helpers import TAU, check_tol, dev, dev_x, oracle_x, sample_idx, weights_dev

pytestmark = pytest.mark.gpu


def _run(fmt, w, X, xtype, N, K, T, mode, extra_rows=0):
    """Runs the dense entry point; returns Y (numpy) and the untouched padding rows."""
    codes, scales, offs = weights_dev(w)
    Xd = dev_x(X, xtype)
    Y = torch.full((T + extra_rows, N), float("nan"), dtype=torch.float32, device="cuda")
    qg.qgemm(fmt, codes, scales, offs, w["group"], Xd, Y, N, K, T, mode)
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    return y[:T], y[T:]


def _ref(orc, fmt, w, X, xtype, N, K, T, ns=None, ts=None):
    Yr, S, _ = orc.gemm(fmt, w["codes"], w["scales"], w.get("offsets"), w["group"], N, K, oracle_x(X, xtype), xtype, T,
                        ns=ns, ts=ts)
    return Yr, S


CASES = [
    # fmt, N, K, T, xtype, mode
    ("q4", 256, 512, 16, "f32", "exact"),        # the tiny Q4 workload
    ("q4", 200, 224, 37, "f16", "exact"),        # ragged N, K % 64 == 32, ragged T
    ("q4", 200, 224, 37, "f16", "fast"),
    ("q4a", 136, 320, 70, "bf16", "fast"),
    ("q4a", 136, 320, 70, "bf16", "exact"),
    ("q4a", 96, 256, 33, "f16", "fast"),
    ("q8", 160, 288, 45, "f32", "exact"),
    ("q8", 160, 288, 45, "bf16", "fast"),
    ("q8", 160, 288, 45, "f16", "fast"),
    ("q4", 96, 128, 9, "bf16", "fast"),          # first T above the GEMV range
    ("q4", 1000, 2048, 300, "f16", "fast"),      # several tiles both ways
    ("q4a", 520, 1024, 260, "bf16", "fast"),
    ("q8", 390, 1024, 130, "f32", "exact"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_dense_tiles(orc, case):
    fmt, N, K, T, xtype, mode = case
    w = synth.make_dense(fmt, N, K, T, xtype, 1.0, 500 + N + K + T)
    Y, pad = _run(fmt, w, w["X"], xtype, N, K, T, mode, extra_rows=3)
    Yr, S = _ref(orc, fmt, w, w["X"], xtype, N, K, T)
    check_tol(Y, Yr, S, TAU[mode], str(case))
    assert np.all(np.isnan(pad)), "rows at or beyond T were written"


@pytest.mark.parametrize("fmt", ["q4", "q4a", "q8"])
@pytest.mark.parametrize("T", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("xtype", ["f32", "f16", "bf16"])
def test_gemv(orc, fmt, T, xtype):
    N, K = 72, 1088          # K not a multiple of the 1024-element wavefront step
    w = synth.make_dense(fmt, N, K, T, xtype, 1.0, 900 + T)
    codes, scales, offs = weights_dev(w)
    Y = torch.full((T + 2, N), float("nan"), dtype=torch.float32, device="cuda")
    qg.qgemv(fmt, codes, scales, offs, w["group"], dev_x(w["X"], xtype), Y, N, K, T)
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    Yr, S = _ref(orc, fmt, w, w["X"], xtype, N, K, T)
    check_tol(y[:T], Yr, S, TAU["exact"], f"gemv {fmt} T={T} {xtype}")
    assert np.all(np.isnan(y[T:]))


def test_mixed_row_magnitudes_exact(orc):
    """X rows of magnitude 1e-3, 1, 300 and 2e5 (the matrix-unit test design of oxinfer src/metal.rs,
    tests: mma_matmul_matches_cpu) at 192 x 512 with T = 150 and 37, exact mode."""
    N, K = 192, 512
    for T in (150, 37):
        for fmt in ("q8", "q4"):
            w = synth.make_dense(fmt, N, K, T, "f32", 1.0, 31 + T)
            mag = np.array([1e-3, 1.0, 300.0, 2e5])[np.arange(T) % 4]
            X = (w["X"].reshape(T, K) * mag[:, None]).astype(np.float32)
            Y, _ = _run(fmt, w, X, "f32", N, K, T, "exact")
            Yr, S = _ref(orc, fmt, w, X, "f32", N, K, T)
            check_tol(Y, Yr, S, TAU["exact"], f"mixed {fmt} T={T}")


def test_edge_shapes(orc):
    # T = 0 launches nothing and leaves Y untouched
    w = synth.make_dense("q4", 64, 64, 4, "f32", 1.0, 1)
    codes, scales, _ = weights_dev(w)
    Y = torch.full((4, 64), 7.0, device="cuda")
    qg.qgemm_q4(codes, scales, dev_x(w["X"], "f32"), Y, 64, 64, 0)
    torch.cuda.synchronize()
    assert torch.all(Y == 7.0)
    # one block, one row, one token
    for (N, K, T, mode, xt) in [(1, 32, 1, "exact", "f32"), (1, 32, 9, "exact", "f32"), (1, 32, 9, "fast", "f16"),
                                (16, 32, 40, "fast", "bf16"), (33, 64, 8, "fast", "f16")]:
        w = synth.make_dense("q4", N, K, T, xt, 1.0, 11 + N + T)
        Y, _ = _run("q4", w, w["X"], xt, N, K, T, mode)
        Yr, S = _ref(orc, "q4", w, w["X"], xt, N, K, T)
        check_tol(Y, Yr, S, TAU[mode], f"edge {N} {K} {T} {mode}")


def test_zero_weights_give_exact_zero(orc):
    """All nibbles 8 (Q4 weight 0): S = 0, so Y must be exactly 0 in every path."""
    N, K = 64, 256
    codes = np.full(N * K // 2, 0x88, np.uint8)
    scales = np.full(N * K // 32, 0x3C00, np.uint16)
    for T, mode, xt in [(4, "exact", "f32"), (40, "exact", "f32"), (40, "fast", "f16")]:
        X = synth.normal_as(5, 3, T * K, 0, 1, xt)
        Y = torch.empty((T, N), device="cuda")
        qg.qgemm_q4(dev(codes), dev(scales), dev_x(X, xt), Y, N, K, T, mode)
        torch.cuda.synchronize()
        assert torch.all(Y == 0), (T, mode)


@pytest.mark.parametrize("fmt", ["q4", "q4a", "q8"])
@pytest.mark.parametrize("shape", [(200, 320, 40), (512, 1024, 300)], ids=["small-tiles", "128x128-tiles"])
def test_fast_blocks_needing_pages_order(orc, fmt, shape):
    """Fast mode through blocks whose one-FMA decode is not the pages' rounding: negative and zero
    scales, and (Q4A) offsets next to scales so large that m - 8d is inexact in f32; every third
    block is affected, so every wavefront re-decodes some blocks in the pages' order."""
    N, K, T = shape
    w = synth.make_dense(fmt, N, K, T, "bf16" if fmt == "q4a" else "f16", 1.0, 77 + N)
    sc = w["scales"].copy()
    nb = sc.size
    neg, zero = np.arange(0, nb, 3), np.arange(1, nb, 9)
    if fmt == "q8":
        sc[neg] = -np.abs(sc[neg])
        sc[zero] = 0.0
    else:
        sc[neg] |= np.uint16(0x8000)
        sc[zero] = 0
    w["scales"] = sc
    if fmt == "q4a":
        off = w["offsets"].copy()
        big = np.arange(2, nb, 3)                     # scale 1024, offset 2^-13: 2^-13 - 8192 is not an f32
        sc[big] = 0x6400
        g_of = (big % (K // 32)) * 32 // w["group"] + (big // (K // 32)) * (K // w["group"])
        off[g_of] = 0x3900
        w["offsets"] = off
    xt = "bf16" if fmt == "q4a" else "f16"
    Y, _ = _run(fmt, w, w["X"], xt, N, K, T, "fast")
    Yr, S = _ref(orc, fmt, w, w["X"], xt, N, K, T)
    check_tol(Y, Yr, S, TAU["fast"], f"fixup {fmt} {shape}")


@pytest.mark.parametrize("T,K", [(2, 10240), (4, 5120), (4, 5248), (8, 2560), (3, 6912)])
def test_gemv_rows_chunked_k(orc, T, K):
    """T rows of X whose K spans several of the multi-row kernel's LDS chunks (4096 values for T <= 4,
    2048 above), the last one ragged or whole."""
    N = 136
    w = synth.make_dense("q4a", N, K, T, "f32", 1.0, 970 + T + K)
    codes, scales, offs = weights_dev(w)
    Y = torch.full((T + 1, N), float("nan"), dtype=torch.float32, device="cuda")
    qg.qgemv("q4a", codes, scales, offs, w["group"], dev_x(w["X"], "f32"), Y, N, K, T)
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    Yr, S = _ref(orc, "q4a", w, w["X"], "f32", N, K, T)
    check_tol(y[:T], Yr, S, TAU["exact"], f"gemv T={T} K={K}")
    assert np.all(np.isnan(y[T:]))


@pytest.mark.parametrize("fmt,N,K,T", [("q8", 4096, 4096, 4), ("q4", 40, 16384, 4), ("q8", 40, 16416, 2),
                                        ("q4a", 33, 16384, 3), ("q8", 1000, 4096, 8), ("q4", 40, 8192, 8),
                                        ("q4a", 40, 8256, 6), ("q8", 24, 8224, 5)])
def test_gemv_few_rows_full_and_long_k(orc, fmt, N, K, T):
    """T = 2..8 rows of X: the Q8 decode shape at full size (every output against the oracle), the
    longest K the K-split kernel takes (16 wavefronts of 1024 values for T <= 4, 8 above), and just
    past it (the chunked kernel)."""
    w = synth.make_dense(fmt, N, K, T, "f32", 1.0, 960 + T + K)
    codes, scales, offs = weights_dev(w)
    Y = torch.full((T + 1, N), float("nan"), dtype=torch.float32, device="cuda")
    qg.qgemv(fmt, codes, scales, offs, w["group"], dev_x(w["X"], "f32"), Y, N, K, T)
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    Yr, S = _ref(orc, fmt, w, w["X"], "f32", N, K, T)
    check_tol(y[:T], Yr, S, TAU["exact"], f"gemv {fmt} N={N} K={K} T={T}")
    assert np.all(np.isnan(y[T:]))


@pytest.mark.parametrize("K", [16384, 16416])
def test_gemv_single_row_long_k(orc, K):
    """T = 1 at the longest K whose X fits the streaming kernel's LDS copy, and just past it (the
    chunked kernel takes over)."""
    N = 40
    w = synth.make_dense("q8", N, K, 1, "f32", 1.0, 990 + K)
    codes, scales, offs = weights_dev(w)
    Y = torch.full((2, N), float("nan"), dtype=torch.float32, device="cuda")
    qg.qgemv("q8", codes, scales, offs, w["group"], dev_x(w["X"], "f32"), Y, N, K, 1)
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    Yr, S = _ref(orc, "q8", w, w["X"], "f32", N, K, 1)
    check_tol(y[:1], Yr, S, TAU["exact"], f"gemv T=1 K={K}")
    assert np.all(np.isnan(y[1:]))


# Shapes that reach each fast tile configuration (sampled outputs): 128 x 256 and 128 x 128 tiles
# with the 4-deep register prefetch, and 64 x 128 tiles over a long K; the stage counts 15, 10 and
# 33 leave 3, 2 and 1 stages after the 4-way unrolled loop.
TILE_SHAPES = [
    ("q4", 6400, 928, 1024, "f16"),
    ("q4a", 3200, 640, 1000, "bf16"),
    ("q8", 4096, 2080, 512, "bf16"),
]


@pytest.mark.parametrize("case", TILE_SHAPES, ids=lambda c: "-".join(map(str, c)))
def test_fast_tile_configs_sampled(orc, case):
    fmt, N, K, T, xtype = case
    print(f"fast tile shape {case}", flush=True)
    w = synth.make_dense(fmt, N, K, T, xtype, 1.0, 700 + K)
    Y, _ = _run(fmt, w, w["X"], xtype, N, K, T, "fast")
    ns = sample_idx(N, 160, 3)
    ts = sample_idx(T, 24, 4)
    Yr, S = _ref(orc, fmt, w, w["X"], xtype, N, K, T, ns=ns, ts=ts)
    check_tol(Y[np.ix_(ts, ns)], Yr, S, TAU["fast"], str(case))
    assert np.all(np.isfinite(Y))


# ---- the workloads at full size (sampled outputs), in the launch configuration the benchmark uses ----
FULL = [
    (1, "exact"), (2, "exact"), (2, "fast"), (3, "fast"),
]


@pytest.mark.parametrize("cfg_mode", FULL, ids=lambda c: f"cfg{c[0]}-{c[1]}")
def test_full_size_sampled(orc, cfg_mode):
    ci, mode = cfg_mode
    c = synth.CONFIGS[ci]
    print(f"full-size workload {c.name} {mode}", flush=True)
    w = synth.make_dense(c.fmt, c.N, c.K, c.T, c.xtype, c.x_sigma, c.seed, group=c.group)
    Y, _ = _run(c.fmt, w, w["X"], c.xtype, c.N, c.K, c.T, mode)
    # the T = 1 decode is checked at every output (16.8 M multiply-adds in the oracle); the prefill
    # shapes at sampled rows and tokens
    ns = np.arange(c.N, dtype=np.int32) if c.T == 1 else sample_idx(c.N, 160, 1)
    ts = sample_idx(c.T, 24, 2)
    Yr, S = _ref(orc, c.fmt, w, w["X"], c.xtype, c.N, c.K, c.T, ns=ns, ts=ts)
    check_tol(Y[np.ix_(ts, ns)], Yr, S, TAU[mode], c.name)
    assert np.all(np.isfinite(Y))
