"""The implicit-GEMM convolution (qg_conv2d) and its normalisation statistics (qg_conv_stats) on the
GPU against the oracle (oracle.conv2d, oracle.conv_stats).

Convolution: |Y - Y_ref| <= tau_exact * S per element, with S = sum_k |w_k| M_k from the oracle: M_k
is |x'_k| plus, for a normalised tap, every magnitude an f32 rounding of (x - mean) rstd gamma + beta
and of SiLU touches, so the f32 evaluation of the gathered input (a few roundings of size 2^-24 M_k)
and the f32 sums both stay far inside tau_exact.  The statistics the convolution reads are given to
both sides as the same f32 values (the oracle's, rounded).

Statistics: each f32 sum of n terms is taken in a fixed order with at most n / 1024 + 22 (group:
1024 threads, a 6-level wavefront tree, 16 wavefront sums) or n / 64 + 6 (pixel) roundings on
partial sums bounded by sum |x|, so |mean - mean_ref| <= (n / 1024 + 24) 2^-24 sum |x| / n (group)
and the relative error of rstd stays below that count plus 8 roundings (its variance sum likewise,
plus the square root and the division)."""
import numpy as np
import pytest
import torch

import block_quantized_weight_affine_amd as qg
import synth
from helpers import TAU, check_tol, dev, sample_idx

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _inputs(fmt, H, W, cin, ksz, n_out, norm, groups, seed):
    K = ksz * ksz * cin
    w = synth.make_dense(fmt, n_out, K, 1, "f32", 1.0, seed)
    X = synth.normal_as(seed, synth.STREAM_X, H * W * cin, 0.3, 1.0, "f32")
    gb = np.concatenate([synth.normal_as(seed, 7, cin, 1.0, 0.3, "f32"), synth.normal_as(seed, 8, cin, 0.0, 0.5, "f32")])
    st = None
    if norm:
        import oracle as orc
        st = orc.conv_stats(X, H * W, cin, groups if norm == "group" else 0, 1e-5).astype(np.float32)
    return w, X, gb, st


def _conv_gpu(fmt, w, X, H, W, cin, ksz, stride, n_out, norm, groups, st, gb, silu):
    oh, ow = qg.conv_out_size(H, W, ksz, stride)
    Y = torch.full((oh * ow + 1, n_out), float("nan"), device="cuda")
    keep = [dev(w["codes"]), dev(w["scales"]), dev(X), dev(gb) if norm else None, dev(st) if norm else None]
    print(f"conv {fmt} H{H} W{W} cin{cin} k{ksz} s{stride} n_out{n_out} {norm} g{groups} silu{silu}", flush=True)
    qg.qg_conv2d(fmt, keep[0], keep[1], keep[2], H, W, cin, ksz, stride, n_out, Y, norm=norm, groups=groups,
                 stats=keep[4], gamma_beta=keep[3], silu=silu)
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    assert np.all(np.isnan(y[oh * ow:])), "rows past the output pixels were written"
    return y[:oh * ow]


CASES = [
    # fmt, H, W, cin, ksize, stride, n_out, norm, groups, silu
    ("q8", 9, 7, 32, 3, 1, 70, None, 0, False),
    ("q4", 8, 8, 64, 3, 2, 130, "group", 8, True),
    ("q4", 5, 11, 96, 1, 1, 256, "layer", 0, False),
    ("q8", 6, 6, 32, 5, 1, 33, "layer", 0, True),
    ("q4", 7, 5, 32, 2, 1, 64, None, 0, False),
    ("q8", 3, 3, 64, 7, 1, 16, "group", 2, False),
    ("q4", 16, 12, 128, 3, 1, 200, "group", 32, True),
    # cin past the kernel's LDS staging of the per-channel parameters (1024): read from memory
    ("q8", 4, 5, 1088, 1, 1, 40, "group", 4, True),
    ("q4", 3, 4, 1056, 3, 1, 24, "layer", 0, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_conv_matches_oracle(orc, case):
    fmt, H, W, cin, ksz, stride, n_out, norm, groups, silu = case
    w, X, gb, st = _inputs(fmt, H, W, cin, ksz, n_out, norm, groups, 3100 + H * W + cin)
    y = _conv_gpu(fmt, w, X, H, W, cin, ksz, stride, n_out, norm, groups, st, gb, silu)
    Yr, S = orc.conv2d(fmt, w["codes"], w["scales"], None, 64, n_out, X, H, W, cin, ksz, stride, norm,
                       groups, st, gb, silu)
    worst = check_tol(y, Yr, S, TAU["exact"], f"conv {case}")
    print(f"worst |dY|/S = {worst:.3e}")


def test_conv_large_tiles_sampled(orc):
    """192 x 192 pixels, 512 output channels: the 64-row tiles of the exact kernel, sampled outputs."""
    fmt, H, W, cin, ksz, stride, n_out = "q8", 192, 192, 32, 3, 1, 512
    w, X, gb, st = _inputs(fmt, H, W, cin, ksz, n_out, "group", 4, 3300)
    y = _conv_gpu(fmt, w, X, H, W, cin, ksz, stride, n_out, "group", 4, st, gb, True)
    ps, os_ = sample_idx(H * W, 300, 1), sample_idx(n_out, 40, 2)
    Yr, S = orc.conv2d(fmt, w["codes"], w["scales"], None, 64, n_out, X, H, W, cin, ksz, stride, "group", 4, st,
                       gb, True, ps=ps, os_=os_)
    check_tol(y[np.ix_(ps, os_)], Yr, S, TAU["exact"], "conv large")
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("shape", [(37, 64, 8), (4096, 256, 32), (100, 96, 0), (4096, 256, 0), (5, 32, 1)])
def test_conv_stats_match_oracle(orc, shape):
    npix, cin, groups = shape
    X = synth.normal_as(3500 + npix, synth.STREAM_X, npix * cin, 0.7, 2.0, "f32")
    n_st = groups if groups else npix
    out = torch.full((n_st, 2), float("nan"), device="cuda")
    print(f"conv stats {shape}", flush=True)
    qg.qg_conv_stats(dev(X), npix, cin, groups, 1e-5, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = orc.conv_stats(X, npix, cin, groups, 1e-5)
    x = np.abs(X.astype(np.float64)).reshape(npix, cin)
    if groups:
        n = npix * (cin // groups)
        sabs = x.reshape(npix, groups, cin // groups).sum(axis=(0, 2))
        k = n / 1024 + 24
    else:
        n = cin
        sabs = x.sum(axis=1)
        k = n / 64 + 8
    assert np.all(np.abs(got[:, 0] - ref[:, 0]) <= k * U * sabs / n + 1e-30)
    assert np.all(np.abs(got[:, 1] / ref[:, 1] - 1) <= (k + 8) * U)


def test_conv_chained_with_device_stats(orc):
    """qg_conv_stats then qg_conv2d on the device (group norm + SiLU) against the oracle's statistics
    and convolution: the device statistics differ from the oracle's by a few 2^-24 relative, far inside
    tau_exact of the same S."""
    fmt, H, W, cin, ksz, stride, n_out, groups = "q4", 20, 17, 64, 3, 1, 96, 8
    w, X, gb, st = _inputs(fmt, H, W, cin, ksz, n_out, "group", groups, 3700)
    sdev = torch.empty((groups, 2), device="cuda")
    Xd = dev(X)
    qg.qg_conv_stats(Xd, H * W, cin, groups, 1e-5, sdev)
    oh, ow = qg.conv_out_size(H, W, ksz, stride)
    Y = torch.empty((oh * ow, n_out), device="cuda")
    c, s, g = dev(w["codes"]), dev(w["scales"]), dev(gb)
    qg.qg_conv2d(fmt, c, s, Xd, H, W, cin, ksz, stride, n_out, Y, norm="group", groups=groups, stats=sdev,
                 gamma_beta=g, silu=True)
    torch.cuda.synchronize()
    Yr, S = orc.conv2d(fmt, w["codes"], w["scales"], None, 64, n_out, X, H, W, cin, ksz, stride, "group", groups, st,
                       gb, True)
    check_tol(Y.cpu().numpy(), Yr, S, TAU["exact"], "conv chained")


def test_conv_1x1_equals_dense_exact_gemm():
    """A 1 x 1 convolution without normalisation is the exact dense matmul over the pixels: the same
    kernel arithmetic, bit for bit."""
    H, W, cin, n_out = 13, 9, 96, 160
    w = synth.make_dense("q8", n_out, cin, H * W, "f32", 1.0, 3900)
    c, s, x = dev(w["codes"]), dev(w["scales"]), dev(w["X"])
    Yc = torch.empty((H * W, n_out), device="cuda")
    Yg = torch.empty((H * W, n_out), device="cuda")
    qg.qg_conv2d("q8", c, s, x, H, W, cin, 1, 1, n_out, Yc)
    qg.qgemm_q8(c, s, x, Yg, n_out, cin, H * W, "exact")
    torch.cuda.synchronize()
    assert torch.equal(Yc, Yg)


def test_conv_bench_shape_sampled(orc):
    """The benchmark's convolution in its launch configuration: 64 x 64 pixels, 256 -> 256 channels,
    3 x 3 taps, Q4 weights, group norm over 32 groups with SiLU, statistics from the device (sampled
    outputs against the oracle's statistics and convolution)."""
    H = W = 64
    cin, n_out, ksz, groups = 256, 256, 3, 32
    K = ksz * ksz * cin
    w = synth.make_dense("q4", n_out, K, 1, "f32", 1.0, 1501)
    X = synth.normal_as(1501, synth.STREAM_X, H * W * cin, 0.0, 1.0, "f32")
    gb = np.concatenate([np.ones(cin, np.float32), np.zeros(cin, np.float32)])
    Xd = dev(X)
    sdev = torch.empty((groups, 2), device="cuda")
    qg.qg_conv_stats(Xd, H * W, cin, groups, 1e-5, sdev)
    Y = torch.full((H * W, n_out), float("nan"), device="cuda")
    qg.qg_conv2d("q4", dev(w["codes"]), dev(w["scales"]), Xd, H, W, cin, ksz, 1, n_out, Y, norm="group",
                 groups=groups, stats=sdev, gamma_beta=dev(gb), silu=True)
    torch.cuda.synchronize()
    st = orc.conv_stats(X, H * W, cin, groups, 1e-5).astype(np.float32)
    ps, os_ = sample_idx(H * W, 200, 11), sample_idx(n_out, 32, 12)
    Yr, S = orc.conv2d("q4", w["codes"], w["scales"], None, 64, n_out, X, H, W, cin, ksz, 1, "group", groups, st,
                       gb, True, ps=ps, os_=os_)
    check_tol(Y.cpu().numpy()[np.ix_(ps, os_)], Yr, S, TAU["exact"], "conv bench shape")
    assert np.all(np.isfinite(Y.cpu().numpy()))
