"""GGUF Q4_0 / Q8_0 blocks (scale inside each block) on the GPU: the device repack into the split
layout against the oracle's repack (bit-exact), and matmuls through the repacked weights against the
oracle's f64 GEMM over its own repack of the same bytes."""
import numpy as np
import pytest
import torch

import block_quantized_weight_affine_amd as qg
import synth
from helpers import TAU, check_tol, dev

pytestmark = pytest.mark.gpu


def _gguf_bytes(gtype, N, K, seed):
    """Random code bytes with seeded f16 scales of both signs (a few subnormal)."""
    bb = {"q4_0": 18, "q8_0": 34}[gtype]
    nb = N * K // 32
    rng = np.random.default_rng(seed)
    src = rng.integers(0, 256, nb * bb).astype(np.uint8).reshape(nb, bb)
    d = synth.f16_uniform(seed, 1, nb, -0.05, 0.05)
    d[::97] = 0x0003                                     # subnormal f16 scales
    src[:, 0], src[:, 1] = d & 0xFF, d >> 8
    return src.reshape(-1)


def _repack(gtype, src, N, K):
    codes = torch.empty(N * K // (2 if gtype == "q4_0" else 1), dtype=torch.uint8, device="cuda")
    scales = torch.empty(N * K // 32, dtype=torch.int16 if gtype == "q4_0" else torch.float32, device="cuda")
    print(f"repack {gtype} N={N} K={K}", flush=True)
    qg.qg_repack_gguf(gtype, dev(src), N, K, codes, scales)
    torch.cuda.synchronize()
    return codes, scales


@pytest.mark.parametrize("gtype", ["q4_0", "q8_0"])
@pytest.mark.parametrize("NK", [(64, 288), (3, 32), (517, 1024)])
def test_repack_bit_exact(orc, gtype, NK):
    N, K = NK
    src = _gguf_bytes(gtype, N, K, 11 + N)
    codes, scales = _repack(gtype, src, N, K)
    rc, rs = orc.gguf_repack(gtype, src, N, K)
    assert np.array_equal(codes.cpu().numpy().view(np.uint8), rc.view(np.uint8))
    got_s = scales.cpu().numpy()
    if gtype == "q4_0":
        assert np.array_equal(got_s.view(np.uint16), rs)
    else:
        assert np.array_equal(got_s.view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("gtype", ["q4_0", "q8_0"])
@pytest.mark.parametrize("case", [("exact", 40, "f32"), ("fast", 96, "f16"), ("exact", 1, "f32"), ("exact", 5, "bf16")],
                         ids=lambda c: f"{c[0]}-T{c[1]}-{c[2]}")
def test_matmul_through_repacked_weights(orc, gtype, case):
    mode, T, xt = case
    N, K = 160, 544
    src = _gguf_bytes(gtype, N, K, 23)
    codes, scales = _repack(gtype, src, N, K)
    X = synth.normal_as(29, synth.STREAM_X, T * K, 0.0, 1.0, xt).reshape(T, K)
    Xd = dev(X)
    if xt == "f16":
        Xd = Xd.view(torch.float16)
    elif xt == "bf16":
        Xd = Xd.view(torch.bfloat16)
    Y = torch.full((T, N), float("nan"), device="cuda")
    if gtype == "q4_0":
        qg.qgemm_q4(codes, scales, Xd, Y, N, K, T, mode)
    else:
        qg.qgemm_q8(codes.view(torch.int8), scales, Xd, Y, N, K, T, mode)
    torch.cuda.synchronize()
    # the oracle's GEMM over the oracle's repack of the same GGUF bytes (the repack is pinned on the
    # CPU to decode bit-identically to the oracle's direct GGUF decoder)
    rc, rsc = orc.gguf_repack(gtype, src, N, K)
    fmt = "q4" if gtype == "q4_0" else "q8"
    Xo = X.view(np.uint16) if xt in ("f16", "bf16") else X
    Yr, S, _ = orc.gemm(fmt, rc, rsc, None, 64, N, K, Xo, xt, T)
    check_tol(Y.cpu().numpy(), Yr, S, TAU[mode], f"{gtype} {mode} T={T}")
