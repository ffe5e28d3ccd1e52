"""q8_2f and q8_row tensors on the GPU (page "cortiq-engine 0.8.3 src/gpu_metal/qi21.rs", the block
loader's codec match; page "cortiq-engine 0.8.41 src/gpu_metal/clover.rs", q8mm) against the oracle:

  * qg_repack_q8f: the f32 block scales (the row scale in every block of its row) and the f32 column
    field, bit for bit;
  * qg_col_scale: X times the column field for every (X type, output type) pair, bit for bit;
  * the matmul the pages run (column field on X, the codes in place as Q8 codes, the row scale per
    block): exact mode with f32 X at tau_exact, the W-exact fast path with f16 X at tau_fast, the
    T = 1 GEMV, and q8_row straight through the Q8 calls, all against the oracle's f64 GEMM over
    w = q col[k] rs[n]."""
import numpy as np
import pytest
import torch

import block_quantized_weight_affine_amd as qg
import synth
from helpers import TAU, check_tol, dev

pytestmark = pytest.mark.gpu

TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _blob(N, K, has_col, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(-128, 128, (N, K)).astype(np.int8)
    rs = synth.f16_uniform(seed, 1, N, -0.02, 0.02)
    rs[::37] = 0x0001                                   # subnormal row scales
    parts = [codes.view(np.uint8).ravel(), rs.astype("<u2").view(np.uint8)]
    if has_col:
        parts.append(synth.f16_uniform(seed, 2, K, 0.05, 4.0).astype("<u2").view(np.uint8))
    return np.concatenate(parts)


def _repack(blob, N, K, has_col):
    b = dev(blob)
    scales = torch.full((N * K // 32,), float("nan"), device="cuda")
    col = torch.full((K,), float("nan"), device="cuda") if has_col else None
    print(f"repack q8f N={N} K={K} col={has_col}", flush=True)
    qg.qg_repack_q8f(b, N, K, has_col, scales, col)
    return b, scales, col


@pytest.mark.parametrize("has_col", [True, False])
def test_repack_q8f_bit_exact(orc, has_col):
    N, K = 77, 320
    blob = _blob(N, K, has_col, 5)
    b, scales, col = _repack(blob, N, K, has_col)
    torch.cuda.synchronize()
    rs, cf = orc.q8f_fields(blob, N, K, has_col)
    assert np.array_equal(scales.cpu().numpy(), np.repeat(rs.astype(np.float32), K // 32))
    if has_col:
        assert np.array_equal(col.cpu().numpy(), cf.astype(np.float32))


@pytest.mark.parametrize("xt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("st", ["f32", "f16", "bf16"])
def test_col_scale_bit_exact(orc, xt, st):
    T, K = 7, 264
    X = synth.normal_as(70, synth.STREAM_X, T * K, 0.0, 3.0, xt)
    X[:3] = synth.normal_as(71, 3, 3, 0.0, 1.0, xt)
    if xt == "f32":
        X[3:6] = [6.0e4, -1e-30, 3.0e38]                 # overflow / underflow of the narrowing
    col = (synth.f16_uniform(72, 2, K, -4.0, 4.0).view(np.float16)).astype(np.float32)
    Xd = dev(X)
    if xt != "f32":
        Xd = Xd.view(TDT[xt])
    Xs = torch.empty((T, K), dtype=TDT[st], device="cuda")
    print(f"col scale {xt} -> {st}", flush=True)
    qg.qg_col_scale(Xd, T, K, dev(col), Xs)
    torch.cuda.synchronize()
    want = orc.col_scale(X, xt, T, K, col, st)
    got = Xs.cpu()
    got = got.numpy() if st == "f32" else got.view(torch.int16).numpy().view(np.uint16)
    if st == "f32":
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    else:
        assert np.array_equal(got, want)


CASES = [
    # N, K, T, mode: T = 1 (streaming GEMV), T <= 8, the exact tiles, the W-exact fast tiles
    (256, 1024, 1, "exact"),
    (200, 512, 5, "exact"),
    (330, 1056, 70, "exact"),
    (512, 1024, 96, "fast_wexact"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_q8f_matmul_matches_oracle(orc, case):
    N, K, T, mode = case
    blob = _blob(N, K, True, 900 + T)
    b, scales, col = _repack(blob, N, K, True)
    xt = "f32" if mode == "exact" else "f16"
    X = synth.normal_as(901 + T, synth.STREAM_X, T * K, 0.0, 1.0, xt)
    Xd = dev(X) if xt == "f32" else dev(X).view(torch.float16)
    Xs = torch.empty((T, K), dtype=TDT[xt], device="cuda")
    qg.qg_col_scale(Xd, T, K, col, Xs)
    Y = torch.full((T + 1, N), float("nan"), device="cuda")
    print(f"q8f matmul {case}", flush=True)
    qg.qgemm_q8(b, scales, Xs, Y, N, K, T, mode)
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    assert np.all(np.isnan(y[T:]))
    Yr, S = orc.q8f_gemm(blob, N, K, True, X, xt, T)
    tau = TAU["exact"] if mode == "exact" else TAU["fast"]
    check_tol(y[:T], Yr, S, tau, f"q8f {case}")
    if T == 1:
        Yv = torch.full((1, N), float("nan"), device="cuda")
        qg.qgemv_q8(b, scales, Xs, Yv, N, K, 1)
        torch.cuda.synchronize()
        check_tol(Yv.cpu().numpy(), Yr, S, TAU["exact"], "q8f gemv")


@pytest.mark.parametrize("T", [1, 40])
def test_q8_row_matmul_matches_oracle(orc, T):
    """q8_row: no column field, the Q8 call on X as it is."""
    N, K = 300, 768
    blob = _blob(N, K, False, 950 + T)
    b, scales, _ = _repack(blob, N, K, False)
    X = synth.normal_as(951, synth.STREAM_X, T * K, 0.0, 1.0, "f32")
    Y = torch.full((T, N), float("nan"), device="cuda")
    print(f"q8_row T={T}", flush=True)
    qg.qgemm_q8(b, scales, dev(X), Y, N, K, T, "exact")
    torch.cuda.synchronize()
    Yr, S = orc.q8f_gemm(blob, N, K, False, X, "f32", T)
    check_tol(Y.cpu().numpy(), Yr, S, TAU["exact"], f"q8_row T={T}")
