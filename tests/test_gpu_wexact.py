"""The W-exact fast mode (QG_FAST_WEXACT) of the dense matmuls against the oracle.

With the codes exact in f16 and X as stored (f16), every product is exact and only f32 sums remain:
each 32-k block's products summed into a block partial, the partial times the block scale, the
results summed over the K / 32 blocks.  Per output that is at most K + K / 16 + 1 roundings of
relative size u = 2^-24 on partial sums bounded by S, so |Y - Y_ref| <= (K + K / 16 + 2) u S -- a
bound for any summation order, far below tau_fast, which the staged (rounded-weight) fast mode
needs."""
import numpy as np
import pytest
import torch

import block_quantized_weight_affine_amd as qg
import synth
from helpers import TAU, check_tol, dev, sample_idx

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def tau_wexact(K: int) -> float:
    return (K + K / 16 + 2) * U


def _run(fmt, w, N, K, T, mode):
    codes, scales = dev(w["codes"]), dev(w["scales"])
    X = dev(w["X"]).view(torch.float16)
    Y = torch.full((T + 2, N), float("nan"), device="cuda")
    if fmt == "q4":
        qg.qgemm_q4(codes, scales, X, Y, N, K, T, mode)
    else:
        qg.qgemm_q8(codes, scales, X, Y, N, K, T, mode)
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    assert np.all(np.isnan(y[T:])), "rows at or beyond T were written"
    return y[:T]


CASES = [
    # fmt, N, K, T: ragged N / T tiles, K % 64 == 32 (a half stage), several stages
    ("q4", 200, 224, 37),
    ("q8", 200, 224, 37),
    ("q4", 520, 1024, 130),
    ("q8", 390, 1056, 70),
    ("q8", 96, 128, 9),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_wexact_matches_oracle(orc, case):
    fmt, N, K, T = case
    w = synth.make_dense(fmt, N, K, T, "f16", 1.0, 1300 + N + K)
    print(f"wexact {case}", flush=True)
    y = _run(fmt, w, N, K, T, "fast_wexact")
    Yr, S, _ = orc.gemm(fmt, w["codes"], w["scales"], None, 64, N, K, w["X"], "f16", T)
    worst = check_tol(y, Yr, S, tau_wexact(K), f"wexact {case}")
    print(f"worst |dY|/S = {worst:.3e} (bound {tau_wexact(K):.3e})")


def test_wexact_q8_prefill_full_size_sampled(orc):
    """The Q8 prefill workload of the benchmark (N = K = 4096, T = 512, f16 X) at sampled outputs."""
    N, K, T = 4096, 4096, 512
    w = synth.make_dense("q8", N, K, T, "f16", 0.5, 1402)
    print("wexact q8 prefill full size", flush=True)
    y = _run("q8", w, N, K, T, "fast_wexact")
    ns, ts = sample_idx(N, 160, 5), sample_idx(T, 24, 6)
    Yr, S, _ = orc.gemm("q8", w["codes"], w["scales"], None, 64, N, K, w["X"], "f16", T, ns=ns, ts=ts)
    check_tol(y[np.ix_(ts, ns)], Yr, S, tau_wexact(K), "wexact q8 prefill")
    assert np.all(np.isfinite(y))


def test_wexact_more_accurate_than_staged(orc):
    """On the same Q8 inputs, the staged fast mode's largest error is larger than the W-exact
    mode's (the rounding of q d to f16 dominates the staged error)."""
    N, K, T = 256, 1024, 64
    w = synth.make_dense("q8", N, K, T, "f16", 1.0, 1501)
    Yr, S, _ = orc.gemm("q8", w["codes"], w["scales"], None, 64, N, K, w["X"], "f16", T)
    e_w = check_tol(_run("q8", w, N, K, T, "fast_wexact"), Yr, S, tau_wexact(K), "wexact")
    e_s = check_tol(_run("q8", w, N, K, T, "fast"), Yr, S, TAU["fast"], "staged")
    print(f"worst |dY|/S: W-exact {e_w:.3e}, staged {e_s:.3e}")
    assert e_w < e_s
