"""Several weight matrices sharing one X (qgemm_batch) on the GPU: every job's Y against the oracle,
for T = 1 (the jobs' rows walked by one streaming GEMV launch per 8 jobs), T = 2..8 (one K-split GEMV
launch per 8 jobs, a column of workgroups per job) and T = 40 (the tile kernels per job); the batched
rows at T <= 8 also equal single-matrix calls bit for bit (the same per-row arithmetic)."""
import numpy as np
import pytest
import torch

import block_quantized_weight_affine_amd as qg
import synth
from helpers import TAU, check_tol, dev

pytestmark = pytest.mark.gpu


def _jobs(fmt, Ns, K, seed):
    ws = [synth.make_dense(fmt, N, K, 1, "f32", 1.0, seed + i, group=64) for i, N in enumerate(Ns)]
    dw = [(dev(w["codes"]), dev(w["scales"]), dev(w["offsets"]) if "offsets" in w else None) for w in ws]
    return ws, dw


@pytest.mark.parametrize("fmt", ["q4", "q4a", "q8"])
@pytest.mark.parametrize("case", [(1, [96, 160, 32, 48]), (1, [64] * 7 + [32, 96, 16]), (3, [96, 160, 32]),
                                  (2, [4096, 1024, 1024]), (5, [64] * 9 + [34]), (8, [200, 40]),
                                  (40, [128, 64])], ids=lambda c: f"T{c[0]}-J{len(c[1])}")
def test_batch_matches_oracle(orc, fmt, case):
    T, Ns = case
    K = 576   # a multiple of the affine group (64); not of the 1024-value step
    ws, dw = _jobs(fmt, Ns, K, 5000)
    X = synth.normal_as(61, synth.STREAM_X, T * K, 0.0, 1.0, "f32").reshape(T, K)
    Ys = [torch.full((T, N), float("nan"), device="cuda") for N in Ns]
    print(f"batch {fmt} T={T} jobs={Ns}", flush=True)
    qg.qgemm_batch(fmt, 64, [(c, s, o, y, N) for (c, s, o), y, N in zip(dw, Ys, Ns)], dev(X), K, T, "exact")
    torch.cuda.synchronize()
    for i, (w, y, N) in enumerate(zip(ws, Ys, Ns)):
        Yr, S, _ = orc.gemm(fmt, w["codes"], w["scales"], w.get("offsets"), 64, N, K, X, "f32", T)
        check_tol(y.cpu().numpy(), Yr, S, TAU["exact"], f"job {i} (N {N})")
    if T <= 8:
        for (c, s, o), y, N in zip(dw, Ys, Ns):
            y1 = torch.full((T, N), float("nan"), device="cuda")
            if fmt == "q4":
                qg.qgemm_q4(c, s, dev(X), y1, N, K, T, "exact")
            elif fmt == "q4a":
                qg.qgemm_q4a(c, s, o, 64, dev(X), y1, N, K, T, "exact")
            else:
                qg.qgemm_q8(c, s, dev(X), y1, N, K, T, "exact")
            torch.cuda.synchronize()
            assert np.array_equal(y1.cpu().numpy().view(np.uint32), y.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("case", [("q4", 1, 576, "f16", "exact"), ("q8", 1, 576, "bf16", "exact"),
                                  ("q4a", 40, 576, "bf16", "fast"), ("q8", 1, 16416, "f32", "exact"),
                                  ("q4", 4, 576, "f16", "exact"), ("q8a", 6, 1024, "bf16", "exact"),
                                  ("q8", 5, 8224, "f32", "exact")],
                         ids=lambda c: f"{c[0]}-T{c[1]}-K{c[2]}-{c[3]}-{c[4]}")
def test_batch_other_paths(orc, case):
    """16-bit X in the batched T = 1 and T = 2..8 kernels, Q8A jobs, fast mode through the per-job
    tile kernels, and K past the batched kernels' limits (every job then runs the chunked GEMV)."""
    fmt, T, K, xt, mode = case
    Ns = [64, 96, 32]
    ws, dw = _jobs(fmt, Ns, K, 5100)
    X = synth.normal_as(67, synth.STREAM_X, T * K, 0.0, 1.0, xt).reshape(T, K)
    Xd = dev(X)
    if xt == "f16":
        Xd = Xd.view(torch.float16)
    elif xt == "bf16":
        Xd = Xd.view(torch.bfloat16)
    Ys = [torch.full((T, N), float("nan"), device="cuda") for N in Ns]
    print(f"batch {fmt} T={T} K={K} {xt} {mode}", flush=True)
    qg.qgemm_batch(fmt, 64, [(c, s, o, y, N) for (c, s, o), y, N in zip(dw, Ys, Ns)], Xd, K, T, mode)
    torch.cuda.synchronize()
    xo = X.view(np.uint16) if X.dtype == np.float16 else X
    for i, (w, y, N) in enumerate(zip(ws, Ys, Ns)):
        Yr, S, _ = orc.gemm(fmt, w["codes"], w["scales"], w.get("offsets"), 64, N, K, xo, xt, T)
        check_tol(y.cpu().numpy(), Yr, S, TAU[mode], f"job {i} (N {N})")


@pytest.mark.parametrize("T", [1, 4])
def test_batch_qkv_decode_shape_sampled(orc, T):
    """The benchmark's batched q / k / v step (Q8, N 4096 + 1024 + 1024, K 4096, f32 X) at T = 1 and
    T = 4, in its launch configuration: sampled outputs of every job against the oracle."""
    from helpers import sample_idx
    K, Ns = 4096, (4096, 1024, 1024)
    ws = [synth.make_dense("q8", N, K, T, "f32", 1.0, 1001 + 10 * i) for i, N in enumerate(Ns)]
    X = synth.normal_as(1001, synth.STREAM_X, T * K, 0.0, 1.0, "f32").reshape(T, K)
    dw = [(dev(w["codes"]), dev(w["scales"])) for w in ws]
    Ys = [torch.full((T, N), float("nan"), device="cuda") for N in Ns]
    print(f"batch qkv T={T}", flush=True)
    qg.qgemm_batch("q8", 64, [(c, s, None, y, N) for (c, s), y, N in zip(dw, Ys, Ns)], dev(X), K, T, "exact")
    torch.cuda.synchronize()
    for i, (w, y, N) in enumerate(zip(ws, Ys, Ns)):
        ns = sample_idx(N, 96, 20 + i)
        Yr, S, _ = orc.gemm("q8", w["codes"], w["scales"], None, 64, N, K, X, "f32", T, ns=ns)
        yy = y.cpu().numpy()
        check_tol(yy[:, ns], Yr, S, TAU["exact"], f"job {i} (N {N})")
        assert np.all(np.isfinite(yy))
