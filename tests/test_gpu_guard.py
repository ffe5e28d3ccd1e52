"""The power-of-two range guard of a half site (qg_x_half_guard; page "cortiq-engine 0.8.3
src/gpu_metal/qi21.rs", Guards / p2) on the GPU against the oracle (oracle.x_half_guard): the f16
values bit for bit, and the guarded rows through the grouped matmul with the guard's factor in the
epilogue, within tau_fast of the oracle's GEMM over the same f16 rows."""
import numpy as np
import pytest
import torch

import block_quantized_weight_affine_amd as qg
import synth
from helpers import TAU, check_tol, dev

pytestmark = pytest.mark.gpu


def _rows(x_rows, K, seed):
    rng = np.random.default_rng(seed)
    X = (rng.normal(0, 1, (x_rows, K)) * np.logspace(-8, 8, x_rows)[:, None]).astype(np.float32)
    X[0, :8] = [1.0, -3.0, 65504.0 * 16, 65520.0 * 16, 2.0**-20, 3.0 * 2.0**-21, 0.0, -0.0]
    X[1, :4] = [np.inf, -np.inf, 1e30, np.nan]
    return X


@pytest.mark.parametrize("shift", [0, 4, 14])
def test_guard_bit_exact(orc, shift):
    x_rows, K = 9, 264
    X = _rows(x_rows, K, 40 + shift)
    src = np.array([0, 1, 8, -1, 3, x_rows, 2, 2, 7, 5, 4], np.int32)
    R = src.size
    Xh = torch.full((R, K), -1, dtype=torch.int16, device="cuda")
    rs = torch.full((R,), float("nan"), device="cuda")
    print(f"guard shift={shift}", flush=True)
    qg.qg_x_half_guard(dev(X), x_rows, dev(src), R, K, shift, Xh, rs)
    torch.cuda.synchronize()
    want, wrs = orc.x_half_guard(X, K, shift, src=src, x_rows=x_rows)
    got = Xh.cpu().numpy().view(np.uint16)
    nan = (want & 0x7C00) == 0x7C00
    nan &= (want & 0x03FF) != 0
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x03FF) != 0)
    assert np.array_equal(rs.cpu().numpy(), wrs)


def test_guard_without_factor_output(orc):
    """rs may be NULL: the f16 rows alone."""
    X = _rows(3, 64, 7)[2:]
    Xh = torch.empty((1, 64), dtype=torch.int16, device="cuda")
    qg.qg_x_half_guard(dev(X), 1, None, 1, 64, 2, Xh, None)
    torch.cuda.synchronize()
    want, _ = orc.x_half_guard(X, 64, 2)
    assert np.array_equal(Xh.cpu().numpy().view(np.uint16), want)


@pytest.mark.parametrize("fmt", ["q4", "q8"])
def test_guarded_rows_through_grouped_matmul(orc, fmt):
    """One expert over 5 guarded rows (shift 6): Y = 2^6 sum w f16(x 2^-6)."""
    N, K, R, shift = 96, 256, 5, 6
    w = synth.make_dense(fmt, N, K, 1, "f32", 1.0, 610)
    X = synth.normal_as(611, synth.STREAM_X, R * K, 0.0, 300.0, "f32").reshape(R, K)
    Xh = torch.empty((R, K), dtype=torch.int16, device="cuda")
    rs = torch.empty((R,), device="cuda")
    qg.qg_x_half_guard(dev(X), R, None, R, K, shift, Xh, rs)
    keep = [(dev(w["codes"]), dev(w["scales"]), None)]  # the table holds raw pointers: keep the tensors
    table = qg.expert_table(keep)
    seg = np.array([0, R], np.int32)
    Y = torch.full((R, N), float("nan"), device="cuda")
    print(f"guarded grouped {fmt}", flush=True)
    qg.qgemm_moe_grouped(fmt, table, 64, dev(seg), None, R, Xh.view(torch.float16), rs, Y, N, K, R, 1, "fast")
    torch.cuda.synchronize()
    xh, _ = orc.x_half_guard(X, K, shift)
    Yr, S, _ = orc.gemm(fmt, w["codes"], w["scales"], None, 64, N, K, xh, "f16", R)
    f = 2.0 ** shift
    check_tol(Y.cpu().numpy(), Yr * f, S * f, TAU["fast"], f"guarded {fmt}")
