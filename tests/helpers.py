"""Shared helpers of the GPU parity tests: device upload of the seeded inputs and the tolerance rule.

Tolerance rule (per element, from the method's statement of the two modes):
    |Y - Y_ref| <= tau * S,  S = sum_k |x_k * w_k|  (x as stored, w the f32 dequantized value),
    tau = 1e-5 (exact mode) or 2e-3 (fast mode); where S == 0, Y must be exactly 0; no NaN / Inf.
"""
import numpy as np
import torch

TAU = {"exact": 1e-5, "fast": 2e-3}

# Relative error of the SwiGLU output a as the chain stores it: the f32 evaluation of
# g / (1 + exp(-g)) * u (a few units in the last place, bounded by 2^-21), plus in fast mode the
# nearest-even f16 rounding of the row-scaled a (2^-11).
RHO_A = {"exact": 2.0 ** -21, "fast": 2.0 ** -11 + 2.0 ** -21}
# The combine sums at most k products in f32 (the combine test's own rule, 1e-6 of sum |w o|), and
# sum_j |w_j o_j| <= b_dn.
RHO_COMBINE = 1e-6


def chain_bound(ref: dict, mode: str) -> np.ndarray:
    """Per-element bound of the MoE chain against the oracle's chain (oracle.moe_ffn): each GEMM
    within tau * S of its own inputs, a stored with relative error RHO_A, the combine within
    RHO_COMBINE: |y - y_ref| <= (tau + RHO_A + RHO_COMBINE) * b_dn + tau * b_gu, to first order."""
    tau = TAU[mode]
    return (tau + RHO_A[mode] + RHO_COMBINE) * ref["b_dn"] + tau * ref["b_gu"]


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> device tensor with the same bytes (uint16 bit patterns travel as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(a).cuda()


def dev_x(X: np.ndarray, xtype: str) -> torch.Tensor:
    t = dev(X)
    if xtype == "bf16":
        return t.view(torch.bfloat16)
    return t


def oracle_x(X: np.ndarray, xtype: str) -> np.ndarray:
    """The activation array as the oracle takes it (16-bit types as raw bits)."""
    if xtype == "f16" and X.dtype == np.float16:
        return X.view(np.uint16)
    return X


def weights_dev(w: dict) -> tuple:
    codes = dev(w["codes"])
    scales = dev(w["scales"])
    offs = dev(w["offsets"]) if "offsets" in w else None
    return codes, scales, offs


def check_tol(Y: np.ndarray, Yref: np.ndarray, S: np.ndarray, tau: float, what: str = ""):
    Y = np.asarray(Y, np.float64)
    assert np.all(np.isfinite(Y)), f"{what}: non-finite output"
    err = np.abs(Y - Yref)
    zero = S == 0
    assert np.all(Y[zero] == 0.0), f"{what}: nonzero output where S == 0"
    ratio = np.where(zero, 0.0, err / np.where(zero, 1.0, S))
    worst = float(ratio.max()) if ratio.size else 0.0
    assert worst <= tau, f"{what}: max |dY|/S = {worst:.3e} > {tau:.1e} at {np.unravel_index(ratio.argmax(), ratio.shape)}"
    return worst


def sample_idx(n: int, m: int, seed: int) -> np.ndarray:
    """m distinct sorted indices of range(n) including the first and last."""
    rng = np.random.default_rng(seed)
    if m >= n:
        return np.arange(n)
    mid = rng.choice(np.arange(1, n - 1), size=m - 2, replace=False)
    return np.sort(np.concatenate([[0, n - 1], mid])).astype(np.int32)
