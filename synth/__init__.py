"""Seeded synthetic inputs for the block-quantized matmul workloads.

This module only draws random numbers and stores them in the storage types the
weight and activation layouts use (raw code bytes, f16 / f32 scales, bf16
offsets, f32 / f16 / bf16 activations, f32 router logits).  It holds none of
the method's arithmetic: it never decodes a nibble, never applies a scale and
never multiplies anything.  Both the CPU oracle and the GPU path consume the
arrays it returns.

Generator.  One linear congruential stream per tensor, with the multiplier and
increment the oxinfer `src/metal.rs` tests use for their random inputs (test
helper `rnd`): s <- s * 6364136223846793005 + 1442695040888963407 (mod 2^64),
and a uniform draw u = (s >> 40) / 2^24 in [0, 1).  The stream's first state is
the splitmix64 finaliser of (seed << 16 | stream id), so streams of one seed do
not overlap in practice.  The stream is computed in closed form with affine
jump-ahead, so large tensors cost a few vectorised numpy passes.

Value recipes (each draw u is one LCG output):
  * Q4 code bytes: each draw yields the 24 bits s >> 40, split into three
    bytes, low byte first; every nibble is therefore uniform on 0..15.
  * Q8 codes: floor(255 u) - 127, uniform on -127..127.
  * Uniform [a, b]: a + (b - a) u in f64, rounded to nearest-even into the
    storage type.
  * Normal N(mu, sigma): Box-Muller in f64 from two draws, u1 = ((s >> 40) + 1)
    / 2^24 in (0, 1] and u2 = u: z = sqrt(-2 ln u1) cos(2 pi u2); mu + sigma z is
    rounded to nearest-even into the storage type (bf16 via f32).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "lcg_states", "uniform", "normal", "q4_code_bytes", "q8_codes",
    "f16_uniform", "f32_uniform", "to_bf16_bits", "normal_as",
    "CONFIGS", "Config", "make_dense", "make_moe",
]

_A = 6364136223846793005
_C = 1442695040888963407
_M64 = (1 << 64) - 1


def _splitmix64(x: int) -> int:
    x = (x + 0x9E3779B97F4A7C15) & _M64
    x = ((x ^ (x >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    x = ((x ^ (x >> 27)) * 0x94D049BB133111EB) & _M64
    return x ^ (x >> 31)


def _jump(n: int) -> tuple[int, int]:
    """(A_n, C_n) with s_{i+n} = A_n s_i + C_n (mod 2^64)."""
    an, cn = 1, 0
    ba, bc = _A, _C
    while n:
        if n & 1:
            an, cn = (ba * an) & _M64, (ba * cn + bc) & _M64
        ba, bc = (ba * ba) & _M64, (ba * bc + bc) & _M64
        n >>= 1
    return an, cn


def lcg_states(seed: int, stream: int, n: int) -> np.ndarray:
    """States s_1..s_n (uint64) of the stream (seed, stream)."""
    s0 = _splitmix64(((seed & 0xFFFFFFFFFFFF) << 16) | (stream & 0xFFFF))
    out = np.empty(n, dtype=np.uint64)
    if n == 0:
        return out
    block = min(n, 1 << 16)
    base = np.array([(_A * s0 + _C) & _M64], dtype=np.uint64)
    while base.size < block:
        a, c = _jump(base.size)
        base = np.concatenate([base, base * np.uint64(a) + np.uint64(c)])
    base = base[:block]
    ab, cb = _jump(block)
    aj, cj = 1, 0
    for j0 in range(0, n, block):
        m = min(block, n - j0)
        out[j0:j0 + m] = base[:m] * np.uint64(aj) + np.uint64(cj)
        aj, cj = (ab * aj) & _M64, (ab * cj + cb) & _M64
    return out


def uniform(seed: int, stream: int, n: int) -> np.ndarray:
    """n draws u in [0, 1), f64."""
    return (lcg_states(seed, stream, n) >> np.uint64(40)).astype(np.float64) / float(1 << 24)


def normal(seed: int, stream: int, n: int) -> np.ndarray:
    """n standard normals (f64) by Box-Muller, two draws each (cosine branch)."""
    hi = (lcg_states(seed, stream, 2 * n) >> np.uint64(40)).astype(np.float64)
    u1 = (hi[0::2] + 1.0) / float(1 << 24)
    u2 = hi[1::2] / float(1 << 24)
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)


def q4_code_bytes(seed: int, stream: int, nbytes: int) -> np.ndarray:
    """nbytes uniformly random bytes (two uniform nibbles each), uint8."""
    ndraw = (nbytes + 2) // 3
    v = (lcg_states(seed, stream, ndraw) >> np.uint64(40)).astype(np.uint32)
    b = np.empty((ndraw, 3), dtype=np.uint8)
    b[:, 0] = v & 0xFF
    b[:, 1] = (v >> 8) & 0xFF
    b[:, 2] = (v >> 16) & 0xFF
    return b.reshape(-1)[:nbytes].copy()


def q8_codes(seed: int, stream: int, n: int) -> np.ndarray:
    """n int8 codes uniform on -127..127."""
    u = uniform(seed, stream, n)
    return (np.floor(255.0 * u) - 127.0).astype(np.int8)


def f16_uniform(seed: int, stream: int, n: int, a: float, b: float) -> np.ndarray:
    """Uniform [a, b] rounded to nearest-even f16; returned as raw uint16 bits."""
    u = uniform(seed, stream, n)
    return (a + (b - a) * u).astype(np.float16).view(np.uint16)


def f32_uniform(seed: int, stream: int, n: int, a: float, b: float) -> np.ndarray:
    u = uniform(seed, stream, n)
    return (a + (b - a) * u).astype(np.float32)


def to_bf16_bits(v64: np.ndarray) -> np.ndarray:
    """f64 -> f32 (nearest-even) -> bf16 (nearest-even), raw uint16 bits.

    Finite inputs only (the recipes never produce NaN or Inf)."""
    u = np.ascontiguousarray(v64, dtype=np.float64).astype(np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def normal_as(seed: int, stream: int, n: int, mu: float, sigma: float, storage: str) -> np.ndarray:
    """N(mu, sigma) values in `storage`: 'f32' -> float32, 'f16' -> float16,
    'bf16' -> uint16 bf16 bits."""
    v = mu + sigma * normal(seed, stream, n)
    if storage == "f32":
        return v.astype(np.float32)
    if storage == "f16":
        return v.astype(np.float16)
    if storage == "bf16":
        return to_bf16_bits(v)
    raise ValueError(storage)


# ----------------------------------------------------------------------------------------------
# The five workloads.  Stream ids, in tensor order: 0 codes, 1 scales, 2 offsets, 3 X, 4 logits,
# 5 down codes, 6 down scales.  Seed = 1000 + workload index.

STREAM_CODES, STREAM_SCALES, STREAM_OFFS, STREAM_X, STREAM_LOGITS, STREAM_DCODES, STREAM_DSCALES = range(7)


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    fmt: str            # 'q4' | 'q4a' | 'q8' | 'moe'
    N: int
    K: int
    T: int
    xtype: str          # 'f32' | 'f16' | 'bf16'
    x_sigma: float
    modes: tuple
    group: int = 64
    extra: dict = field(default_factory=dict)

    @property
    def seed(self) -> int:
        return 1000 + self.index


CONFIGS = {
    0: Config(0, "q4_gemm_tiny_N256_K512_T16", "q4", 256, 512, 16, "f32", 1.0, ("exact",)),
    1: Config(1, "q8_gemv_decode_T1_N4096_K4096", "q8", 4096, 4096, 1, "f32", 1.0, ("exact",)),
    2: Config(2, "q4_prefill_N4096_K4096_T512", "q4", 4096, 4096, 512, "f16", 0.5, ("exact", "fast")),
    3: Config(3, "q4a_upproj_N14336_K4096_T1024", "q4a", 14336, 4096, 1024, "bf16", 1.0, ("fast",)),
    4: Config(4, "moe_E128_top8_T32_H2048_I1536", "moe", 2048, 2048, 32, "f32", 1.0, ("exact", "fast"),
              extra={"experts": 128, "top_k": 8, "inter": 1536}),
}


def make_dense(fmt: str, N: int, K: int, T: int, xtype: str, x_sigma: float, seed: int,
               group: int = 64) -> dict:
    """Weights and activations of one dense workload, as host numpy arrays.

    q4 / q4a: codes uint8 [N*K/2], scales f16 bits uint16 [N*K/32] uniform [0.01, 0.05];
    q4a adds offsets bf16 bits uint16 [N*K/group] from N(0, 0.02).
    q8: codes int8 [N*K] uniform -127..127, scales f32 [N*K/32] uniform [0.002, 0.01];
    q8a adds offsets f32 [N*K/32] from N(0, 0.2).
    X: N(0, x_sigma) [T*K] in xtype (f32 / f16 / bf16 bits)."""
    out = {"fmt": fmt, "N": N, "K": K, "T": T, "xtype": xtype, "group": group}
    if fmt in ("q4", "q4a"):
        out["codes"] = q4_code_bytes(seed, STREAM_CODES, N * K // 2)
        out["scales"] = f16_uniform(seed, STREAM_SCALES, N * K // 32, 0.01, 0.05)
        if fmt == "q4a":
            out["offsets"] = normal_as(seed, STREAM_OFFS, N * K // group, 0.0, 0.02, "bf16")
    elif fmt in ("q8", "q8a"):
        out["codes"] = q8_codes(seed, STREAM_CODES, N * K)
        out["scales"] = f32_uniform(seed, STREAM_SCALES, N * K // 32, 0.002, 0.01)
        if fmt == "q8a":
            out["offsets"] = normal_as(seed, STREAM_OFFS, N * K // 32, 0.0, 0.2, "f32")
    else:
        raise ValueError(fmt)
    out["X"] = normal_as(seed, STREAM_X, T * K, 0.0, x_sigma, xtype)
    return out


def make_moe(E: int, H: int, I: int, T: int, seed: int, experts_drawn: int | None = None) -> dict:
    """MoE block inputs: per expert a fused [gate | up] Q4 matrix [2I x H] and a down Q4 matrix
    [H x I], scales uniform [0.01, 0.05]; router logits N(0, 1) f32 [T x E]; X N(0, 1) f32 [T x H].

    Expert e's tensors use the same streams at seed + 7919 * e, so an expert's bytes do not depend
    on how many experts are drawn."""
    ne = E if experts_drawn is None else experts_drawn
    gu_codes = np.empty((ne, 2 * I * H // 2), np.uint8)
    gu_scales = np.empty((ne, 2 * I * H // 32), np.uint16)
    dn_codes = np.empty((ne, H * I // 2), np.uint8)
    dn_scales = np.empty((ne, H * I // 32), np.uint16)
    for e in range(ne):
        s = seed + 7919 * (e + 1)
        gu_codes[e] = q4_code_bytes(s, STREAM_CODES, 2 * I * H // 2)
        gu_scales[e] = f16_uniform(s, STREAM_SCALES, 2 * I * H // 32, 0.01, 0.05)
        dn_codes[e] = q4_code_bytes(s, STREAM_DCODES, H * I // 2)
        dn_scales[e] = f16_uniform(s, STREAM_DSCALES, H * I // 32, 0.01, 0.05)
    return {
        "E": E, "H": H, "I": I, "T": T,
        "gu_codes": gu_codes, "gu_scales": gu_scales,
        "dn_codes": dn_codes, "dn_scales": dn_scales,
        "logits": normal_as(seed, STREAM_LOGITS, T * E, 0.0, 1.0, "f32"),
        "X": normal_as(seed, STREAM_X, T * H, 0.0, 1.0, "f32"),
    }
