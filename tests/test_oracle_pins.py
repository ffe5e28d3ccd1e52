"""Pins of the CPU oracle to facts fixed outside it: hand-worked decoder values, IEEE encodings,
library rounding routines, closed forms, exact rational brute force and routing by full sort.

Each test is chosen so that a plausible mistake in the oracle (swapped nibble halves, a dropped
offset, a wrong block or group index, a transposed operand, a wrong tie rule) fails it."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _h(s):
    return int(s, 16)


# ---- 16-bit float encodings ----------------------------------------------------------------------

def test_f16_known_and_all_patterns(orc):
    g = json.load(open(os.path.join(GOLD, "q4a_q8_blocks.json")))
    for bits, val in g["f16_known"]["pairs"]:
        assert orc.f16_values(np.array([_h(bits)], np.uint16))[0] == val
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.f16_values(allb)
    ref = allb.view(np.float16).astype(np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[np.isinf(ref)], ref[np.isinf(ref)])


def test_bf16_known_and_all_patterns(orc):
    g = json.load(open(os.path.join(GOLD, "q4a_q8_blocks.json")))
    for bits, val in g["bf16_known"]["pairs"]:
        assert orc.bf16_values(np.array([_h(bits)], np.uint16))[0] == val
    allb = np.arange(65536, dtype=np.int32).astype(np.int16)
    ref = torch.from_numpy(allb).view(torch.bfloat16).to(torch.float64).numpy()
    ours = orc.bf16_values(allb.view(np.uint16))
    fin = np.isfinite(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))


def _f32_sample(rng, n):
    """Random f32 patterns over all exponents, plus exact halfway points of the f16 and bf16
    grids (ties), the f16 overflow boundary and the subnormal ranges."""
    bits = rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # f16 ties: odd multiples of 2^(e-11) for exponents across the f16 range
    m = rng.integers(0, 2048, 20000)
    e = rng.integers(-25, 16, 20000)
    ties16 = ((2 * m + 1) * np.ldexp(1.0, e - 11)).astype(np.float32)
    # bf16 ties: bit 15 set, bits 0..14 clear
    tb = (rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    tiesb = tb.view(np.float32)
    tiesb = tiesb[np.isfinite(tiesb)]
    edge = np.array([65504, 65519.99, 65520, 65535, 65536, 1e-8, 2.0**-24, 2.0**-25, 3 * 2.0**-26, 2.0**-14,
                     -0.0, 0.0, 1.0, -1.0, 3.4e38, 1e-45, 2.0**-133, 2.0**-134, 3 * 2.0**-135], np.float32)
    return np.concatenate([x, ties16, -ties16, tiesb, edge]).astype(np.float32)


def test_f32_to_f16_matches_numpy(orc):
    rng = np.random.default_rng(5)
    x = _f32_sample(rng, 1 << 20)
    ours = orc.f32_to_f16(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f32_to_bf16_matches_torch(orc):
    rng = np.random.default_rng(6)
    x = _f32_sample(rng, 1 << 20)
    ours = orc.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# ---- decoders against hand-worked blocks -----------------------------------------------------------

def test_q4_hand_packed_blocks(orc):
    g = json.load(open(os.path.join(GOLD, "q4_blocks.json")))
    for c in g["cases"]:
        codes = np.frombuffer(bytes.fromhex(c["bytes_hex"]), np.uint8)
        scales = np.array([_h(c["scale_f16_bits"])], np.uint16)
        got = [orc.weight_exact("q4", codes, scales, None, 64, 1, 32, 0, k) for k in range(32)]
        if c.get("expected") is not None:
            exp = [float(v) for v in c["expected"]]
        else:
            exp = [f * c["scale_value"] for f in c["expected_factor"]]
        assert got == exp, c["name"]
        v32 = orc.dequant_tile("q4", codes, scales, None, 64, 1, 32, 0, 0, 1, 32, "f32")[0]
        assert [float(v) for v in v32] == exp, c["name"]


def test_q4_block_and_row_addressing(orc):
    """Two rows of two blocks with distinct scales: element (n, k) must use block k // 32 of row n."""
    ramp = bytes.fromhex("f0e1d2c3b4a5968778695a4b3c2d1e0f")
    zero = bytes(16)
    codes = np.frombuffer(ramp + zero + zero + ramp, np.uint8)    # row 0: [ramp, zero], row 1: [zero, ramp]
    scales = np.array([0x3C00, 0x4000, 0x4200, 0x4400], np.uint16)  # 1, 2, 3, 4
    fac = list(range(-8, 8)) + list(range(7, -9, -1))
    W = orc.dequant_exact("q4", codes, scales, None, 64, 2, 64)
    assert list(W[0, :32]) == [1.0 * f for f in fac]
    assert list(W[0, 32:]) == [-16.0] * 32
    assert list(W[1, :32]) == [-24.0] * 32
    assert list(W[1, 32:]) == [4.0 * f for f in fac]


def test_q4a_hand_packed(orc):
    g = json.load(open(os.path.join(GOLD, "q4a_q8_blocks.json")))
    for c in g["q4a_cases"]:
        K, group = c["K"], c["group"]
        codes = np.frombuffer(b"".join(bytes.fromhex(h) for h in c["bytes_hex_per_block"]), np.uint8)
        scales = np.array([_h(s) for s in c["scales_f16_bits"]], np.uint16)
        offs = np.array([_h(s) for s in c["offsets_bf16_bits"]], np.uint16)
        W = orc.dequant_exact("q4a", codes, scales, offs, group, 1, K)[0]
        if "expected_group_values" in c:
            for gi, v in enumerate(c["expected_group_values"]):
                assert list(W[gi * group:(gi + 1) * group]) == [v] * group, c["name"]
        else:
            for b, v in enumerate(c["expected_block_values"]):
                assert list(W[b * 32:(b + 1) * 32]) == [v] * 32, c["name"]
        v32 = orc.dequant_tile("q4a", codes, scales, offs, group, 1, K, 0, 0, 1, K, "f32")[0]
        assert np.array_equal(v32.astype(np.float64), W)


def test_q8_hand_codes(orc):
    g = json.load(open(os.path.join(GOLD, "q4a_q8_blocks.json")))
    for c in g["q8_cases"]:
        codes = np.array(c["codes"], np.int8)
        scales = np.array([c["scale"]], np.float32)
        W = orc.dequant_exact("q8", codes, scales, None, 64, 1, 32)[0]
        assert list(W) == c["expected"]
    # block indexing: K = 64, second block has its own scale
    codes = np.full(64, 3, np.int8)
    scales = np.array([0.5, -0.25], np.float32)
    W = orc.dequant_exact("q8", codes, scales, None, 64, 1, 64)[0]
    assert list(W) == [1.5] * 32 + [-0.75] * 32


def test_staged_f32_rounding_q8_q4a(orc):
    """The f32 decode rounds once: q * d (Q8) and (nib-8) * d + m (Q4A), nearest-even in f32."""
    rng = np.random.default_rng(11)
    N, K = 3, 64
    codes8 = rng.integers(-127, 128, N * K).astype(np.int8)
    sc8 = rng.uniform(0.002, 0.01, N * K // 32).astype(np.float32)
    v = orc.dequant_tile("q8", codes8, sc8, None, 64, N, K, 0, 0, N, K, "f32")
    ref = codes8.reshape(N, K).astype(np.float32) * np.repeat(sc8.reshape(N, K // 32), 32, axis=1)
    assert np.array_equal(v, ref)
    codes4 = rng.integers(0, 256, N * K // 2).astype(np.uint8)
    sc4 = rng.uniform(0.01, 0.05, N * K // 32).astype(np.float16).view(np.uint16)
    off = torch.from_numpy(rng.normal(0, 0.02, N * K // 64).astype(np.float32)).to(torch.bfloat16)
    offb = off.view(torch.int16).numpy().view(np.uint16)
    v = orc.dequant_tile("q4a", codes4, sc4, offb, 64, N, K, 0, 0, N, K, "f32")
    nib = np.empty((N, K), np.int32)
    cb = codes4.reshape(N, K // 32, 16)
    nib[:, :] = np.concatenate([cb & 15, cb >> 4], axis=2).reshape(N, K)
    d = np.repeat(sc4.view(np.float16).astype(np.float32).reshape(N, K // 32), 32, axis=1)
    m = np.repeat(off.to(torch.float32).numpy().reshape(N, K // 64), 64, axis=1)
    prod = (nib - 8).astype(np.float32) * d
    assert np.array_equal(v, prod + m)
    # and the fast-mode tiles are nearest-even narrowings of exactly these f32 values
    t16 = orc.dequant_tile("q4a", codes4, sc4, offb, 64, N, K, 0, 0, N, K, "f16")
    assert np.array_equal(t16, (prod + m).astype(np.float16).view(np.uint16))
    tb = orc.dequant_tile("q4a", codes4, sc4, offb, 64, N, K, 0, 0, N, K, "bf16")
    refb = torch.from_numpy(prod + m).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(tb, refb)


# ---- GEMM ------------------------------------------------------------------------------------------

def _frac_f16(bits):
    s = -1 if bits >> 15 else 1
    e = (bits >> 10) & 31
    f = bits & 1023
    if e == 0:
        return s * Fraction(f, 1 << 24)
    return s * Fraction(f + 1024, 1 << 10) * (Fraction(2) ** (e - 15))


@pytest.mark.parametrize("fmt", ["q4", "q8"])
def test_gemm_brute_force_rationals(orc, fmt):
    """Tiny shapes: Y from the raw bytes in exact rationals (Q4 values are exact; Q8 values are
    the f32 products, rounded by numpy's IEEE f32 multiply); the oracle's f64 sums must agree to
    f64 rounding (K terms: |err| <= K * 2^-52 * S)."""
    rng = np.random.default_rng(3)
    for (N, K, T) in [(3, 32, 2), (4, 64, 3), (1, 64, 1)]:
        if fmt == "q4":
            codes = rng.integers(0, 256, N * K // 2).astype(np.uint8)
            scales = rng.uniform(0.01, 0.05, N * K // 32).astype(np.float16).view(np.uint16)
        else:
            codes = rng.integers(-127, 128, N * K).astype(np.int8)
            scales = rng.uniform(0.002, 0.01, N * K // 32).astype(np.float32)
        X = rng.normal(0, 1, T * K).astype(np.float32)
        Y, S, _ = orc.gemm(fmt, codes, scales, None, 64, N, K, X, "f32", T, threads=1)
        for t in range(T):
            for n in range(N):
                acc = Fraction(0)
                for k in range(K):
                    b = k // 32
                    if fmt == "q4":
                        byte = int(codes[n * K // 2 + 16 * b + (k % 32) % 16])
                        nib = byte & 15 if (k % 32) < 16 else byte >> 4
                        w = (nib - 8) * _frac_f16(int(scales[n * K // 32 + b]))
                    else:
                        # the decoder evaluates q * d in f32 (one nearest-even rounding)
                        w = Fraction(float(np.float32(int(codes[n * K + k])) * np.float32(scales[n * K // 32 + b])))
                    acc += Fraction(float(X[t * K + k])) * w
                assert abs(Fraction(Y[t, n]) - acc) <= Fraction(K) * Fraction(2) ** -52 * Fraction(S[t, n])


def test_gemm_identity_and_one_hot(orc):
    K = N = 64
    # identity: nibble 9 on the diagonal, 8 elsewhere, scale 1.0 -> W = I, so Y = X exactly
    nib = np.full((N, K), 8, np.uint8)
    np.fill_diagonal(nib, 9)
    codes = np.empty((N, K // 32, 16), np.uint8)
    nb = nib.reshape(N, K // 32, 32)
    codes[:] = nb[:, :, :16] | (nb[:, :, 16:] << 4)
    scales = np.full(N * K // 32, 0x3C00, np.uint16)
    X = np.random.default_rng(1).normal(0, 1, (5, K)).astype(np.float32)
    Y, S, _ = orc.gemm("q4", codes.reshape(-1), scales, None, 64, N, K, X, "f32", 5)
    assert np.array_equal(Y, X.astype(np.float64))
    assert np.array_equal(S, np.abs(X.astype(np.float64)))
    # one-hot: a single nonzero weight at (n*, k*) = (17, 40): nibble 15, scale 0.25 -> 1.75
    nib = np.full((N, K), 8, np.uint8)
    nib[17, 40] = 15
    nb = nib.reshape(N, K // 32, 32)
    codes[:] = nb[:, :, :16] | (nb[:, :, 16:] << 4)
    scales = np.full(N * K // 32, 0x3400, np.uint16)
    Y, _, _ = orc.gemm("q4", codes.reshape(-1), scales, None, 64, N, K, X, "f32", 5)
    exp = np.zeros((5, N))
    exp[:, 17] = X[:, 40].astype(np.float64) * 1.75
    assert np.array_equal(Y, exp)


def test_gemm_orientation_one_hot_tokens(orc):
    """x[t][k] = [k == t] makes Y[t][n] = w[n][t]: pins Y = X W^T, not its transpose."""
    rng = np.random.default_rng(8)
    N, K, T = 6, 64, 5
    codes = rng.integers(0, 256, N * K // 2).astype(np.uint8)
    scales = rng.uniform(0.01, 0.05, N * K // 32).astype(np.float16).view(np.uint16)
    W = orc.dequant_exact("q4", codes, scales, None, 64, N, K)
    X = np.zeros((T, K), np.float32)
    for t in range(T):
        X[t, t] = 1.0
    Y, _, _ = orc.gemm("q4", codes, scales, None, 64, N, K, X, "f32", T)
    assert np.array_equal(Y, W[:, :T].T)


def test_gemm_closed_form_constant_blocks(orc):
    """Every nibble of block b of row n equal to c[n][b] and x = 1: Y[n] = 32 sum_b (c-8) d + 64 sum_g m."""
    rng = np.random.default_rng(4)
    N, K = 5, 256
    c = rng.integers(0, 16, (N, K // 32))
    codes = np.repeat((c | (c << 4)).astype(np.uint8), 16, axis=1).reshape(-1)
    scales = rng.uniform(0.01, 0.05, N * K // 32).astype(np.float16).view(np.uint16)
    offs = torch.from_numpy(rng.normal(0, 0.02, N * K // 64).astype(np.float32)).to(torch.bfloat16)
    offb = offs.view(torch.int16).numpy().view(np.uint16)
    X = np.ones((1, K), np.float32)
    d = scales.view(np.float16).astype(np.float64).reshape(N, K // 32)
    m = offs.to(torch.float64).numpy().reshape(N, K // 64)
    Y, _, _ = orc.gemm("q4", codes, scales, None, 64, N, K, X, "f32", 1)
    assert np.allclose(Y[0], 32 * ((c - 8) * d).sum(1), rtol=1e-14, atol=0)
    Y, _, _ = orc.gemm("q4a", codes, scales, offb, 64, N, K, X, "f32", 1)
    # each element rounds to f32 once; compare within that rounding
    exact = 32 * ((c - 8) * d).sum(1) + 64 * m.sum(1)
    assert np.allclose(Y[0], exact, rtol=0, atol=K * 2.0**-24 * 0.5)


def test_gemm_x_storage_types(orc):
    """f16 and bf16 activations are widened exactly; the result equals the f32-typed call."""
    rng = np.random.default_rng(9)
    N, K, T = 4, 64, 3
    codes = rng.integers(0, 256, N * K // 2).astype(np.uint8)
    scales = rng.uniform(0.01, 0.05, N * K // 32).astype(np.float16).view(np.uint16)
    x16 = rng.normal(0, 1, T * K).astype(np.float16)
    Ya, _, _ = orc.gemm("q4", codes, scales, None, 64, N, K, x16.view(np.uint16), "f16", T)
    Yb, _, _ = orc.gemm("q4", codes, scales, None, 64, N, K, x16.astype(np.float32), "f32", T)
    assert np.array_equal(Ya, Yb)
    xb = torch.from_numpy(rng.normal(0, 1, T * K).astype(np.float32)).to(torch.bfloat16)
    Ya, _, _ = orc.gemm("q4", codes, scales, None, 64, N, K, xb.view(torch.int16).numpy().view(np.uint16), "bf16", T)
    Yb, _, _ = orc.gemm("q4", codes, scales, None, 64, N, K, xb.to(torch.float32).numpy(), "f32", T)
    assert np.array_equal(Ya, Yb)


def test_gemm_sampled_matches_full(orc):
    rng = np.random.default_rng(10)
    N, K, T = 40, 128, 7
    codes = rng.integers(-127, 128, N * K).astype(np.int8)
    scales = rng.uniform(0.002, 0.01, N * K // 32).astype(np.float32)
    X = rng.normal(0, 1, T * K).astype(np.float32)
    Yf, Sf, _ = orc.gemm("q8", codes, scales, None, 64, N, K, X, "f32", T, threads=3)
    ns, ts = np.array([39, 0, 17]), np.array([6, 2])
    Ys, Ss, _ = orc.gemm("q8", codes, scales, None, 64, N, K, X, "f32", T, ns=ns, ts=ts)
    assert np.array_equal(Ys, Yf[np.ix_(ts, ns)])
    assert np.array_equal(Ss, Sf[np.ix_(ts, ns)])


# ---- row scaling to f16 -------------------------------------------------------------------------------

def test_x_half_closed_forms(orc):
    K = 8
    X = np.array([
        [1.0, -0.5, 0.25, 0, 0, 0, 0, 0],          # amax 1 = 0.5 * 2^1 -> scale 2^13
        [3.0, 1.0, 0, 0, 0, 0, 0, 0],              # amax 3 = 0.75 * 2^2 -> scale 2^12
        [0, 0, 0, 0, 0, 0, 0, 0],                  # zero row -> scale 1
        [2.0**-120, 0, 0, 0, 0, 0, 0, 0],          # frexp exponent -119 -> 14 + 119 clamped to 100
        [np.inf, 1.0, 0, 0, 0, 0, 0, 0],           # non-finite amax -> scale 1
    ], np.float32)
    xh, rs = orc.x_half(X, K)
    assert list(rs) == [2.0**-13, 2.0**-12, 1.0, 2.0**-100, 1.0]
    v = xh.view(np.float16).astype(np.float64)
    assert list(v[0, :3]) == [8192.0, -4096.0, 2048.0]
    assert list(v[1, :2]) == [12288.0, 4096.0]
    assert not v[2].any()
    assert v[3, 0] == 2.0**-20
    assert v[4, 0] == np.inf and v[4, 1] == 1.0
    # gather: row r is source row src[r]
    xh2, rs2 = orc.x_half(X, K, src=np.array([1, 0, 1]))
    assert np.array_equal(xh2[0], xh[1]) and np.array_equal(xh2[1], xh[0]) and list(rs2) == [2.0**-12, 2.0**-13, 2.0**-12]


def test_x_half_range_random(orc):
    rng = np.random.default_rng(12)
    X = (rng.normal(0, 1, (50, 96)) * np.logspace(-6, 6, 50)[:, None]).astype(np.float32)
    xh, rs = orc.x_half(X, 96)
    v = xh.view(np.float16).astype(np.float64)
    amax = np.abs(v).max(1)
    assert np.all(amax >= 2.0**13) and np.all(amax < 2.0**14 + 1)
    assert np.all(np.log2(rs) == np.round(np.log2(rs)))
    back = v * rs[:, None]
    assert np.all(np.abs(back - X) <= 2.0**-11 * np.abs(X) + 1e-300)


# ---- q8_2f / q8_row -----------------------------------------------------------------------------------

def _q8f_blob(codes, rs_bits, col_bits=None):
    parts = [np.asarray(codes, np.int8).view(np.uint8).ravel(), np.asarray(rs_bits, "<u2").view(np.uint8)]
    if col_bits is not None:
        parts.append(np.asarray(col_bits, "<u2").view(np.uint8))
    return np.concatenate(parts)


def test_q8f_hand_worked(orc):
    """A 2 x 4 q8_2f tensor worked by hand (page cortiq-engine 0.8.3 qi21.rs, the codec match: codes,
    then f16 row scales, then the f16 column field): w = q col[k] rs[n]."""
    codes = [[3, -2, 0, 127], [-128, 1, 5, -1]]
    rs = [0x3800, 0xC000]                     # 0.5, -2
    col = [0x3C00, 0x3400, 0x4200, 0x0001]    # 1, 0.25, 3, 2^-24
    X = np.array([[2.0, 4.0, 1.0, 2.0**20]], np.float32)
    blob = _q8f_blob(codes, rs, col)
    r, c = orc.q8f_fields(blob, 2, 4, True)
    assert list(r) == [0.5, -2.0] and list(c) == [1.0, 0.25, 3.0, 2.0**-24]
    Y, S = orc.q8f_gemm(blob, 2, 4, True, X, "f32", 1)
    # row 0: 2*1.5 + 4*(-0.25) + 0 + 2^20 * 127 * 2^-25;  row 1: 2*256 + 4*(-0.5) + 1*(-30) + 2^20 * 2^-23
    assert list(Y[0]) == [5.96875, 480.125] and list(S[0]) == [7.96875, 544.125]
    # q8_row: the same codes and row scales, no column field
    Yr, Sr = orc.q8f_gemm(_q8f_blob(codes, rs), 2, 4, False, X, "f32", 1)
    # row 0: w = 1.5, -1, 0, 63.5;  row 1: w = 256, -2, -10, 2
    assert list(Yr[0]) == [2 * 1.5 - 4 * 1.0 + 2.0**20 * 63.5, 2 * 256.0 - 4 * 2.0 - 10.0 + 2.0**21]
    assert list(Sr[0]) == [3 + 4 + 2.0**20 * 63.5, 512 + 8 + 10 + 2.0**21]


def test_q8f_reduces_to_q8(orc):
    """q8_row is Q8 with the row scale in every block (bit for bit, Y and S), and q8_2f is q8_row over
    X times the column field (each product is the exact product rounded once in f64)."""
    rng = np.random.default_rng(21)
    N, K, T = 5, 96, 3
    codes = rng.integers(-128, 128, (N, K)).astype(np.int8)
    rs = synth.f16_uniform(22, 1, N, -2.0, 2.0)
    col = synth.f16_uniform(22, 2, K, 0.0, 4.0)
    X = rng.normal(0, 1, (T, K)).astype(np.float32)
    Yr, Sr = orc.q8f_gemm(_q8f_blob(codes, rs), N, K, False, X, "f32", T)
    rsv, _ = orc.q8f_fields(_q8f_blob(codes, rs), N, K, False)
    scales = np.repeat(rsv.astype(np.float32), K // 32)
    Yq, Sq, _ = orc.gemm("q8", codes, scales, None, 64, N, K, X, "f32", T)
    assert np.array_equal(Yr, Yq) and np.array_equal(Sr, Sq)
    _, colv = orc.q8f_fields(_q8f_blob(codes, rs, col), N, K, True)
    Yf, Sf = orc.q8f_gemm(_q8f_blob(codes, rs, col), N, K, True, X, "f32", T)
    Yc, Sc = orc.q8f_gemm(_q8f_blob(codes, rs), N, K, False, X.astype(np.float64) * colv, "f64", T)
    assert np.array_equal(Yf, Yc) and np.array_equal(Sf, Sc)


def test_col_scale_closed_forms(orc):
    """The column field on X: the f32 product (IEEE round to nearest), then nearest-even narrowing."""
    X = np.array([[3.0, 1 + 2.0**-10, 1 + 2.0**-23, -2.0, 65504.0, 1e-8, 0.0, -0.0]], np.float32)
    col = np.array([0.5, 1 + 2.0**-11, 1 + 2.0**-23, 0.25, 2.0, 1.0, 5.0, 5.0], np.float32)
    f = orc.col_scale(X, "f32", 1, 8, col, "f32")[0]
    # (1 + 2^-10)(1 + 2^-11) is exact in f32; (1 + 2^-23)^2 = 1 + 2^-22 + 2^-46 rounds to 1 + 2^-22
    assert list(f) == [1.5, 1 + 2.0**-10 + 2.0**-11 + 2.0**-21, 1 + 2.0**-22, -0.5, 131008.0,
                       float(np.float32(1e-8)), 0.0, 0.0]
    assert np.signbit(f[7]) and not np.signbit(f[6])
    h = orc.col_scale(X, "f32", 1, 8, col, "f16")[0]
    # 1 + 1.5 2^-10 + 2^-21 is past the midpoint: up to 1 + 2^-9; 131008 overflows; 1e-8 < 2^-25
    assert [int(v) for v in h] == [0x3E00, 0x3C02, 0x3C00, 0xB800, 0x7C00, 0x0000, 0x0000, 0x8000]
    b = orc.col_scale(X, "f32", 1, 8, col, "bf16")[0]
    # bf16 keeps 7 fraction bits: 131008 = 0x47FFE000 rounds up to 0x4800; 1e-8 = 0x322BCC77 to 0x322C
    assert [int(v) for v in b] == [0x3FC0, 0x3F80, 0x3F80, 0xBF00, 0x4800, 0x322C, 0x0000, 0x8000]
    # f16 input: the f16 value is exact in f32
    xh = np.array([[0x3C01, 0xC000]], np.uint16)          # 1 + 2^-10, -2
    assert list(orc.col_scale(xh, "f16", 1, 2, np.array([2.0, 0.5], np.float32), "f32")[0]) == [2 + 2.0**-9, -1.0]


def test_x_half_guard_closed_forms(orc):
    """The fixed power-of-two guard (page cortiq-engine 0.8.3 qi21.rs, Guards / p2): x 2^-s to f16,
    nearest-even, overflow to infinity, factor 2^s.  Values worked by hand for s = 4."""
    K = 8
    X = np.array([
        [1.0, -3.0, 65504.0 * 16, 65520.0 * 16, 2.0**-20, 3.0 * 2.0**-21, 0.0, -0.0],
        [1e30, -1e30, 3.0 * 2.0**-26, 2.0**-21, 0.5, 6.0, 7.0, 8.0],
    ], np.float32)
    xh, rs = orc.x_half_guard(X, K, 4)
    assert list(rs) == [16.0, 16.0]
    want0 = [0x2C00,   # 2^-4
             0xB200,   # -0.1875 = -1.5 2^-3
             0x7BFF,   # 65504, the largest f16
             0x7C00,   # 65520 is halfway to 65536: nearest-even gives 2^16, infinity
             0x0001,   # 2^-24, the smallest subnormal
             0x0002,   # 1.5 2^-24: a tie, to the even subnormal 2
             0x0000, 0x8000]
    want1 = [0x7C00, 0xFC00,
             0x0000,   # 3 2^-30 < 2^-25: rounds to zero
             0x0000,   # 2^-25, halfway to the smallest subnormal: a tie to even zero
             0x2800,   # 2^-5
             0x3600,   # 0.375 = 1.5 2^-2
             0x3700,   # 0.4375 = 1.75 2^-2
             0x3800]   # 0.5
    assert list(xh[0]) == want0 and list(xh[1]) == want1
    # shift 0 is the plain conversion; the gather reads zeros outside [0, x_rows)
    xh0, rs0 = orc.x_half_guard(X[:, 4:], 4, 0)
    assert xh0[1, 0] == 0x3800 and list(rs0) == [1.0, 1.0]
    xg, rg = orc.x_half_guard(X, K, 4, src=np.array([1, -1, 2, 0]), x_rows=2)
    assert np.array_equal(xg[0], xh[1]) and np.array_equal(xg[3], xh[0])
    assert not xg[1].any() and not xg[2].any() and list(rg) == [16.0] * 4


def test_x_half_guard_matches_row_scaling(orc):
    """When a row's own power-of-two scale is 2^-s (amax in [2^(13+s), 2^(14+s))), the guard and the
    per-row scaling store the same f16 values and the same factor."""
    rng = np.random.default_rng(5)
    for s in (0, 3, 9, 14):
        X = rng.uniform(-1, 1, (6, 64)).astype(np.float32) * np.float32(2.0 ** (13 + s))
        X[:, 0] = np.float32(1.5 * 2.0 ** (13 + s))
        xg, rg = orc.x_half_guard(X, 64, s)
        xr, rr = orc.x_half(X, 64)
        assert np.array_equal(xg, xr) and np.array_equal(rg, rr), s


def test_swiglu_closed_forms(orc):
    g = np.array([0.0, math.log(3.0), -50.0, 2.0])
    u = np.array([5.0, 2.0, 3.0, 1.0])
    a = orc.swiglu(g, u)
    assert a[0] == 0.0
    assert abs(a[1] - 0.75 * math.log(3.0) * 2.0) < 1e-15
    assert abs(a[2]) < 1e-19
    assert abs(a[3] - 2.0 / (1.0 + math.exp(-2.0))) < 1e-15


# ---- routing plan and combine --------------------------------------------------------------------------

def test_moe_plan_brute_force(orc):
    rng = np.random.default_rng(13)
    T, E, k = 32, 128, 8
    lg = rng.normal(0, 1, (T, E)).astype(np.float32)
    lg[3, 10] = lg[3, 20] = lg[3, 30] = 9.0      # a three-way tie at the top
    lg[4, :] = 0.5                               # all equal: experts 0..7 in order
    p = orc.moe_plan(lg, T, E, k)
    assert p["R"] == T * k
    seg, src, srow, sw, se = p["seg_off"], p["row_src"], p["slot_row"], p["slot_w"], p["slot_expert"]
    assert seg[0] == 0 and seg[-1] == T * k and np.all(np.diff(seg) >= 0)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))[:k]
        assert list(se[t * k:(t + 1) * k]) == order
        ex = np.exp(lg[t, order].astype(np.float64) - float(lg[t, order[0]]))
        assert np.allclose(sw[t * k:(t + 1) * k], ex / ex.sum(), rtol=1e-15, atol=0)
        assert abs(sw[t * k:(t + 1) * k].sum() - 1.0) < 1e-15
        for j, e in enumerate(order):
            r = srow[t * k + j]
            assert seg[e] <= r < seg[e + 1] and src[r] == t
    assert list(se[3 * k:3 * k + 3]) == [10, 20, 30]
    assert list(se[4 * k:5 * k]) == list(range(8))
    assert np.allclose(sw[4 * k:5 * k], 1.0 / 8, rtol=0, atol=1e-16)
    for e in range(E):
        rows = src[seg[e]:seg[e + 1]]
        assert np.all(np.diff(rows) > 0)                 # ascending tokens within a segment
        assert len(rows) == sum(e in se[t * k:(t + 1) * k] for t in range(T))


def test_moe_combine_closed_forms(orc):
    O = np.arange(12, dtype=np.float64).reshape(3, 4)
    y, b = orc.moe_combine(O, 4, np.array([2]), np.array([1.0]), 1, 1)
    assert np.array_equal(y[0], O[2])
    y, b = orc.moe_combine(O, 4, np.array([0, 1, 1, 2]), np.array([0.7, 0.3, 0.25, -0.5]), 2, 2)
    assert np.allclose(y[0], 0.7 * O[0] + 0.3 * O[1], rtol=1e-15)
    assert np.allclose(y[1], 0.25 * O[1] - 0.5 * O[2], rtol=1e-15)
    assert np.allclose(b[1], 0.25 * O[1] + 0.5 * O[2], rtol=1e-15)


# ---- GGUF blocks with in-block scales (oxinfer src/metal.rs, SHADER_SRC, Q4_0W and Q8_0W) ---------
def _gguf_q4_0_block(d_bits, nib_bytes):
    return np.concatenate([[d_bits & 0xFF, d_bits >> 8], nib_bytes]).astype(np.uint8)


def test_gguf_q4_0_hand_blocks(orc):
    """Two rows of two blocks, values worked by hand: block = f16 scale then 16 bytes whose low
    nibble is element j and high nibble element j + 16; value (nibble - 8) * d."""
    nib = np.full(16, 0x88, np.uint8)
    nib[0], nib[15] = 0xF0, 0x1F
    b00 = _gguf_q4_0_block(0x3800, nib)                      # d = 0.5
    b01 = _gguf_q4_0_block(0xC000, np.full(16, 0xFF, np.uint8))  # d = -2, every nibble 15
    b10 = _gguf_q4_0_block(0x3C00, np.zeros(16, np.uint8))   # d = 1, every nibble 0
    b11 = _gguf_q4_0_block(0x0001, np.full(16, 0x9A, np.uint8))  # d = 2^-24 (subnormal), nibbles 10 / 9
    src = np.concatenate([b00, b01, b10, b11])
    w = orc.gguf_dequant("q4_0", src, 2, 64)
    exp0 = np.zeros(32)
    exp0[0], exp0[16], exp0[15], exp0[31] = -4.0, 3.5, 3.5, -3.5
    assert np.array_equal(w[0, :32], exp0)
    assert np.all(w[0, 32:] == -14.0)                        # (15 - 8) * -2
    assert np.all(w[1, :32] == -8.0)
    assert np.all(w[1, 32:48] == 2.0 * 2.0 ** -24) and np.all(w[1, 48:] == 1.0 * 2.0 ** -24)


def test_gguf_q8_0_hand_block(orc):
    """Q8_0: f16 scale then 32 signed bytes; value q * d."""
    q = np.zeros(32, np.int8)
    q[0], q[1], q[2], q[31] = 127, -128, -1, 5
    src = np.concatenate([[0x00, 0x34], q.view(np.uint8)]).astype(np.uint8)   # d = 0.25
    w = orc.gguf_dequant("q8_0", src, 1, 32)
    exp = np.zeros(32)
    exp[0], exp[1], exp[2], exp[31] = 31.75, -32.0, -0.25, 1.25
    assert np.array_equal(w[0], exp)


@pytest.mark.parametrize("gtype", ["q4_0", "q8_0"])
def test_gguf_repack_matches_direct_decode(orc, gtype):
    """The split-layout repack, decoded by the Q4 / Q8 decoders, gives every GGUF element's value
    bit for bit (two independent paths: the in-block decoder and the split-layout decoder)."""
    rng = np.random.default_rng(5)
    N, K = 5, 128
    nb = N * K // 32
    bb = orc.GGUF_BLOCK_BYTES[gtype]
    src = rng.integers(0, 256, nb * bb).astype(np.uint8).reshape(nb, bb)
    d = synth.f16_uniform(9, 1, nb, -0.05, 0.05)                # negative scales too
    src[:, 0], src[:, 1] = d & 0xFF, d >> 8
    src = src.reshape(-1)
    codes, scales = orc.gguf_repack(gtype, src, N, K)
    direct = orc.gguf_dequant(gtype, src, N, K)
    fmt = "q4" if gtype == "q4_0" else "q8"
    split = orc.dequant_tile(fmt, codes, scales, None, 64, N, K, 0, 0, N, K, "f32")
    assert np.array_equal(direct.view(np.uint32), split.view(np.uint32))


# ---- the MoE chain (oxinfer src/metal.rs, Backend::moe and the reference loop of its test
# mma_moe_matches_cpu: gate = the first I rows of the fused matrix, up = the next I) -------------
def _pack_nibbles(nib):
    """Nibble matrix [N][K] -> Q4 code bytes (byte j of block b: element 32b+j low, 32b+16+j high),
    written out here by hand so the pins do not depend on any packing helper."""
    N, K = nib.shape
    out = np.zeros((N, K // 2), np.uint8)
    for n in range(N):
        for b in range(K // 32):
            for j in range(16):
                out[n, 16 * b + j] = nib[n, 32 * b + j] | (nib[n, 32 * b + 16 + j] << 4)
    return out.reshape(-1)


def _diag_q4(rows, cols, pairs):
    """Q4 matrix with weight 0 (nibble 8) except w[r][c] = v for (r, c, v) in pairs; scale 1."""
    nib = np.full((rows, cols), 8, np.uint8)
    for r, c, v in pairs:
        nib[r, c] = 8 + v
    return _pack_nibbles(nib), np.full(rows * cols // 32, 0x3C00, np.uint16)


def _silu(x):
    return x / (1.0 + math.exp(-x))


def _moe_identity(E, H, down_gain, fmt="q4"):
    """E experts with I = H: gate = identity, up = 2 * identity, down = down_gain[e] * identity."""
    I = H
    gu_c, gu_s, dn_c, dn_s = [], [], [], []
    for e in range(E):
        if fmt == "q4":
            c, s = _diag_q4(2 * I, H, [(i, i, 1) for i in range(I)] + [(I + i, i, 2) for i in range(I)])
            gu_c.append(c), gu_s.append(s)
            c, s = _diag_q4(H, I, [(i, i, down_gain[e]) for i in range(H)])
            dn_c.append(c), dn_s.append(s)
        else:   # Q8: int8 codes, f32 scale 1
            g = np.zeros((2 * I, H), np.int8)
            g[np.arange(I), np.arange(I)] = 1
            g[I + np.arange(I), np.arange(I)] = 2
            d = np.zeros((H, I), np.int8)
            d[np.arange(H), np.arange(H)] = down_gain[e]
            gu_c.append(g.reshape(-1)), gu_s.append(np.ones(2 * I * H // 32, np.float32))
            dn_c.append(d.reshape(-1)), dn_s.append(np.ones(H * I // 32, np.float32))
    return np.array(gu_c), np.array(gu_s), np.array(dn_c), np.array(dn_s)


@pytest.mark.parametrize("fmt", ["q4", "q8"])
def test_moe_chain_closed_form(orc, fmt):
    """Identity gate, doubled identity up, and down = 1x (expert 0) or 3x (expert 1) identity:
    every routed row gives o = a = SiLU(x) * 2x (times the gain), so with router logits (0, ln 3)
    the weights are 1/4 and 3/4 and y = (3/4 * 3 + 1/4 * 1) * SiLU(x) * 2x = 2.5 * 2x SiLU(x).
    Swapping gate and up would give SiLU(2x) * x instead, which differs clearly for 0 < |x| <= 4."""
    E, H, T, k = 2, 32, 3, 2
    gu_c, gu_s, dn_c, dn_s = _moe_identity(E, H, [1, 3], fmt)
    X = np.array([[0.5 * (c + 1) * (-1) ** c for c in range(H)],
                  [-3.0 + 0.25 * c for c in range(H)],
                  [0.0] * (H - 1) + [7.0]], np.float32)
    lg = np.tile(np.array([0.0, math.log(3.0)], np.float32), (T, 1))
    plan = orc.moe_plan(lg, T, E, k)
    m = {"E": E, "H": H, "I": H, "T": T, "X": X, "gu_codes": gu_c, "gu_scales": gu_s, "dn_codes": dn_c,
         "dn_scales": dn_s}
    r = orc.moe_ffn(m, plan, fmt=fmt)
    w1 = 1.0 / (1.0 + math.exp(float(np.float32(0.0)) - float(np.float32(math.log(3.0)))))
    for t in range(T):
        for c in range(H):
            x = float(X[t, c])
            a = _silu(x) * 2.0 * x
            want = w1 * 3.0 * a + (1.0 - w1) * a
            assert abs(r["y"][t, c] - want) <= 1e-14 * max(1.0, abs(want)), (t, c)
            swapped = w1 * 3.0 * _silu(2.0 * x) * x + (1.0 - w1) * _silu(2.0 * x) * x
            if x != 0.0 and abs(x) <= 4.0:     # (for large |x| both forms tend to 2 x^2)
                assert abs(r["y"][t, c] - swapped) > 1e-3 * abs(want)
    # the stage values: gate | up = (x, 2x), a, and o of expert 1 (row order: experts ascending)
    src = plan["row_src"]
    assert np.allclose(r["GU"][:, :H], X[src].astype(np.float64), rtol=0, atol=0)
    assert np.allclose(r["GU"][:, H:], 2.0 * X[src].astype(np.float64), rtol=0, atol=0)
    seg = plan["seg_off"]
    assert np.allclose(r["O"][seg[1]:seg[2]], 3.0 * r["A"][seg[1]:seg[2]], rtol=1e-15, atol=0)


def test_moe_chain_bound_one_hot(orc):
    """The bound components for one token, one expert, identity gate and down, doubled identity up
    and x = v e_0: g = v e_0, u = 2 v e_0, a_0 = SiLU(v) 2v; b_dn[0] = |a_0|;
    b_gu[0] = 1.1 |u_0| Sg_0 + |SiLU(g_0)| Su_0 = 1.1 |2v| |v| + |SiLU(v)| |2v| (Sg_0 = |v|,
    Su_0 = |2v|); every other column has zero bounds and zero output."""
    E, H, T, k = 1, 32, 1, 1
    I = H
    gu_c, gu_s = _diag_q4(2 * I, H, [(i, i, 1) for i in range(I)] + [(I + i, i, 2) for i in range(I)])
    dn_c, dn_s = _diag_q4(H, I, [(i, i, 1) for i in range(H)])
    for v in (1.5, -2.25, 0.0):
        X = np.zeros((T, H), np.float32)
        X[0, 0] = v
        plan = orc.moe_plan(np.zeros((T, E), np.float32), T, E, k)
        m = {"E": E, "H": H, "I": I, "T": T, "X": X, "gu_codes": gu_c[None], "gu_scales": gu_s[None],
             "dn_codes": dn_c[None], "dn_scales": dn_s[None]}
        r = orc.moe_ffn(m, plan)
        a0 = _silu(v) * 2.0 * v
        assert r["y"][0, 0] == pytest.approx(a0, rel=1e-15, abs=0)
        assert r["b_dn"][0, 0] == pytest.approx(abs(a0), rel=1e-15, abs=0)
        assert r["b_gu"][0, 0] == pytest.approx(1.1 * abs(2.0 * v) * abs(v) + abs(_silu(v)) * abs(2.0 * v),
                                                rel=1e-15, abs=0)
        assert np.all(r["y"][0, 1:] == 0) and np.all(r["b_dn"][0, 1:] == 0) and np.all(r["b_gu"][0, 1:] == 0)


def test_moe_chain_brute_force(orc):
    """A small random chain (3 experts, H 64, I 32, 5 tokens, top 2, Q4) against plain Python loops
    over weights decoded here from the raw bytes: gate rows first, then up rows, SiLU(g) u, down,
    and the weighted sum in slot order."""
    import synth
    E, H, I, T, k = 3, 64, 32, 5, 2
    m = synth.make_moe(E, H, I, T, 91)
    lg = m["logits"].reshape(T, E)
    plan = orc.moe_plan(lg, T, E, k)
    r = orc.moe_ffn(m, plan)
    X = m["X"].reshape(T, H).astype(np.float64)

    def w_of(codes, scales, K, n, kk):
        b, j = divmod(kk, 32)
        byte = int(codes[n * (K // 2) + 16 * b + (j % 16)])
        nib = byte & 15 if j < 16 else byte >> 4
        return float(np.float32(nib - 8) * np.float32(np.uint16(scales[n * (K // 32) + b]).view(np.float16)))

    for t in range(T):
        for j in range(k):
            e = int(plan["slot_expert"][t * k + j])
            gu = [sum(X[t, h] * w_of(m["gu_codes"][e], m["gu_scales"][e], H, n, h) for h in range(H))
                  for n in range(2 * I)]
            a = [_silu(gu[i]) * gu[I + i] for i in range(I)]
            o = [sum(a[i] * w_of(m["dn_codes"][e], m["dn_scales"][e], I, c, i) for i in range(I)) for c in range(H)]
            row = plan["slot_row"][t * k + j]
            assert np.allclose(r["O"][row], o, rtol=1e-12, atol=1e-12)
    for t in range(T):
        want = sum(plan["slot_w"][t * k + j] * r["O"][plan["slot_row"][t * k + j]] for j in range(k))
        assert np.allclose(r["y"][t], want, rtol=1e-15, atol=0)


# ---- affine GGUF blocks (oxinfer src/metal.rs, GGUF_SHADER_SRC: load_q45, Q4_KW / scale_min_k4) ---
def _golden_affine():
    with open(os.path.join(GOLD, "gguf_affine_blocks.json")) as f:
        return json.load(f)["cases"]


def _expected_row(spec, n):
    out = np.full(n, spec["default"], np.float64)
    for key, v in spec.items():
        if key != "default":
            out[int(key)] = v
    return out


@pytest.mark.parametrize("case", _golden_affine(), ids=lambda c: c["name"])
def test_gguf_affine_hand_blocks(orc, case):
    """Q4_1, Q5_0, Q5_1, Q4_K and Q5_K blocks worked by hand (tests/golden/gguf_affine_blocks.json): every
    element's decoded value, and +0 (not -0) where the value is zero."""
    src = np.frombuffer(bytes.fromhex("".join(case["fields_hex"])), np.uint8)
    K = case["K"]
    w = orc.gguf_dequant(case["type"], src, 1, K)[0].astype(np.float64)
    if "expected" in case:
        exp = _expected_row(case["expected"], K)
    else:
        exp = np.concatenate([_expected_row(s, 32) for s in case["expected_subblocks"]])
    assert np.array_equal(w, exp), f"{case['name']}: first mismatch at {np.argmax(w != exp)}"
    assert not np.any(np.signbit(w) & (w == 0)), "a zero value came out as -0"


@pytest.mark.parametrize("gtype", ["q4_1", "q5_0", "q5_1", "q4_k", "q5_k"])
def test_gguf_affine_repack_matches_direct_decode(orc, gtype):
    """The Q8A repack (int8 code, f32 scale, f32 offset per 32 elements), decoded by the Q8A decoder
    (code * scale, then + offset), gives every element's GGUF value bit for bit -- random blocks with
    negative scales and mins (the Q8A order of operations equals each type's)."""
    rng = np.random.default_rng(17)
    N, K = 3, 512
    import synth
    if gtype in ("q4_k", "q5_k"):
        nsb = N * K // 256
        sbb = 144 if gtype == "q4_k" else 176
        src = rng.integers(0, 256, nsb * sbb).astype(np.uint8).reshape(nsb, sbb)
        d = synth.f16_uniform(11, 1, nsb, -0.05, 0.05)
        dm = synth.f16_uniform(12, 1, nsb, -0.05, 0.05)
        src[:, 0], src[:, 1], src[:, 2], src[:, 3] = d & 0xFF, d >> 8, dm & 0xFF, dm >> 8
    else:
        nb = N * K // 32
        bb = orc.GGUF_BLOCK_BYTES[gtype]
        src = rng.integers(0, 256, nb * bb).astype(np.uint8).reshape(nb, bb)
        d = synth.f16_uniform(11, 1, nb, -0.05, 0.05)
        src[:, 0], src[:, 1] = d & 0xFF, d >> 8
        if gtype in ("q4_1", "q5_1"):
            m = synth.f16_uniform(12, 1, nb, -1.0, 1.0)
            src[:, 2], src[:, 3] = m & 0xFF, m >> 8
    src = src.reshape(-1)
    direct = orc.gguf_dequant(gtype, src, N, K)
    codes, scales, offs = orc.gguf_repack_q8a(gtype, src, N, K)
    split = orc.dequant_tile("q8a", codes, scales, offs, 32, N, K, 0, 0, N, K, "f32")
    assert np.array_equal(direct.view(np.uint32), split.view(np.uint32))
    lo, hi = {"q4_1": (0, 15), "q5_0": (-16, 15), "q5_1": (0, 31), "q4_k": (0, 15), "q5_k": (0, 31)}[gtype]
    assert codes.min() >= lo and codes.max() <= hi


# ---- convolution as an implicit GEMM (oxinfer src/metal.rs, SHADER_SRC conv_body / norm4,
# group_stats / row_stats, Backend::conv2d) --------------------------------------------------------
def _q8_onehot(n_out, K, entries):
    """Q8 weights [n_out][K], scale 1, code q at (o, k) for (o, k, q) in entries, else 0."""
    codes = np.zeros((n_out, K), np.int8)
    for o, k, q in entries:
        codes[o, k] = q
    return codes.reshape(-1), np.ones(n_out * K // 32, np.float32)


def test_conv_1x1_is_the_gemm_over_pixels(orc):
    """A 1 x 1 convolution with stride 1 is the GEMM with the pixels as tokens, bit for bit."""
    import synth
    H, W, cin, n_out = 3, 5, 64, 40
    w = synth.make_dense("q4", n_out, cin, H * W, "f32", 1.0, 61)
    Yc, Sc = orc.conv2d("q4", w["codes"], w["scales"], None, 64, n_out, w["X"], H, W, cin, 1, 1)
    Yg, Sg, _ = orc.gemm("q4", w["codes"], w["scales"], None, 64, n_out, cin, w["X"], "f32", H * W)
    assert np.array_equal(Yc, Yg) and np.array_equal(Sc, Sg)


@pytest.mark.parametrize("stride", [1, 2])
def test_conv_one_hot_taps_and_zero_padding(orc, stride):
    """Output channel o = (ky, kx, c) picks input channel c at tap (ky, kx): y[oy][ox] =
    x[oy*s + ky - 1][ox*s + kx - 1][c], or 0 outside the image (3 x 3 kernel, pad 1).  Pins the
    (ky, kx, ci) order of K, the sign of the tap offset, the padding and the output size."""
    H, W, cin, ksz = 4, 5, 32, 3
    K = ksz * ksz * cin
    taps = [(ky, kx, c) for ky in range(3) for kx in range(3) for c in (0, 7, 31)]
    codes, scales = _q8_onehot(len(taps), K, [(o, (ky * 3 + kx) * cin + c, 1) for o, (ky, kx, c) in enumerate(taps)])
    X = (np.arange(H * W * cin, dtype=np.float32) + 1.0)         # distinct, exact values
    Y, _ = orc.conv2d("q8", codes, scales, None, 64, len(taps), X, H, W, cin, ksz, stride)
    oh, ow = (H - 1) // stride + 1, (W - 1) // stride + 1
    assert orc.conv_out_size(H, W, ksz, stride) == (oh, ow) and Y.shape == (oh * ow, len(taps))
    x = X.reshape(H, W, cin)
    for oy in range(oh):
        for ox in range(ow):
            for o, (ky, kx, c) in enumerate(taps):
                iy, ix = oy * stride + ky - 1, ox * stride + kx - 1
                want = x[iy, ix, c] if 0 <= iy < H and 0 <= ix < W else 0.0
                assert Y[oy * ow + ox, o] == want


def test_conv_even_kernel_geometry(orc):
    """ksz = 2: pad 1, output (H + 1) x (W + 1); tap (ky, kx) of pixel (oy, ox) reads x[oy + ky - 1][ox + kx - 1]."""
    H, W, cin = 3, 2, 32
    K = 4 * cin
    codes, scales = _q8_onehot(4, K, [(o, o * cin + 5, 1) for o in range(4)])
    X = np.arange(H * W * cin, dtype=np.float32) + 1.0
    Y, _ = orc.conv2d("q8", codes, scales, None, 64, 4, X, H, W, cin, 2, 1)
    assert orc.conv_out_size(H, W, 2, 1) == (4, 3)
    x = X.reshape(H, W, cin)
    for oy in range(4):
        for ox in range(3):
            for o in range(4):
                iy, ix = oy + o // 2 - 1, ox + o % 2 - 1
                want = x[iy, ix, 5] if 0 <= iy < H and 0 <= ix < W else 0.0
                assert Y[oy * 3 + ox, o] == want


@pytest.mark.parametrize("stride", [1, 2])
def test_conv_matches_scipy_correlate(orc, stride):
    """Random Q8 weights, 3 x 3 and 5 x 5 kernels: the sum over input channels of scipy's 2-D
    cross-correlation ('same', zero fill) of each channel with the decoded kernel slice, taken at
    every stride-th pixel."""
    from scipy.signal import correlate2d
    import synth
    rng = np.random.default_rng(3 + stride)
    for ksz in (3, 5):
        H, W, cin, n_out = 7, 6, 32, 3
        K = ksz * ksz * cin
        w = synth.make_dense("q8", n_out, K, 1, "f32", 1.0, 70 + ksz)
        X = rng.standard_normal(H * W * cin).astype(np.float32)
        Y, _ = orc.conv2d("q8", w["codes"], w["scales"], None, 64, n_out, X, H, W, cin, ksz, stride)
        Wd = orc.dequant_tile("q8", w["codes"], w["scales"], None, 64, n_out, K, 0, 0, n_out, K, "f32")
        Wd = Wd.astype(np.float64).reshape(n_out, ksz, ksz, cin)
        x = X.reshape(H, W, cin).astype(np.float64)
        oh, ow = orc.conv_out_size(H, W, ksz, stride)
        for o in range(n_out):
            ref = sum(correlate2d(x[:, :, c], Wd[o, :, :, c], mode="same", boundary="fill") for c in range(cin))
            ref = ref[::stride, ::stride]
            assert ref.shape == (oh, ow)
            np.testing.assert_allclose(Y[:, o].reshape(oh, ow), ref, rtol=1e-12, atol=1e-12)


def test_conv_stats_against_numpy(orc):
    """Group statistics over (all pixels, the group's channels) and per-pixel statistics over the
    channels: mean and 1 / sqrt(var + eps) with the population variance, as numpy computes them."""
    rng = np.random.default_rng(9)
    npix, cin, groups, eps = 37, 64, 8, 1e-5
    X = (rng.standard_normal(npix * cin) * 3 + 1).astype(np.float32)
    x = X.reshape(npix, cin).astype(np.float64)
    g = orc.conv_stats(X, npix, cin, groups, eps)
    xg = x.reshape(npix, groups, cin // groups)
    np.testing.assert_allclose(g[:, 0], xg.mean(axis=(0, 2)), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(g[:, 1], 1 / np.sqrt(xg.var(axis=(0, 2)) + eps), rtol=1e-12)
    l = orc.conv_stats(X, npix, cin, 0, eps)
    np.testing.assert_allclose(l[:, 0], x.mean(axis=1), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l[:, 1], 1 / np.sqrt(x.var(axis=1) + eps), rtol=1e-12)
    c = orc.conv_stats(np.full(npix * cin, 2.5, np.float32), npix, cin, 4, 0.25)   # constant image
    assert np.all(c[:, 0] == 2.5) and np.all(c[:, 1] == 2.0)


def test_conv_normalised_gather_closed_forms(orc):
    """The gathered value of a normalised tap: y = (v - mean) rstd gamma + beta, then SiLU; padding
    taps stay 0 (not beta); group norm takes stats[c // cpg], layer norm stats[input pixel]."""
    H, W, cin = 1, 2, 32
    X = np.zeros(H * W * cin, np.float32)
    X[0 * cin + 3] = 2.0          # pixel 0, channel 3
    X[1 * cin + 3] = 5.0          # pixel 1, channel 3
    gb = np.zeros(2 * cin, np.float32)
    gb[3], gb[cin + 3] = 3.0, -1.0                 # gamma 3, beta -1 on channel 3
    # group norm, 4 groups of 8 channels: channel 3 -> group 0 (mean 1, rstd 2)
    st = np.array([[1.0, 2.0], [9.0, 9.0], [9.0, 9.0], [9.0, 9.0]], np.float32)
    A, M = orc.conv_gather(X, H, W, cin, 3, 1, "group", 4, st, gb, False, ps=[0])
    # pixel 0's centre tap (ky = kx = 1) reads pixel 0; tap (1, 2) reads pixel 1; tap (0, 0) is padding
    centre, right, pad = (1 * 3 + 1) * cin + 3, (1 * 3 + 2) * cin + 3, 3
    assert A[0, centre] == (2.0 - 1.0) * 2.0 * 3.0 - 1.0 == 5.0
    assert A[0, right] == (5.0 - 1.0) * 2.0 * 3.0 - 1.0
    assert A[0, pad] == 0.0 and M[0, pad] == 0.0
    assert A[0, centre + 1] == (0.0 - 9.0) * 9.0 * 0.0 + 0.0      # gamma 0, beta 0 on channel 4
    As, _ = orc.conv_gather(X, H, W, cin, 3, 1, "group", 4, st, gb, True, ps=[0])
    assert As[0, centre] == 5.0 / (1.0 + math.exp(-5.0))
    assert As[0, centre + 1] == 0.0                                 # SiLU(0) = 0
    # layer norm: stats per input pixel
    sl = np.array([[1.0, 2.0], [4.0, 0.5]], np.float32)
    Al, Ml = orc.conv_gather(X, H, W, cin, 3, 1, "layer", 0, sl, gb, False, ps=[0])
    assert Al[0, centre] == (2.0 - 1.0) * 2.0 * 3.0 - 1.0
    assert Al[0, right] == (5.0 - 4.0) * 0.5 * 3.0 - 1.0
    assert np.all(Ml >= np.abs(Al))
    A0, M0 = orc.conv_gather(X, H, W, cin, 3, 1)
    assert np.array_equal(M0, np.abs(A0))


# ---- the K-quants with a scale per 16 elements (oxinfer src/metal.rs, GGUF_SHADER_SRC: the loaders
# Q6_KW, Q3_KW, Q2_KW) and the Q8A16 layout they are repacked into ----------------------------------
def _kquant_block(nbytes, sets):
    b = np.zeros(nbytes, np.uint8)
    for i, v in sets.items():
        b[i] = v
    return b


def test_gguf_q6_k_hand_block(orc):
    """Q6_K: ql, qh, 16 signed scales, f16 d at byte 208 (d = 0.5).  Element 0: low nibble of ql[0]
    (10) with bits 0-1 of qh[0] (2) -> q 42, scale 0 (3): (42 - 32) * 1.5 = 15.  Element 71
    (sub-block 2, 16-block 4): high nibble of ql[7] (12), bits 4-5 of qh[7] (3) -> q 60, scale 2:
    28 * 1.0 = 28.  Element 245 (sub-block 7, 16-block 15): high nibble of ql[64 + 32 + 21] (3), bits
    6-7 of qh[32 + 21] (1) -> q 19, scale -5: -13 * -2.5 = 32.5."""
    src = _kquant_block(210, {0: 0x7A, 128: 0x02, 7: 0xC1, 135: 0x30, 117: 0x3F, 181: 0x40,
                              192: 3, 196: 2, 207: 0xFB, 208: 0x00, 209: 0x38})
    w = orc.gguf_dequant("q6_k", src, 1, 256)[0]
    assert (w[0], w[71], w[245]) == (15.0, 28.0, 32.5)
    # an all-zero code byte pattern gives q = 0: (0 - 32) * d * scale
    assert w[1] == -32 * 1.5 and w[16] == 0.0       # element 16 is 16-block 1, scale 0


def test_gguf_q3_k_hand_block(orc):
    """Q3_K: hmask, qs, 12 scale bytes, f16 d at byte 108 (d = 2).  Element 0: bits 0-1 of qs[0]
    (3), hmask[0] bit 0 clear -> code -1; 6-bit scale 0: low (scales[0] & 15) 5, high (bits 0-1 of
    scales[8]) 2 -> 37 - 32 = 5: -1 * 10 = -10.  Element 100 (sub-block 3, 16-block 6): bits 6-7 of
    qs[4] (1), hmask[4] bit 3 set -> code 1; scale: low (scales[6] & 15) 15, high (bits 2-3 of
    scales[10]) 3 -> 63 - 32 = 31: 62.  Element 245 (16-block 15): bits 6-7 of qs[32 + 21] (2),
    hmask[21] bit 7 set -> code 2; scale: low (scales[7] >> 4) 14, high (bits 6-7 of scales[11]) 0
    -> -18: 2 * -36 = -72."""
    src = _kquant_block(110, {32: 0x03, 96: 0x05, 104: 0x02, 36: 0x40, 4: 0x08, 102: 0x0F, 106: 0x0C,
                              85: 0x80, 21: 0x80, 103: 0xE0, 108: 0x00, 109: 0x40})
    w = orc.gguf_dequant("q3_k", src, 1, 256)[0]
    assert (w[0], w[100], w[245]) == (-10.0, 62.0, -72.0)


def test_gguf_q2_k_hand_block(orc):
    """Q2_K: 16 scale bytes, qs, f16 d and dmin at bytes 80, 82 (d = 1, dmin = 0.5).  Element 0:
    bits 0-1 of qs[0] (3), scale byte 0x27: 3 * 7 - 0.5 * 2 = 20.  Element 50 (sub-block 1,
    16-block 3): bits 2-3 of qs[18] (2), scale byte 0x09: 2 * 9 - 0 = 18.  Element 245 (16-block
    15): bits 6-7 of qs[32 + 21] (1), scale byte 0xF3: 1 * 3 - 0.5 * 15 = -4.5."""
    src = _kquant_block(84, {16: 0x03, 0: 0x27, 34: 0x08, 3: 0x09, 69: 0x40, 15: 0xF3,
                             80: 0x00, 81: 0x3C, 82: 0x00, 83: 0x38})
    w = orc.gguf_dequant("q2_k", src, 1, 256)[0]
    assert (w[0], w[50], w[245]) == (20.0, 18.0, -4.5)


def _random_kquant(orc, gtype, N, K, seed):
    rng = np.random.default_rng(seed)
    nsb = N * K // 256
    sbb = orc.GGUF_SUPER_BYTES[gtype]
    src = rng.integers(0, 256, nsb * sbb).astype(np.uint8).reshape(nsb, sbb)
    d = synth.f16_uniform(seed, 1, nsb, -0.05, 0.05)            # negative scales too
    if gtype == "q2_k":
        dm = synth.f16_uniform(seed, 2, nsb, -0.05, 0.05)
        src[:, 80], src[:, 81], src[:, 82], src[:, 83] = d & 0xFF, d >> 8, dm & 0xFF, dm >> 8
    else:
        at = sbb - 2
        src[:, at], src[:, at + 1] = d & 0xFF, d >> 8
    return src.reshape(-1)


@pytest.mark.parametrize("gtype", ["q6_k", "q3_k", "q2_k"])
def test_gguf_q8a16_repack_matches_direct_decode(orc, gtype):
    """The Q8A16 repack, decoded by the split-layout decoder, gives every element's value bit for bit
    (zeros' signs included) -- the in-block loader and the split decoder are independent paths --
    and the codes stay in the type's range."""
    N, K = 3, 768
    src = _random_kquant(orc, gtype, N, K, 21)
    direct = orc.gguf_dequant(gtype, src, N, K)
    codes, scales, offs = orc.gguf_repack_q8a16(gtype, src, N, K)
    split = orc.dequant_tile("q8a16", codes, scales, offs, 32, N, K, 0, 0, N, K, "f32")
    assert np.array_equal(direct.view(np.uint32), split.view(np.uint32))
    assert np.any(direct.view(np.uint32) == 0x80000000) or gtype == "q2_k"
    lo, hi = {"q6_k": (-32, 31), "q3_k": (-4, 3), "q2_k": (0, 3)}[gtype]
    assert codes.min() >= lo and codes.max() <= hi


def test_q8a16_reduces_to_q8a(orc):
    """Q8A16 whose two 16-element halves of every 32-element block share one scale and offset is
    the Q8A matrix with those blocks: the same Y and S, bit for bit."""
    rng = np.random.default_rng(4)
    N, K, T = 7, 96, 3
    codes = rng.integers(-128, 128, N * K).astype(np.int8)
    s32 = rng.uniform(-0.1, 0.1, N * K // 32).astype(np.float32)
    o32 = rng.uniform(-1, 1, N * K // 32).astype(np.float32)
    X = rng.standard_normal(T * K).astype(np.float32)
    Ya, Sa, _ = orc.gemm("q8a", codes, s32, o32, 32, N, K, X, "f32", T)
    Yb, Sb, _ = orc.gemm("q8a16", codes, np.repeat(s32, 2), np.repeat(o32, 2), 32, N, K, X, "f32", T)
    assert np.array_equal(Ya, Yb) and np.array_equal(Sa, Sb)
    # and a scale change in one half moves exactly that half's elements
    s16 = np.repeat(s32, 2)
    s16[1] *= 2
    w = orc.dequant_tile("q8a16", codes, s16, np.repeat(o32, 2), 32, N, K, 0, 0, 1, 32, "f32")[0]
    w0 = orc.dequant_tile("q8a", codes, s32, o32, 32, N, K, 0, 0, 1, 32, "f32")[0]
    assert np.array_equal(w[:16], w0[:16]) and not np.array_equal(w[16:], w0[16:])


@pytest.mark.parametrize("gtype", ["q6_k", "q3_k"])
def test_gguf_q8a16_without_offsets(orc, gtype):
    """Q6_K and Q3_K need no offset: the offset-free Q8A16 layout (float(q) * scale alone) decodes
    every element as the in-block loader does, bit for bit, and its GEMM equals the one with the
    explicit -0 offsets."""
    N, K, T = 3, 512, 2
    src = _random_kquant(orc, gtype, N, K, 23)
    codes, scales, offs = orc.gguf_repack_q8a16(gtype, src, N, K, with_offsets=False)
    assert offs is None
    direct = orc.gguf_dequant(gtype, src, N, K)
    split = orc.dequant_tile("q8a16", codes, scales, None, 32, N, K, 0, 0, N, K, "f32")
    assert np.array_equal(direct.view(np.uint32), split.view(np.uint32))
    X = np.random.default_rng(2).standard_normal(T * K).astype(np.float32)
    c2, s2, o2 = orc.gguf_repack_q8a16(gtype, src, N, K)
    assert np.all(o2.view(np.uint32) == 0x80000000)
    Ya, Sa, _ = orc.gemm("q8a16", codes, scales, None, 32, N, K, X, "f32", T)
    Yb, Sb, _ = orc.gemm("q8a16", c2, s2, o2, 32, N, K, X, "f32", T)
    assert np.array_equal(Ya, Yb) and np.array_equal(Sa, Sb)
