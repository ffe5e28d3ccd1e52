"""The expert-row kernel of short-segment grouped matmuls and the three-launch expert block built on it,
against the oracle: every format and activation path on ragged segments (1..9 rows, an empty expert,
rows outside X), the fused f16 row scaling equal bit for bit to qg_x_half followed by the f16 call, the
fused expert block equal bit for bit to the separate calls, and the block against the oracle's chain
bound for Q4, Q4A and Q8 experts."""
import numpy as np
import pytest
import torch

import block_quantized_weight_affine_amd as qg
import synth
from helpers import TAU, chain_bound, check_tol, dev

pytestmark = pytest.mark.gpu

SIZES = [3, 0, 1, 4, 9, 2, 5, 0, 6, 1]          # segments: empty, 1..9 rows (chunks of 4 and tails)


def _grouped_case(fmt, N, K, x_rows, seed):
    E = len(SIZES)
    seg = np.concatenate([[0], np.cumsum(SIZES)]).astype(np.int32)
    R = int(seg[-1])
    ws = [synth.make_dense(fmt, N, K, 1, "f32", 1.0, seed + 101 * e) for e in range(E)]
    dw = [(dev(w["codes"]), dev(w["scales"]), dev(w["offsets"]) if "offsets" in w else None) for w in ws]
    rng = np.random.default_rng(seed)
    row_src = rng.integers(0, x_rows, R).astype(np.int32)
    return E, seg, R, ws, dw, qg.expert_table(dw), row_src


def _check_experts(orc, fmt, y, seg, ws, N, K, Xo, xt, tau, what):
    worst = 0.0
    for e in range(len(seg) - 1):
        r0, r1 = int(seg[e]), int(seg[e + 1])
        if r0 == r1:
            continue
        w = ws[e]
        Yr, Sr, _ = orc.gemm(fmt, w["codes"], w["scales"], w.get("offsets"), 64, N, K, Xo[r0:r1], xt, r1 - r0)
        worst = max(worst, check_tol(y[r0:r1], Yr, Sr, tau, f"{what}: expert {e} ({r1 - r0} rows)"))
    return worst


@pytest.mark.parametrize("fmt", ["q4", "q4a", "q8"])
@pytest.mark.parametrize("path", ["exact_f32", "exact_f16", "exact_bf16", "fast_f16", "fast_bf16", "fast_f32"])
@pytest.mark.parametrize("kcase", ["k320", "k96", "k1024"])
def test_rows_grouped_matches_oracle(orc, fmt, path, kcase):
    """Short segments (R = 31 <= 8 E): N = 198 (a ragged last batch of weight rows), K = 320 (16-byte
    lane chunks, lanes past K idle), a multiple of 96 (Q4 / Q4A: K 1152, 12-byte lane chunks over two
    blocks, 48 lanes busy; Q8: K 768) or 1024 (exact mode: the f32 matrix-core kernel), rows gathered through row_src with two ids outside X (zero rows)
    and one row scaled by 1e-4.  Exact paths at tau_exact against X as stored; fast f16 / bf16 against
    X as stored, fast f32 (rows scaled to f16 in the kernel) against the f32 rows, both at tau_fast."""
    mode, xt = path.split("_")
    N, x_rows = 198, 23
    K = 320 if kcase == "k320" else 1024 if kcase == "k1024" else 768 if fmt == "q8" else 1152
    E, seg, R, ws, dw, table, row_src = _grouped_case(fmt, N, K, x_rows, 900 + len(path))
    row_src[[2, 17]] = [-1, x_rows]                      # outside X: zero rows
    X = synth.normal_as(61, synth.STREAM_X, x_rows * K, 0.0, 1.0, xt).reshape(x_rows, K)
    if xt == "f32":
        X[row_src[5]] *= 1e-4
    Xd = dev(X)
    if xt == "f16":
        Xd = Xd.view(torch.float16)
    elif xt == "bf16":
        Xd = Xd.view(torch.bfloat16)
    Y = torch.full((R, N), float("nan"), device="cuda")
    print(f"rows grouped {fmt} {path} K={K} R={R}", flush=True)
    qg.qgemm_moe_grouped(fmt, table, 64, dev(seg), dev(row_src), x_rows, Xd, None, Y, N, K, R, E, mode)
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    if xt == "f32":
        Xz = np.concatenate([X, np.zeros((1, K), np.float32)])
    else:
        Xz = np.concatenate([X.view(np.uint16), np.zeros((1, K), np.uint16)])
    Xo = np.ascontiguousarray(Xz[np.where((row_src >= 0) & (row_src < x_rows), row_src, x_rows)])
    worst = _check_experts(orc, fmt, y, seg, ws, N, K, Xo, xt, TAU[mode], f"{fmt} {path}")
    print(f"worst |dY|/S = {worst:.3e}")
    assert np.all(np.isnan(y[seg[-1]:]))  # no rows past the last segment


@pytest.mark.parametrize("fmt", ["q4", "q4a", "q8"])
def test_rows_fast_f32_equals_x_half_then_f16(orc, fmt):
    """Fast mode from f32 rows: the in-kernel row scaling gives what qg_x_half followed by the f16 call
    gives, bit for bit (both take the expert-row kernel at R <= 8 E)."""
    N, K, x_rows = 200, 512 if fmt != "q8" else 256, 19
    E, seg, R, ws, dw, table, row_src = _grouped_case(fmt, N, K, x_rows, 700)
    X = synth.normal_as(62, synth.STREAM_X, x_rows * K, 0.0, 1.0, "f32").reshape(x_rows, K)
    X[3] *= 3e4
    X[7] *= 1e-5
    X[11] = 0.0
    Y1 = torch.full((R, N), float("nan"), device="cuda")
    Y2 = torch.full((R, N), float("nan"), device="cuda")
    print(f"rows fast f32 vs x_half {fmt} R={R}", flush=True)
    qg.qgemm_moe_grouped(fmt, table, 64, dev(seg), dev(row_src), x_rows, dev(X), None, Y1, N, K, R, E, "fast")
    Xh = torch.empty((R, K), dtype=torch.int16, device="cuda")
    rs = torch.empty(R, dtype=torch.float32, device="cuda")
    qg.qg_x_half(dev(X), x_rows, dev(row_src), R, K, Xh, rs)
    qg.qgemm_moe_grouped(fmt, table, 64, dev(seg), None, R, Xh.view(torch.float16), rs, Y2, N, K, R, E, "fast")
    torch.cuda.synchronize()
    a, b = Y1.cpu().numpy(), Y2.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{np.sum(a != b)} outputs differ"
    _check_experts(orc, fmt, a, seg, ws, N, K, np.ascontiguousarray(X[row_src]), "f32", TAU["fast"], fmt)


def test_rows_fast_f32_long_segment(orc):
    """Fast mode from f32 rows with R > 8 E (one expert takes 40 rows, ten passes of 4 rows over its
    weights): still the expert-row kernel, against the oracle at tau_fast."""
    N, K, x_rows = 96, 256, 40
    sizes = [40, 1, 0]
    seg = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    R, E = int(seg[-1]), len(sizes)
    ws = [synth.make_dense("q4", N, K, 1, "f32", 1.0, 500 + e) for e in range(E)]
    dw = [(dev(w["codes"]), dev(w["scales"]), None) for w in ws]      # kept alive: the table points into them
    table = qg.expert_table(dw)
    row_src = np.concatenate([np.arange(40), [7]]).astype(np.int32)
    X = synth.normal_as(63, synth.STREAM_X, x_rows * K, 0.0, 1.0, "f32").reshape(x_rows, K)
    Y = torch.full((R, N), float("nan"), device="cuda")
    print(f"rows fast f32 long segment R={R}", flush=True)
    qg.qgemm_moe_grouped("q4", table, 64, dev(seg), dev(row_src), x_rows, dev(X), None, Y, N, K, R, E, "fast")
    torch.cuda.synchronize()
    _check_experts(orc, "q4", Y.cpu().numpy(), seg, ws, N, K, np.ascontiguousarray(X[row_src]), "f32",
                   TAU["fast"], "long segment")


def _moe_inputs(fmt, E, H, I, T, seed):
    """An expert block of format fmt: Q4 from synth.make_moe; Q4A and Q8 experts drawn per expert with
    the dense generator (gate|up [2I][H], down [H][I])."""
    if fmt == "q4":
        return synth.make_moe(E, H, I, T, seed)
    m = synth.make_moe(E, 32, 32, T, seed)          # logits only (X redrawn below)
    gu = [synth.make_dense(fmt, 2 * I, H, 1, "f32", 1.0, seed + 31 * e) for e in range(E)]
    dn = [synth.make_dense(fmt, H, I, 1, "f32", 1.0, seed + 31 * e + 17) for e in range(E)]
    out = {"E": E, "H": H, "I": I, "T": T, "logits": m["logits"],
           "X": synth.normal_as(seed, synth.STREAM_X, T * H, 0.0, 1.0, "f32"),
           "gu_codes": np.stack([w["codes"] for w in gu]), "gu_scales": np.stack([w["scales"] for w in gu]),
           "dn_codes": np.stack([w["codes"] for w in dn]), "dn_scales": np.stack([w["scales"] for w in dn])}
    if fmt == "q4a":
        out["gu_offsets"] = np.stack([w["offsets"] for w in gu])
        out["dn_offsets"] = np.stack([w["offsets"] for w in dn])
    return out


def _tables(m, fmt):
    E = m["E"]
    keep = []

    def table(which):
        C, S = dev(m[f"{which}_codes"]), dev(m[f"{which}_scales"])
        O = dev(m[f"{which}_offsets"]) if fmt == "q4a" else None
        keep.extend([C, S, O])
        return qg.expert_table([(C[e], S[e], O[e] if O is not None else None) for e in range(E)])

    return table("gu"), table("dn"), keep


def _run_ffn(m, fmt, plan, k, mode):
    E, H, I, T = m["E"], m["H"], m["I"], m["T"]
    tg, td, keep = _tables(m, fmt)
    # the device plan in the library's types (the oracle's weights are f64)
    pd = {key: dev(np.ascontiguousarray(plan[key], dtype=np.float32 if key == "slot_w" else np.int32))
          for key in ("seg_off", "row_src", "slot_row", "slot_w")}
    ws_bytes = qg.qg_moe_ffn_workspace(H, I, T, k, mode)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    Y = torch.zeros((T, H), device="cuda")
    X = dev(np.asarray(m["X"]).reshape(T, H))
    qg.qg_moe_ffn(fmt, tg, td, 64, E, H, I, X, T, k, pd["seg_off"], pd["row_src"], pd["slot_row"], pd["slot_w"],
                  Y, 0, mode, ws, ws_bytes)
    # the same chain as separate calls: grouped gate|up from the f32 rows, SwiGLU to f32, grouped down
    # from the f32 rows of A, combine
    R = int(plan["seg_off"][-1])
    GU = torch.empty((R, 2 * I), device="cuda")
    A = torch.empty((R, I), device="cuda")
    O = torch.empty((R, H), device="cuda")
    Y2 = torch.zeros((T, H), device="cuda")
    qg.qgemm_moe_grouped(fmt, tg, 64, pd["seg_off"], pd["row_src"], T, X, None, GU, 2 * I, H, R, E, mode)
    qg.qg_swiglu(GU, R, I, A, qg.QG_X_F32)
    qg.qgemm_moe_grouped(fmt, td, 64, pd["seg_off"], None, R, A, None, O, H, I, R, E, mode)
    qg.qg_moe_combine(O, R, pd["slot_row"], pd["slot_w"], Y2, H, T, k, 0)
    torch.cuda.synchronize()
    return Y.cpu().numpy(), Y2.cpu().numpy()


@pytest.mark.parametrize("mode", ["exact", "fast"])
@pytest.mark.parametrize("shape", ["small", "workload"])
def test_rows_ffn_equals_separate_calls(orc, mode, shape):
    """The three-launch expert block (SwiGLU in the gate|up epilogue, fast-mode row scaling inside both
    matmuls) equals the separate calls bit for bit: a small block (16 experts, H 256, I 160, 7 tokens,
    top 3) and the 128-expert top-8 workload (H 2048, I 1536, 32 tokens)."""
    if shape == "small":
        E, H, I, T, k, seed = 16, 256, 160, 7, 3, 77
    else:
        c = synth.CONFIGS[4]
        E, H, I, T, k, seed = c.extra["experts"], c.N, c.extra["inter"], c.T, c.extra["top_k"], c.seed
    m = _moe_inputs("q4", E, H, I, T, seed)
    plan = orc.moe_plan(m["logits"].reshape(T, E), T, E, k)
    print(f"rows ffn vs separate {shape} {mode}", flush=True)
    y, y2 = _run_ffn(m, "q4", plan, k, mode)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), f"{np.sum(y != y2)} outputs differ"
    if shape == "small":
        ref = orc.moe_ffn(m, plan)
        check_tol(y, ref["y"], chain_bound(ref, mode), 1.0, f"ffn small {mode}")


@pytest.mark.parametrize("fmt", ["q4", "q4a", "q8"])
@pytest.mark.parametrize("mode", ["exact", "fast"])
def test_rows_ffn_formats_vs_oracle(orc, fmt, mode):
    """The three-launch expert block with Q4, Q4A and Q8 experts (12 experts, H 512, I 192, 9 tokens,
    top 4, one expert unused) against the oracle's chain bound, and equal bit for bit to the separate
    calls."""
    E, H, I, T, k = 12, 512, 192, 9, 4
    m = _moe_inputs(fmt, E, H, I, T, 300 + len(fmt))
    lg = m["logits"].reshape(T, E).copy()
    lg[:, 7] = -1e9
    plan = orc.moe_plan(lg, T, E, k)
    assert plan["seg_off"][8] == plan["seg_off"][7]
    print(f"rows ffn {fmt} {mode}", flush=True)
    y, y2 = _run_ffn(m, fmt, plan, k, mode)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    ref = orc.moe_ffn(m, plan, fmt=fmt)
    check_tol(y, ref["y"], chain_bound(ref, mode), 1.0, f"ffn {fmt} {mode}")
