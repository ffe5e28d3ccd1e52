"""MoE pieces on the GPU against the oracle: the device routing plan, row scaling to f16, the ragged
grouped matmul (exact and fast), SwiGLU, the weighted combine, and the whole expert block end to end
(small design with an unused expert and uneven loads, and the 128-expert top-8 workload, also with the
plan built on the device)."""
import numpy as np
import pytest
import torch

import block_quantized_weight_affine_amd as qg
import synth
from helpers import TAU, chain_bound, check_tol, dev

pytestmark = pytest.mark.gpu


def test_x_half_bit_exact(orc):
    R, K, T = 12, 256, 5
    X = synth.normal_as(3, 3, T * K, 0, 1, "f32").reshape(T, K)
    X *= np.array([1e-6, 1.0, 3.0, 2e5, 0.0])[:, None].astype(np.float32)
    src = np.array([0, 1, 2, 3, 4, 4, 3, 2, 1, 0, 7, -1], np.int32)   # 7 and -1: outside X -> zero rows
    Xh = torch.empty((R, K), dtype=torch.int16, device="cuda")
    rs = torch.empty(R, dtype=torch.float32, device="cuda")
    qg.qg_x_half(dev(X), T, dev(src), R, K, Xh, rs)
    torch.cuda.synchronize()
    Xz = np.concatenate([X, np.zeros((1, K), np.float32)])
    srcz = np.where((src >= 0) & (src < T), src, T)
    xh_ref, rs_ref = orc.x_half(Xz, K, src=srcz)
    got = Xh.cpu().numpy().view(np.uint16)
    bad = np.argwhere(got != xh_ref)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:4].tolist()}: {got[tuple(bad[0])]:#06x} vs {xh_ref[tuple(bad[0])]:#06x}"
    assert np.array_equal(rs.cpu().numpy(), rs_ref)


def _experts(m, which):
    """Device tensors of every expert's gate|up or down weights plus the device table."""
    if which == "gu":
        codes, scales = m["gu_codes"], m["gu_scales"]
    else:
        codes, scales = m["dn_codes"], m["dn_scales"]
    C = dev(codes)
    S = dev(scales)
    table = qg.expert_table([(C[e], S[e], None) for e in range(codes.shape[0])])
    return C, S, table


def _plan_dev(plan):
    return {k: dev(np.ascontiguousarray(v)) for k, v in plan.items() if isinstance(v, np.ndarray)}


@pytest.mark.parametrize("mode", ["exact", "fast", "fast_gather", "fast_long_segment", "exact_long_segment"])
def test_grouped_matches_oracle(orc, mode):
    """Grouped gate|up on seeded rows: every expert's segment against the oracle (rows gathered through
    row_src in exact mode; pre-scaled f16 rows in fast mode; f16 rows gathered through row_src in
    fast_gather; one expert taking every token, so its segment spans several row tiles, in
    fast_long_segment; the same in exact mode, where R = 150 > 8 E sends the call to the f32 MFMA
    tile kernel instead of the GEMV)."""
    E, H, I, T, k = 8, 256, 96, 75, 2
    m = synth.make_moe(E, H, I, T, 21)
    lg = m["logits"].reshape(T, E).copy()
    lg[:, 5] = -1e9                      # expert 5 unused
    if mode.endswith("long_segment"):
        lg[:, 2] += 1e6                  # expert 2 in every token's top k
    plan = orc.moe_plan(lg, T, E, k)
    R = plan["R"]
    C, S, table = _experts(m, "gu")
    pd = _plan_dev({"seg_off": plan["seg_off"], "row_src": plan["row_src"]})
    X = m["X"].reshape(T, H)
    Y = torch.full((R, 2 * I), float("nan"), device="cuda")
    if mode.startswith("exact"):
        qg.qgemm_moe_grouped("q4", table, 64, pd["seg_off"], pd["row_src"], T, dev(X), None, Y, 2 * I, H, R, E,
                             "exact")
        Xo, xt = X[plan["row_src"]], "f32"
    elif mode == "fast_gather":
        X16 = X.astype(np.float16)
        qg.qgemm_moe_grouped("q4", table, 64, pd["seg_off"], pd["row_src"], T, dev(X16), None, Y, 2 * I, H, R, E,
                             "fast")
        Xo, xt = np.ascontiguousarray(X16[plan["row_src"]]).view(np.uint16), "f16"
    else:
        Xh = torch.empty((R, H), dtype=torch.int16, device="cuda")
        rs = torch.empty(R, dtype=torch.float32, device="cuda")
        qg.qg_x_half(dev(X), T, pd["row_src"], R, H, Xh, rs)
        qg.qgemm_moe_grouped("q4", table, 64, pd["seg_off"], None, R, Xh.view(torch.float16), rs, Y, 2 * I, H, R, E,
                             "fast")
        Xo, xt = X[plan["row_src"]], "f32"
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    seg = plan["seg_off"]
    for e in range(E):
        r0, r1 = seg[e], seg[e + 1]
        if r0 == r1:
            continue
        Yr, Sr, _ = orc.gemm("q4", m["gu_codes"][e], m["gu_scales"][e], None, 64, 2 * I, H, Xo[r0:r1], xt, r1 - r0)
        check_tol(y[r0:r1], Yr, Sr, TAU["exact" if mode.startswith("exact") else "fast"], f"expert {e}")
    assert seg[6] - seg[5] == 0
    if mode.endswith("long_segment"):
        assert seg[3] - seg[2] == T


@pytest.mark.parametrize("at", ["f32", "f16"])
def test_swiglu(orc, at):
    R, I = 9, 200
    GU = synth.normal_as(8, 3, R * 2 * I, 0, 2, "f32").reshape(R, 2 * I)
    GU[3] *= 1e4
    GU[4] = 0
    A = torch.empty((R, I), dtype=torch.float32 if at == "f32" else torch.int16, device="cuda")
    rs = torch.empty(R, device="cuda")
    qg.qg_swiglu(dev(GU), R, I, A, qg.QG_X_F32 if at == "f32" else qg.QG_X_F16, rs if at == "f16" else None)
    torch.cuda.synchronize()
    ref = orc.swiglu(GU[:, :I].astype(np.float64), GU[:, I:].astype(np.float64))
    if at == "f32":
        a = A.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(a - ref) <= 4e-6 * np.abs(ref) + 1e-30)
    else:
        a = A.cpu().numpy().view(np.uint16).view(np.float16).astype(np.float64)
        r = rs.cpu().numpy().astype(np.float64)
        amax = np.abs(a).max(axis=1)
        nz = np.abs(ref).max(axis=1) > 0
        assert np.all(amax[nz] >= 2.0**13) and np.all(amax[nz] < 2.0**14)
        assert np.all(r[~nz] == 1.0)
        assert np.all(np.log2(r) == np.round(np.log2(r)))
        back = a * r[:, None]
        assert np.all(np.abs(back - ref) <= 2.0**-11 * np.abs(ref) + 4e-6 * np.abs(ref) + 1e-30)


def test_combine(orc):
    T, k, H, R = 6, 3, 64, 18
    O = synth.normal_as(9, 3, R * H, 0, 1, "f32").reshape(R, H)
    rng = np.random.default_rng(0)
    slot_row = rng.permutation(R).astype(np.int32)
    slot_w = rng.uniform(0, 1, T * k).astype(np.float32)
    y0 = synth.normal_as(9, 4, T * H, 0, 1, "f32").reshape(T, H)
    for acc in (0, 1):
        Y = dev(y0.copy())
        qg.qg_moe_combine(dev(O), R, dev(slot_row), dev(slot_w), Y, H, T, k, acc)
        torch.cuda.synchronize()
        yr, b = orc.moe_combine(O.astype(np.float64), H, slot_row, slot_w.astype(np.float64), T, k)
        if acc:
            yr = yr + y0
            b = b + np.abs(y0)
        check_tol(Y.cpu().numpy(), yr, b, 1e-6, f"combine acc={acc}")


def _ffn(orc, E, H, I, T, k, seed, mode, unused=None, sample=None):
    m = synth.make_moe(E, H, I, T, seed)
    lg = m["logits"].reshape(T, E).copy()
    if unused is not None:
        lg[:, unused] = -1e9
    plan = orc.moe_plan(lg, T, E, k)
    hp = qg.qg_moe_plan_host(lg, T, E, k)
    for key in ("seg_off", "row_src", "slot_row"):
        assert np.array_equal(hp[key], plan[key])
    Cg, Sg, tg = _experts(m, "gu")
    Cd, Sd, td = _experts(m, "dn")
    pd = _plan_dev({k2: hp[k2] for k2 in ("seg_off", "row_src", "slot_row", "slot_w")})
    ws_bytes = qg.qg_moe_ffn_workspace(H, I, T, k, mode)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    Y = torch.zeros((T, H), device="cuda")
    qg.qg_moe_ffn("q4", tg, td, 64, E, H, I, dev(m["X"].reshape(T, H)), T, k, pd["seg_off"], pd["row_src"],
                  pd["slot_row"], pd["slot_w"], Y, 0, mode, ws, ws_bytes)
    torch.cuda.synchronize()
    ref = orc.moe_ffn(m, plan)
    return Y.cpu().numpy(), ref


@pytest.mark.parametrize("mode", ["exact", "fast"])
def test_ffn_small_design(orc, mode):
    """8 experts, h = 128, mi = 64, t = 75, two routes per token, one expert unused (the MoE test design
    of oxinfer src/metal.rs, tests: mma_moe_matches_cpu), end to end against the oracle's bound."""
    y, ref = _ffn(orc, 8, 128, 64, 75, 2, 7, mode, unused=5)
    check_tol(y, ref["y"], chain_bound(ref, mode), 1.0, f"ffn small {mode}")


@pytest.mark.parametrize("mode", ["exact", "fast"])
def test_ffn_full_workload(orc, mode):
    """128 experts, H 2048, I 1536, 32 tokens, top-8: the whole chain against the oracle."""
    c = synth.CONFIGS[4]
    print(f"moe workload {c.name} {mode}", flush=True)
    y, ref = _ffn(orc, c.extra["experts"], c.N, c.extra["inter"], c.T, c.extra["top_k"], c.seed, mode)
    check_tol(y, ref["y"], chain_bound(ref, mode), 1.0, f"ffn full {mode}")


# ---- routing plan on the device ------------------------------------------------------------------
PLAN_CASES = [
    (32, 128, 8, 1004, None),       # the MoE workload's routing shape
    (75, 8, 2, 7, "unused"),        # an expert nobody picks
    (5, 16, 16, 3, "ties"),         # k = E; an all-tied row; a tie at the top
    (1, 1, 1, 11, None),            # one token, one expert
    (300, 100, 6, 12, None),        # E not a multiple of 64; several tokens per wavefront
    (2048, 64, 4, 13, "neg_inf"),   # T*k = 8192: many 64-slot scan chunks; -inf logits tie by index
    (64, 1024, 32, 14, None),       # E and k at their maxima
]


def _device_plan(lg, T, E, k, status_init=-7):
    out = {
        "seg_off": torch.full((E + 1,), -5, dtype=torch.int32, device="cuda"),
        "row_src": torch.full((T * k,), -5, dtype=torch.int32, device="cuda"),
        "slot_row": torch.full((T * k,), -5, dtype=torch.int32, device="cuda"),
        "slot_w": torch.full((T * k,), -5.0, dtype=torch.float32, device="cuda"),
        "slot_expert": torch.full((T * k,), -5, dtype=torch.int32, device="cuda"),
        "status": torch.full((1,), status_init, dtype=torch.int32, device="cuda"),
    }
    print(f"device plan T={T} E={E} k={k}", flush=True)
    qg.qg_moe_plan(dev(np.ascontiguousarray(lg, np.float32)), T, E, k, out["seg_off"], out["row_src"],
                   out["slot_row"], out["slot_w"], out["slot_expert"], out["status"])
    torch.cuda.synchronize()
    return {key: v.cpu().numpy() for key, v in out.items()}


@pytest.mark.parametrize("case", PLAN_CASES, ids=lambda c: f"T{c[0]}-E{c[1]}-k{c[2]}-{c[4]}")
def test_device_plan_matches_oracle(orc, case):
    """Every index output equal to the oracle's plan (full sort per token, ties to the lower index);
    weights within one f32 unit in the last place of the oracle's f64 weights."""
    T, E, k, seed, kind = case
    lg = synth.normal_as(seed, synth.STREAM_LOGITS, T * E, 0.0, 1.0, "f32").reshape(T, E).copy()
    if kind == "unused":
        lg[:, 5] = -1e9
    elif kind == "ties":
        lg[1, :] = 0.25
        lg[2, 3] = lg[2, 9] = 5.0
    elif kind == "neg_inf":
        lg[:, ::3] = -np.inf
        lg[7, :] = -np.inf
        lg[7, 10] = lg[7, 20] = lg[7, 30] = lg[7, 40] = 0.0    # exactly k finite logits, rest tied at -inf
    ref = orc.moe_plan(lg, T, E, k)
    got = _device_plan(lg, T, E, k)
    assert got["status"][0] == 0
    for key in ("seg_off", "row_src", "slot_row", "slot_expert"):
        assert np.array_equal(got[key], ref[key]), key
    w = got["slot_w"].astype(np.float64)
    assert np.all(np.abs(w - ref["slot_w"]) <= 2.0 ** -23 * np.abs(ref["slot_w"])), "weights"
    host = qg.qg_moe_plan_host(lg, T, E, k)
    for key in ("seg_off", "row_src", "slot_row", "slot_expert"):
        assert np.array_equal(got[key], host[key]), key


def test_device_plan_nan_logit_sets_status(orc):
    """A NaN logit: status QG_EPLAN, and the plan is still well formed (every index in range, each
    gathered row used once)."""
    T, E, k = 6, 40, 3
    lg = synth.normal_as(15, synth.STREAM_LOGITS, T * E, 0.0, 1.0, "f32").reshape(T, E).copy()
    lg[2, 7] = np.nan
    got = _device_plan(lg, T, E, k, status_init=0)
    assert got["status"][0] == qg.QG_EPLAN
    seg = got["seg_off"]
    assert seg[0] == 0 and seg[-1] == T * k and np.all(np.diff(seg) >= 0)
    assert np.array_equal(np.sort(got["slot_row"]), np.arange(T * k))
    assert np.all((got["row_src"] >= 0) & (got["row_src"] < T))
    assert np.all((got["slot_expert"] >= 0) & (got["slot_expert"] < E))
    # rows outside the NaN token are the oracle's
    ok = np.ones(T, bool)
    ok[2] = False
    ref = orc.moe_plan(np.where(np.isnan(lg), -np.inf, lg), T, E, k)
    se = got["slot_expert"].reshape(T, k)
    assert np.array_equal(se[ok], ref["slot_expert"].reshape(T, k)[ok])


@pytest.mark.parametrize("mode", ["exact", "fast"])
def test_ffn_full_workload_device_plan(orc, mode):
    """The 128-expert top-8 block with its plan built on the device: the same plan as the host's, and
    the chain's output within the oracle's bound."""
    c = synth.CONFIGS[4]
    E, H, I, T, k = c.extra["experts"], c.N, c.extra["inter"], c.T, c.extra["top_k"]
    m = synth.make_moe(E, H, I, T, c.seed)
    lg = m["logits"].reshape(T, E)
    plan = orc.moe_plan(lg, T, E, k)
    seg_off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    row_src = torch.empty(T * k, dtype=torch.int32, device="cuda")
    slot_row = torch.empty(T * k, dtype=torch.int32, device="cuda")
    slot_w = torch.empty(T * k, dtype=torch.float32, device="cuda")
    Cg, Sg, tg = _experts(m, "gu")
    Cd, Sd, td = _experts(m, "dn")
    ws_bytes = qg.qg_moe_ffn_workspace(H, I, T, k, mode)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    Y = torch.zeros((T, H), device="cuda")
    print(f"moe workload {c.name} {mode} with the device plan", flush=True)
    qg.qg_moe_plan(dev(np.ascontiguousarray(lg)), T, E, k, seg_off, row_src, slot_row, slot_w)
    qg.qg_moe_ffn("q4", tg, td, 64, E, H, I, dev(m["X"].reshape(T, H)), T, k, seg_off, row_src, slot_row, slot_w,
                  Y, 0, mode, ws, ws_bytes)
    torch.cuda.synchronize()
    for key, t in (("seg_off", seg_off), ("row_src", row_src), ("slot_row", slot_row)):
        assert np.array_equal(t.cpu().numpy(), plan[key]), key
    ref = orc.moe_ffn(m, plan)
    check_tol(Y.cpu().numpy(), ref["y"], chain_bound(ref, mode), 1.0, f"ffn full {mode}, device plan")


# ---- grouped exact GEMV: chunk walking, K chunks, gathered and zero rows --------------------------
@pytest.mark.parametrize("fmt", ["q4", "q4a", "q8"])
@pytest.mark.parametrize("xt", ["f32", "f16"])
@pytest.mark.parametrize("K", [3104, 8192, 8224])
def test_grouped_gemv_exact_chunks(orc, fmt, xt, K):
    """Short segments (R <= 8 E, so the grouped GEMV runs): 12 experts with 0..9 rows each (segments
    longer than 4 rows take several row chunks of 1..4 rows), N = 96 (a partial last batch of weight
    rows), X rows gathered through row_src with some ids outside X (zero rows).  K = 3104 (a ragged
    last wavefront of the K split) and 8192 (its longest K, 8 wavefronts) run the K-split kernel;
    8224 the chunked LDS kernel (2048-value K chunks, f32 X staged straight into LDS)."""
    E, N, x_rows, group = 12, 96, 20, 32
    sizes = [0, 1, 2, 3, 4, 5, 9, 0, 1, 6, 2, 3]
    seg = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    R = int(seg[-1])
    assert R <= 8 * E
    rng = np.random.default_rng(31)
    row_src = rng.integers(0, x_rows, R).astype(np.int32)
    row_src[[3, 11, 17]] = [-1, x_rows, x_rows + 5]       # outside X: zero rows
    ws = [synth.make_dense(fmt, N, K, 1, "f32", 1.0, 4000 + e, group=group) for e in range(E)]
    X = synth.normal_as(77, synth.STREAM_X, x_rows * K, 0.0, 1.0, xt).reshape(x_rows, K)
    dw = [(dev(w["codes"]), dev(w["scales"]), dev(w["offsets"]) if "offsets" in w else None) for w in ws]
    table = qg.expert_table(dw)
    Y = torch.full((R, N), float("nan"), device="cuda")
    Xd = dev(X).view(torch.float16) if xt == "f16" else dev(X)
    print(f"grouped exact GEMV {fmt} {xt} R={R} K={K}", flush=True)
    qg.qgemm_moe_grouped(fmt, table, group, dev(seg), dev(row_src), x_rows, Xd, None, Y, N, K, R, E, "exact")
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    Xz = np.concatenate([X, np.zeros((1, K), X.dtype)])
    src = np.where((row_src >= 0) & (row_src < x_rows), row_src, x_rows)
    Xg = np.ascontiguousarray(Xz[src])
    for e in range(E):
        r0, r1 = seg[e], seg[e + 1]
        if r0 == r1:
            continue
        w = ws[e]
        Yr, Sr, _ = orc.gemm(fmt, w["codes"], w["scales"], w.get("offsets"), group, N, K, Xg[r0:r1], xt, r1 - r0)
        check_tol(y[r0:r1], Yr, Sr, TAU["exact"], f"expert {e} ({r1 - r0} rows)")
    for r in (3, 11, 17):
        assert np.all(y[r] == 0.0), f"zero row {r}"


@pytest.mark.parametrize("xt", ["f32", "f16"])
def test_grouped_gemv_exact_no_x_rows(xt):
    """x_rows = 0 with every row_src id outside X: such a call goes to the range-checked chunked
    kernel (the K-split kernel would load X row 0 for a zero row), and every output row is zero."""
    E, N, K, group = 3, 40, 3104, 32
    seg = np.array([0, 2, 2, 5], np.int32)
    R = int(seg[-1])
    row_src = np.array([-1, 0, 3, -7, 1], np.int32)
    ws = [synth.make_dense("q4", N, K, 1, "f32", 1.0, 4100 + e, group=group) for e in range(E)]
    dw = [(dev(w["codes"]), dev(w["scales"]), None) for w in ws]
    table = qg.expert_table(dw)
    Xd = torch.zeros(4, dtype=torch.float32, device="cuda")
    if xt == "f16":
        Xd = Xd.view(torch.float16)
    Y = torch.full((R, N), float("nan"), device="cuda")
    print(f"grouped exact GEMV, no X rows, {xt}", flush=True)
    qg.qgemm_moe_grouped("q4", table, group, dev(seg), dev(row_src), 0, Xd, None, Y, N, K, R, E, "exact")
    torch.cuda.synchronize()
    assert np.all(Y.cpu().numpy() == 0.0)


# ---- every stage of the 128-expert block on its own, per element at tau -------------------------
# Each stage is fed seeded inputs of the shapes and layouts the chain hands it (nothing computed by
# the GPU feeds the oracle): gate|up from the seeded X through the seeded plan, down from a seeded
# activation A, the combine from seeded expert outputs O.  The launches are the ones qg_moe_ffn
# makes for the mode.
def _c4_setup(orc):
    c = synth.CONFIGS[4]
    E, H, I, T, k = c.extra["experts"], c.N, c.extra["inter"], c.T, c.extra["top_k"]
    m = synth.make_moe(E, H, I, T, c.seed)
    plan = orc.moe_plan(m["logits"].reshape(T, E), T, E, k)
    return c, m, plan, (E, H, I, T, k)


def _per_expert(orc, y, plan, codes, scales, N, K, Xo, xt, tau, what):
    seg = plan["seg_off"]
    used = 0
    for e in range(len(seg) - 1):
        r0, r1 = int(seg[e]), int(seg[e + 1])
        if r0 == r1:
            continue
        used += 1
        Yr, Sr, _ = orc.gemm("q4", codes[e], scales[e], None, 64, N, K, Xo[r0:r1], xt, r1 - r0)
        check_tol(y[r0:r1], Yr, Sr, tau, f"{what}: expert {e} ({r1 - r0} rows)")
    return used


@pytest.mark.parametrize("mode", ["exact", "fast"])
def test_moe_workload_gate_up_stage(orc, mode):
    """Grouped gate|up (128 experts, [3072 x 2048] each, 32 tokens, top 8): exact from the f32 rows
    gathered through row_src; fast from qg_x_half's row-scaled f16 rows with the inverse scale in the
    epilogue.  Every expert's segment against the oracle at tau * S (X as the f32 rows)."""
    c, m, plan, (E, H, I, T, k) = _c4_setup(orc)
    R = plan["R"]
    _, _, table = _experts(m, "gu")
    pd = _plan_dev({"seg_off": plan["seg_off"], "row_src": plan["row_src"]})
    X = m["X"].reshape(T, H)
    Y = torch.full((R, 2 * I), float("nan"), device="cuda")
    print(f"moe workload gate|up stage {mode}", flush=True)
    if mode == "exact":
        qg.qgemm_moe_grouped("q4", table, 64, pd["seg_off"], pd["row_src"], T, dev(X), None, Y, 2 * I, H, R, E,
                             "exact")
    else:
        Xh = torch.empty((R, H), dtype=torch.int16, device="cuda")
        rs = torch.empty(R, dtype=torch.float32, device="cuda")
        qg.qg_x_half(dev(X), T, pd["row_src"], R, H, Xh, rs)
        qg.qgemm_moe_grouped("q4", table, 64, pd["seg_off"], None, R, Xh.view(torch.float16), rs, Y, 2 * I, H, R, E,
                             "fast")
    torch.cuda.synchronize()
    used = _per_expert(orc, Y.cpu().numpy(), plan, m["gu_codes"], m["gu_scales"], 2 * I, H,
                       np.ascontiguousarray(X[plan["row_src"]]), "f32", TAU[mode], f"gate|up {mode}")
    assert used > 100


@pytest.mark.parametrize("mode", ["exact", "fast"])
def test_moe_workload_down_stage(orc, mode):
    """Grouped down projection (128 experts, [2048 x 1536] each) over the seeded plan's 256 rows, no
    gather (row r reads A row r), as the chain runs it: exact from f32 A, fast from f16 A with a
    power-of-two inverse row scale rs (what qg_swiglu hands over).  The oracle takes A as the values
    the kernel is given: the f32 rows, or the f16 values times rs (exact in f64)."""
    c, m, plan, (E, H, I, T, k) = _c4_setup(orc)
    R = plan["R"]
    _, _, table = _experts(m, "dn")
    pd = _plan_dev({"seg_off": plan["seg_off"]})
    O = torch.full((R, H), float("nan"), device="cuda")
    print(f"moe workload down stage {mode}", flush=True)
    if mode == "exact":
        A = synth.normal_as(c.seed, 20, R * I, 0.0, 1.0, "f32").reshape(R, I)
        qg.qgemm_moe_grouped("q4", table, 64, pd["seg_off"], None, R, dev(A), None, O, H, I, R, E, "exact")
        Ao, xt = A, "f32"
    else:
        A16 = synth.normal_as(c.seed, 20, R * I, 0.0, 4096.0, "f16").reshape(R, I)
        rs = np.exp2(np.arange(R) % 9 - 16.0).astype(np.float32)     # 2^-16 .. 2^-8
        qg.qgemm_moe_grouped("q4", table, 64, pd["seg_off"], None, R, dev(A16), dev(rs), O, H, I, R, E, "fast")
        Ao = orc.f16_values(A16.view(np.uint16)) * rs.astype(np.float64)[:, None]
        xt = "f64"
    torch.cuda.synchronize()
    used = _per_expert(orc, O.cpu().numpy(), plan, m["dn_codes"], m["dn_scales"], H, I, np.ascontiguousarray(Ao), xt,
                       TAU[mode], f"down {mode}")
    assert used > 100


def test_moe_workload_combine_stage(orc):
    """The weighted combine at the block's shape (32 tokens x top 8 over 256 routed rows of 2048):
    seeded O through the seeded plan's slots, within 1e-6 of sum_j |w_j o_j| (an f32 sum of 8
    products)."""
    c, m, plan, (E, H, I, T, k) = _c4_setup(orc)
    R = plan["R"]
    O = synth.normal_as(c.seed, 21, R * H, 0.0, 1.0, "f32").reshape(R, H)
    sw = plan["slot_w"].astype(np.float32)
    Y = torch.full((T, H), float("nan"), device="cuda")
    qg.qg_moe_combine(dev(O), R, dev(plan["slot_row"].astype(np.int32)), dev(sw), Y, H, T, k, 0)
    torch.cuda.synchronize()
    yr, b = orc.moe_combine(O.astype(np.float64), H, plan["slot_row"], sw.astype(np.float64), T, k)
    check_tol(Y.cpu().numpy(), yr, b, 1e-6, "combine, block shape")


@pytest.mark.parametrize("fmt", ["q4a", "q8"])
@pytest.mark.parametrize("path", ["x_half", "gather_f16", "gather_bf16"])
def test_grouped_fast_formats(orc, fmt, path):
    """Fast grouped matmul with affine Q4 and Q8 experts: 9 experts with 0..40 rows (an empty expert,
    segments over several 32-row tiles), N = 200 (a ragged weight-row tile), K = 320.  x_half: f32
    rows gathered and row-scaled to f16 by qg_x_half (the chain's path); gather_*: 16-bit rows
    gathered through row_src (ids outside X read as zero rows)."""
    E, N, K, x_rows, group = 9, 200, 320, 30, 64
    sizes = [3, 0, 40, 1, 7, 33, 2, 12, 5]
    seg = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    R = int(seg[-1])
    rng = np.random.default_rng(41)
    row_src = rng.integers(0, x_rows, R).astype(np.int32)
    ws = [synth.make_dense(fmt, N, K, 1, "f32", 1.0, 4200 + e, group=group) for e in range(E)]
    dw = [(dev(w["codes"]), dev(w["scales"]), dev(w["offsets"]) if "offsets" in w else None) for w in ws]
    table = qg.expert_table(dw)
    Y = torch.full((R, N), float("nan"), device="cuda")
    print(f"grouped fast {fmt} {path} R={R}", flush=True)
    if path == "x_half":
        X = synth.normal_as(43, synth.STREAM_X, x_rows * K, 0.0, 1.0, "f32").reshape(x_rows, K)
        X[4] *= 1e-4
        Xh = torch.empty((R, K), dtype=torch.int16, device="cuda")
        rs = torch.empty(R, dtype=torch.float32, device="cuda")
        qg.qg_x_half(dev(X), x_rows, dev(row_src), R, K, Xh, rs)
        qg.qgemm_moe_grouped(fmt, table, group, dev(seg), None, R, Xh.view(torch.float16), rs, Y, N, K, R, E, "fast")
        Xo, xt = np.ascontiguousarray(X[row_src]), "f32"
        zero_rows = []
    else:
        xt = "f16" if path == "gather_f16" else "bf16"
        row_src[[5, 20]] = [-3, x_rows]                       # zero rows
        X = synth.normal_as(44, synth.STREAM_X, x_rows * K, 0.0, 1.0, xt).reshape(x_rows, K)
        Xd = dev(X)
        Xd = Xd.view(torch.float16) if xt == "f16" else Xd.view(torch.bfloat16)
        qg.qgemm_moe_grouped(fmt, table, group, dev(seg), dev(row_src), x_rows, Xd, None, Y, N, K, R, E, "fast")
        Xb = X.view(np.uint16)
        Xz = np.concatenate([Xb, np.zeros((1, K), np.uint16)])
        Xo = np.ascontiguousarray(Xz[np.where((row_src >= 0) & (row_src < x_rows), row_src, x_rows)])
        zero_rows = [5, 20]
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    for e in range(E):
        r0, r1 = seg[e], seg[e + 1]
        if r0 == r1:
            continue
        w = ws[e]
        Yr, Sr, _ = orc.gemm(fmt, w["codes"], w["scales"], w.get("offsets"), group, N, K, Xo[r0:r1], xt, r1 - r0)
        check_tol(y[r0:r1], Yr, Sr, TAU["fast"], f"expert {e} ({r1 - r0} rows)")
    for r in zero_rows:
        assert np.all(y[r] == 0.0), f"zero row {r}"
