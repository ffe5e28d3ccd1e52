"""The expert block through qg_moe_ffn_noalloc (intermediates in the library's fixed device scratch,
no workspace argument, nothing allocated) against the workspace entry point qg_moe_ffn: two calls in a
row on one GPU, the 128-expert top-8 block and then a smaller block, each bit-identical to the
workspace call on the same inputs (the same kernels run) and within the chain's bound of the oracle."""
import numpy as np
import pytest
import torch

import block_quantized_weight_affine_amd as qg
import synth
from helpers import chain_bound, check_tol, dev

pytestmark = pytest.mark.gpu


def _table(codes, scales):
    C, S = dev(codes), dev(scales)
    return (C, S), qg.expert_table([(C[e], S[e], None) for e in range(codes.shape[0])])


@pytest.mark.parametrize("mode", ["exact", "fast"])
def test_noalloc_matches_workspace_entry(orc, mode):
    c = synth.CONFIGS[4]
    blocks = [
        (c.extra["experts"], c.N, c.extra["inter"], c.T, c.extra["top_k"], c.seed, 0),   # 128 experts, top 8
        (16, 256, 128, 5, 2, 77, 1),                                                      # smaller, accumulate
    ]
    for E, H, I, T, k, seed, acc in blocks:
        print(f"no-alloc expert block E={E} H={H} I={I} T={T} k={k} {mode} accumulate={acc}", flush=True)
        m = synth.make_moe(E, H, I, T, seed)
        lg = m["logits"].reshape(T, E)
        plan = orc.moe_plan(lg, T, E, k)
        hp = qg.qg_moe_plan_host(lg, T, E, k)
        pd = {key: dev(np.ascontiguousarray(hp[key])) for key in ("seg_off", "row_src", "slot_row", "slot_w")}
        keep_g, tg = _table(m["gu_codes"], m["gu_scales"])
        keep_d, td = _table(m["dn_codes"], m["dn_scales"])
        X = dev(m["X"].reshape(T, H))
        y0 = synth.normal_as(seed, 22, T * H, 0.0, 1.0, "f32").reshape(T, H) if acc else np.zeros((T, H), np.float32)
        ws_bytes = qg.qg_moe_ffn_workspace(H, I, T, k, mode)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        Y_ws = dev(y0.copy())
        qg.qg_moe_ffn("q4", tg, td, 64, E, H, I, X, T, k, pd["seg_off"], pd["row_src"], pd["slot_row"], pd["slot_w"],
                      Y_ws, acc, mode, ws, ws_bytes)
        Y_na = dev(y0.copy())
        qg.qg_moe_ffn_noalloc("q4", tg, td, 64, E, H, I, X, T, k, pd["seg_off"], pd["row_src"], pd["slot_row"],
                              pd["slot_w"], Y_na, acc, mode)
        torch.cuda.synchronize()
        y_ws, y_na = Y_ws.cpu().numpy(), Y_na.cpu().numpy()
        assert np.array_equal(y_na.view(np.uint32), y_ws.view(np.uint32)), \
            f"differs from the workspace entry point at {np.argwhere(y_na != y_ws)[:4].tolist()}"
        ref = orc.moe_ffn(m, plan)
        yr = ref["y"] + y0.astype(np.float64)
        bound = chain_bound(ref, mode) + (np.abs(y0) * 2.0 ** -23 if acc else 0.0)
        check_tol(y_na, yr, bound, 1.0, f"no-alloc block E={E} {mode}")
        del ws
