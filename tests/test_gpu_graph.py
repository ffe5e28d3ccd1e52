"""The library under HIP graph capture (torch.cuda.graph): every entry point called inside the capture
block takes torch's current stream at call time, which there is the capture stream, and the library
makes no allocation, copy, memset or synchronisation call, so the graph holds exactly its kernels.
Each graph is replayed several times, with new inputs written eagerly and a synchronisation between
replays, and every replay is compared bit for bit with the same calls made eagerly."""
import numpy as np
import pytest
import torch

import block_quantized_weight_affine_amd as qg
import synth
from helpers import dev

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _bits(t):
    return t.cpu().numpy().view(np.uint32)


def test_graph_dense_gemv_and_exact_gemm():
    N, K = 4096, 4096
    w8 = synth.make_dense("q8", N, K, 1, "f32", 1.0, 5101)
    c8, s8 = dev(w8["codes"]), dev(w8["scales"])
    Nq, Kq, Tq = 512, 1024, 64
    w4 = synth.make_dense("q4", Nq, Kq, Tq, "f32", 1.0, 5102)
    c4, s4 = dev(w4["codes"]), dev(w4["scales"])
    X8 = dev(w8["X"].reshape(1, K))
    X4 = dev(w4["X"].reshape(Tq, Kq))
    Y8, Y4 = torch.empty((1, N), device="cuda"), torch.empty((Tq, Nq), device="cuda")
    # eager warm-up (the library's per-device look-ups happen here, outside the capture)
    qg.qgemv_q8(c8, s8, X8, Y8, N, K, 1)
    qg.qgemm_q4(c4, s4, X4, Y4, Nq, Kq, Tq, "exact")
    torch.cuda.synchronize()
    print("graph capture: q8 GEMV T1 4096 x 4096, q4 exact 512 x 1024 T64", flush=True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qg.qgemv_q8(c8, s8, X8, Y8, N, K, 1)
        qg.qgemm_q4(c4, s4, X4, Y4, Nq, Kq, Tq, "exact")
    torch.cuda.synchronize()
    R8, R4 = torch.empty_like(Y8), torch.empty_like(Y4)
    for r in range(REPLAYS):
        X8.copy_(dev(synth.normal_as(5200 + r, synth.STREAM_X, K, 0.0, 1.0, "f32").reshape(1, K)))
        X4.copy_(dev(synth.normal_as(5300 + r, synth.STREAM_X, Tq * Kq, 0.0, 1.0, "f32").reshape(Tq, Kq)))
        Y8.fill_(float("nan"))
        Y4.fill_(float("nan"))
        torch.cuda.synchronize()
        print(f"replay {r}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        qg.qgemv_q8(c8, s8, X8, R8, N, K, 1)
        qg.qgemm_q4(c4, s4, X4, R4, Nq, Kq, Tq, "exact")
        torch.cuda.synchronize()
        assert np.array_equal(_bits(Y8), _bits(R8)), f"replay {r}: GEMV differs from the eager call"
        assert np.array_equal(_bits(Y4), _bits(R4)), f"replay {r}: GEMM differs from the eager call"
    del g


@pytest.mark.parametrize("mode", ["exact", "fast"])
def test_graph_moe_block_noalloc(mode):
    """The device routing plan and the no-allocation expert block (128 experts, top 8, T 32) captured
    together; new logits and X before every replay."""
    c = synth.CONFIGS[4]
    E, H, I, T, k = c.extra["experts"], c.N, c.extra["inter"], c.T, c.extra["top_k"]
    m = synth.make_moe(E, H, I, T, c.seed)
    C_g, S_g = dev(m["gu_codes"]), dev(m["gu_scales"])
    C_d, S_d = dev(m["dn_codes"]), dev(m["dn_scales"])
    tg = qg.expert_table([(C_g[e], S_g[e], None) for e in range(E)])
    td = qg.expert_table([(C_d[e], S_d[e], None) for e in range(E)])
    X = dev(m["X"].reshape(T, H))
    L = dev(m["logits"].reshape(T, E))
    seg = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    rsrc = torch.empty(T * k, dtype=torch.int32, device="cuda")
    srow = torch.empty(T * k, dtype=torch.int32, device="cuda")
    sw = torch.empty(T * k, dtype=torch.float32, device="cuda")
    Y = torch.empty((T, H), device="cuda")

    def block(out):
        qg.qg_moe_plan(L, T, E, k, seg, rsrc, srow, sw)
        qg.qg_moe_ffn_noalloc("q4", tg, td, 64, E, H, I, X, T, k, seg, rsrc, srow, sw, out, 0, mode)

    block(Y)
    torch.cuda.synchronize()
    print(f"graph capture: MoE block noalloc {mode}", flush=True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        block(Y)
    torch.cuda.synchronize()
    R = torch.empty_like(Y)
    for r in range(REPLAYS):
        L.copy_(dev(synth.normal_as(5400 + r, 4, T * E, 0.0, 1.0, "f32").reshape(T, E)))
        X.copy_(dev(synth.normal_as(5500 + r, synth.STREAM_X, T * H, 0.0, 1.0, "f32").reshape(T, H)))
        Y.fill_(float("nan"))
        torch.cuda.synchronize()
        print(f"replay {r}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        block(R)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(Y), _bits(R)), f"replay {r}: MoE block differs from the eager call"
    del g
