"""Benchmark of the block-quantized weight matmul on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-also] [--no-cpu]

Prints ONE JSON line.  The headline workload (`value`) is the T = 1 Q8 GEMV decode (N = K = 4096,
int8 weights with f32 block scales, f32 activations), reported in HBM GB/s of algorithmic bytes
(codes + scales + X + Y) per step; each step reads the next of 16 weight copies (302 MB > the 256 MB
Infinity Cache) so the bytes come from HBM.  The timed region holds exactly K steps bracketed by
torch.cuda.synchronize(); HIP events on the launch stream time it.  Each step is one pre-bound call
of the C entry point (arguments marshalled beforehand), so the host side keeps ahead of the GPU.
`roofline` relates the dominant kernel's achieved rate to the chip's peak; `cpu_baseline` times the
CPU oracle on the host cores.
`also` lists the prefill GEMMs (TFLOP/s vs the MFMA peak; the Q8 prefill shape in both fast modes,
weights rounded to f16 and kept exact), the MoE expert block (GB/s), the GGUF
Q4_0 repack of a 4096 x 4096 matrix (GB/s), a 3 x 3 convolution with group norm and SiLU (TFLOP/s), a batched q / k / v decode step (GB/s, with the time
of the same three matrices as separate calls) and the Q8 GEMV with T = 4 (GB/s), each on
its own synthetic workload; `--workload` selects one of them as the headline instead.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"hbm": 8000.0, "f32": 157.3, "f16": 2500.0, "bf16": 2500.0}   # GB/s, TFLOP/s (dense)

WORKLOADS = {
    # name: (config index, mode)
    "q8_gemv_decode": (1, "exact"),
    "q4_tiny_exact": (0, "exact"),
    "q4_prefill_exact": (2, "exact"),
    "q4_prefill_fast": (2, "fast"),
    "q4a_upproj_fast": (3, "fast"),
    "moe_block_exact": (4, "exact"),
    "moe_block_fast": (4, "fast"),
}
HEADLINE = "q8_gemv_decode"
# The sources each workload's kernels are built from: the kernel files, the device and launch headers,
# and the C entry point that picks and launches them.  A committed traffic figure counts only while
# these are unchanged.
_BASE_SOURCES = ["qg_device.hpp", "qg_internal.hpp", "qg_capi.cpp"]
KERNEL_SOURCES = {
    "q8_gemv_decode": _BASE_SOURCES + ["qg_gemv.hip"],
    "moe_block_exact": _BASE_SOURCES + ["qg_moe.hip", "qg_misc.hip"],
    "moe_block_fast": _BASE_SOURCES + ["qg_moe.hip", "qg_misc.hip"],
}


def kernel_source_hash(name: str = HEADLINE) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(name, _BASE_SOURCES + ["qg_gemm.hip", "qg_gemv.hip"]):
        with open(os.path.join(ROOT, "block_quantized_weight_affine_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _dev(a):
    import torch
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()


def _timed(fn, steps: int, warmup: int):
    """Runs fn(i) `warmup` times untimed, then times exactly `steps` calls with events recorded on
    the launch stream.  fn is a pre-bound C-ABI call (all arguments marshalled beforehand), so the
    host cost of a launch stays below the GPU time of a step."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    s.record()
    for i in range(steps):
        fn(warmup + i)
    e.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return s.elapsed_time(e) / steps, wall


def _bound(name: str, *args):
    """A step function calling the C entry point `name` with pre-marshalled integer arguments;
    args may hold per-step lists (indexed by the step number modulo their length)."""
    import block_quantized_weight_affine_amd as qg
    f = getattr(qg.lib(), name)
    rot = [i for i, a in enumerate(args) if isinstance(a, list)]
    base = list(args)

    if not rot:
        def step(i):
            st = f(*base)
            if st:
                raise qg.QGError(st, name)
    else:
        period = len(args[rot[0]])
        table = []
        for j in range(period):
            a = list(base)
            for r in rot:
                a[r] = args[r][j]
            table.append(tuple(a))

        def step(i):
            st = f(*table[i % period])
            if st:
                raise qg.QGError(st, name)
    return step


# ---------------------------------------------------------------------------------------------------
def _fast_kernel(fmt: str, N: int, T: int) -> str:
    """The kernel the fast-mode dispatcher picks for a dense call: decoded tiles (256 x 256, 128 x 256
    or 128 x 128 rows x tokens) while they still give about 200 workgroups, else 128 x 64 tiles with K
    split over the wavefronts (Q8A: 128 x 128 decoded tiles)."""
    def wgs(bt, bn):
        return ((N + bn - 1) // bn) * ((T + bt - 1) // bt)
    if wgs(256, 256) >= 200 or wgs(128, 256) >= 200 or wgs(128, 128) >= 200 or fmt == "q8a":
        return "gemm_fast_lds_kernel"
    return "gemm_fast_kz_kernel"


def setup_dense(ci: int, mode: str, copies: int):
    import torch
    import block_quantized_weight_affine_amd as qg
    import synth
    c = synth.CONFIGS[ci]
    w = synth.make_dense(c.fmt, c.N, c.K, c.T, c.xtype, c.x_sigma, c.seed, group=c.group)
    codes = [_dev(w["codes"]) for _ in range(copies)]
    scales = [_dev(w["scales"]) for _ in range(copies)]
    offs = [_dev(w["offsets"]) for _ in range(copies)] if c.fmt == "q4a" else [None] * copies
    X = _dev(w["X"])
    if c.xtype == "bf16":
        X = X.view(torch.bfloat16)
    Y = torch.empty((c.T, c.N), dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    xt = {"f32": qg.QG_X_F32, "f16": qg.QG_X_F16, "bf16": qg.QG_X_BF16}[c.xtype]
    cp = [t.data_ptr() for t in codes]
    sp = [t.data_ptr() for t in scales]
    md = qg.MODE[mode]
    if c.fmt == "q4a":
        op = [t.data_ptr() for t in offs]
        step = _bound("qgemm_q4a", cp, sp, op, c.group, X.data_ptr(), xt, Y.data_ptr(), c.N, c.K, c.T, md, st)
    else:
        step = _bound("qgemm_" + c.fmt, cp, sp, X.data_ptr(), xt, Y.data_ptr(), c.N, c.K, c.T, md, st)

    wbytes = w["codes"].nbytes + w["scales"].nbytes + (w["offsets"].nbytes if c.fmt == "q4a" else 0)
    xbytes = w["X"].nbytes
    ybytes = c.T * c.N * 4
    info = {
        "name": c.name, "cfg": c, "mode": mode, "flops": 2.0 * c.T * c.N * c.K,
        "bytes": float(wbytes + xbytes + ybytes), "copies": copies, "weights": w,
        "dtype": ("f32" if mode == "exact" else c.xtype),
        "kernel": (("gemv1_split_kernel" if c.T == 1 and c.K <= 16384 else
                    "gemv_ksplit_kernel" if c.T >= 2 and c.K <= (16384 if c.T <= 4 else 8192) else "gemv_kernel")
                   if c.T <= 8
                   else ("gemm_exact_kernel" if mode == "exact" else _fast_kernel(c.fmt, c.N, c.T))),
        "keep": (codes, scales, offs, X, Y),
    }
    return step, info


def setup_moe(mode: str):
    import torch
    import block_quantized_weight_affine_amd as qg
    import synth
    c = synth.CONFIGS[4]
    E, H, I, T, k = c.extra["experts"], c.N, c.extra["inter"], c.T, c.extra["top_k"]
    m = synth.make_moe(E, H, I, T, c.seed)
    t0 = time.perf_counter()
    plan = qg.qg_moe_plan_host(m["logits"].reshape(T, E), T, E, k)
    plan_ms = (time.perf_counter() - t0) * 1e3
    G, GS = _dev(m["gu_codes"]), _dev(m["gu_scales"])
    D, DS = _dev(m["dn_codes"]), _dev(m["dn_scales"])
    tg = qg.expert_table([(G[e], GS[e], None) for e in range(E)])
    td = qg.expert_table([(D[e], DS[e], None) for e in range(E)])
    pd = {key: _dev(plan[key]) for key in ("seg_off", "row_src", "slot_row", "slot_w")}
    X = _dev(m["X"].reshape(T, H))
    Y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws_bytes = qg.qg_moe_ffn_workspace(H, I, T, k, mode)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    step = _bound("qg_moe_ffn", qg.QG_FMT_Q4, tg.data_ptr(), td.data_ptr(), 64, E, H, I, X.data_ptr(), T, k,
                  pd["seg_off"].data_ptr(), pd["row_src"].data_ptr(), pd["slot_row"].data_ptr(),
                  pd["slot_w"].data_ptr(), Y.data_ptr(), 0, qg.MODE[mode], ws.data_ptr(), ws_bytes, st)
    # the routing plan built on the device instead (qg_moe_plan), timed on its own: the step keeps the
    # host plan, whose time is reported as plan_host_ms
    lg = _dev(np.ascontiguousarray(m["logits"].reshape(T, E), dtype=np.float32))
    dp = [torch.empty(n, dtype=dt, device="cuda") for n, dt in
          ((E + 1, torch.int32), (T * k, torch.int32), (T * k, torch.int32), (T * k, torch.float32))]
    plan_step = _bound("qg_moe_plan", lg.data_ptr(), T, E, k, *[t.data_ptr() for t in dp], None, None, st)
    plan_dev_ms, _ = _timed(plan_step, 200, 20)
    keep = (G, GS, D, DS, tg, td, pd, X, Y, ws, lg, dp)

    used = int(np.count_nonzero(np.diff(plan["seg_off"])))
    gu_b = m["gu_codes"][0].nbytes + m["gu_scales"][0].nbytes
    dn_b = m["dn_codes"][0].nbytes + m["dn_scales"][0].nbytes
    info = {
        "name": c.name, "cfg": c, "mode": mode, "flops": 2.0 * T * k * (2 * I * H + H * I),
        "bytes": float(used * (gu_b + dn_b) + 2 * T * H * 4), "used_experts": used, "plan_host_ms": plan_ms,
        "plan_device_us": plan_dev_ms * 1e3,
        "copies": 1, "dtype": "f32" if mode == "exact" else "f16",
        "kernel": "grouped_rows_kernel", "keep": keep,
    }
    return step, info


def setup(name: str):
    ci, mode = WORKLOADS[name]
    if ci == 4:
        return setup_moe(mode)
    copies = 16 if ci == 1 else 1
    return setup_dense(ci, mode, copies)


def measure_batch(steps: int, warmup: int) -> dict:
    """Decode step of three Q8 matrices sharing X (q / k / v shaped: N 4096, 1024, 1024; K 4096; T 1)
    as one qgemm_batch call, against the same three matrices as three qgemv_q8 calls.  Each step
    reads the next of 12 weight sets (340 MB, more than the 256 MB Infinity Cache)."""
    import torch
    import block_quantized_weight_affine_amd as qg
    import synth
    K, Ns, copies = 4096, (4096, 1024, 1024), 12
    base = [synth.make_dense("q8", N, K, 1, "f32", 1.0, 1001 + 10 * i) for i, N in enumerate(Ns)]
    dev_sets = []
    for c in range(copies):
        js = []
        for w, N in zip(base, Ns):
            js.append((_dev(w["codes"]), _dev(w["scales"]), torch.empty((1, N), device="cuda"), N))
        dev_sets.append(js)
    X = _dev(base[0]["X"].reshape(1, K))
    st = torch.cuda.current_stream().cuda_stream
    arrs = [qg.job_array([(c_, s_, None, y, N) for (c_, s_, y, N) in js]) for js in dev_sets]
    import ctypes as C
    batch = _bound("qgemm_batch", qg.QG_FMT_Q8, 64, [C.cast(a, C.c_void_p).value for a in arrs], 3, X.data_ptr(),
                   qg.QG_X_F32, K, 1, qg.QG_EXACT, st)
    singles = [_bound("qgemv_q8", [js[i][0].data_ptr() for js in dev_sets], [js[i][1].data_ptr() for js in dev_sets],
                      X.data_ptr(), qg.QG_X_F32, [js[i][2].data_ptr() for js in dev_sets], Ns[i], K, 1, st)
               for i in range(3)]

    def separate(i):
        for f in singles:
            f(i)
    ms_b, _ = _timed(batch, steps, warmup)
    ms_s, _ = _timed(separate, steps, warmup)
    # the same three matrices with T = 4 rows of X (the K-split GEMV: one launch for the three jobs,
    # against three)
    X4 = _dev(synth.normal_as(1001, synth.STREAM_X, 4 * K, 0.0, 1.0, "f32").reshape(4, K))
    y4 = [[torch.empty((4, N), device="cuda") for N in Ns] for _ in range(copies)]
    arrs4 = [qg.job_array([(c_, s_, None, y, N) for (c_, s_, _, N), y in zip(js, ys)])
             for js, ys in zip(dev_sets, y4)]
    batch4 = _bound("qgemm_batch", qg.QG_FMT_Q8, 64, [C.cast(a, C.c_void_p).value for a in arrs4], 3,
                    X4.data_ptr(), qg.QG_X_F32, K, 4, qg.QG_EXACT, st)
    singles4 = [_bound("qgemv_q8", [js[i][0].data_ptr() for js in dev_sets], [js[i][1].data_ptr() for js in dev_sets],
                       X4.data_ptr(), qg.QG_X_F32, [ys[i].data_ptr() for ys in y4], Ns[i], K, 4, st)
                for i in range(3)]

    def separate4(i):
        for f in singles4:
            f(i)
    ms_b4, _ = _timed(batch4, steps, warmup)
    ms_s4, _ = _timed(separate4, steps, warmup)
    nbytes = float(sum(N * (K + K // 32 * 4) + 4 * N for N in Ns) + 4 * K)
    gbs = nbytes / (ms_b * 1e-3) / 1e9
    return {"workload": "q8_batch_qkv_decode", "config": "q8_jobs_N4096_1024_1024_K4096_T1", "mode": "exact",
            "ms_per_step": ms_b, "us_per_step": ms_b * 1e3, "dtype": "f32", "kernel": "gemv1_split_kernel",
            "value": gbs, "unit": "GB/s", "bound": "hbm", "peak": PEAK["hbm"], "frac": gbs / PEAK["hbm"],
            "bytes_per_step": nbytes, "us_three_separate_calls": ms_s * 1e3,
            "us_T4_batched": ms_b4 * 1e3, "us_T4_three_separate_calls": ms_s4 * 1e3,
            "keep": (arrs, dev_sets, X, arrs4, y4, X4)}


def measure_gemv_t(T: int, steps: int, warmup: int, fmt: str = "q8") -> dict:
    """The GEMV decode shape (N = K = 4096, f32 X) with T rows of X, Q8 or Q4 weights: HBM GB/s of its
    algorithmic bytes over rotating weight copies beyond the 256 MB Infinity Cache (Q8: 16 copies,
    302 MB; Q4: 32 copies, 302 MB)."""
    import torch
    import block_quantized_weight_affine_amd as qg
    import synth
    N = K = 4096
    w = synth.make_dense(fmt, N, K, T, "f32", 1.0, 1001)
    copies = 16 if fmt == "q8" else 32
    C_ = [_dev(w["codes"]) for _ in range(copies)]
    S_ = [_dev(w["scales"]) for _ in range(copies)]
    X = _dev(w["X"].reshape(T, K))
    Y = torch.empty((T, N), device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    step = _bound(f"qgemv_{fmt}", [c.data_ptr() for c in C_], [s.data_ptr() for s in S_], X.data_ptr(),
                  qg.QG_X_F32, Y.data_ptr(), N, K, T, st)
    ms, _ = _timed(step, steps, warmup)
    wbytes = N * K + N * K // 32 * 4 if fmt == "q8" else N * K // 2 + N * K // 32 * 2
    nbytes = float(wbytes + T * K * 4 + T * N * 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"{fmt}_gemv_T{T}", "config": f"{fmt}_gemv_T{T}_N4096_K4096", "mode": "exact",
            "ms_per_step": ms, "us_per_step": ms * 1e3, "dtype": "f32",
            "kernel": "gemv1_split_kernel" if T == 1 else "gemv_ksplit_kernel",
            "value": gbs, "unit": "GB/s", "bound": "hbm", "peak": PEAK["hbm"], "frac": gbs / PEAK["hbm"],
            "bytes_per_step": nbytes}


def measure_q6k_decode(steps: int, warmup: int) -> dict:
    """A GGUF Q6_K matrix (N = K = 4096, seeded super-block bytes) repacked on the device into the
    offset-free Q8A16 layout, then the T = 1 decode GEMV (qgemv_q8a16, f32 X, no offsets): HBM GB/s of
    the bytes the GEMV reads (codes N K, an f32 scale per 16 elements, X, Y), 16 rotating weight
    copies (336 MB)."""
    import torch
    import block_quantized_weight_affine_amd as qg
    import synth
    N = K = 4096
    nsb = N * K // 256
    rng = np.random.default_rng(1601)
    src = rng.integers(0, 256, nsb * 210).astype(np.uint8).reshape(nsb, 210)
    d = synth.f16_uniform(1601, 1, nsb, 0.001, 0.004)
    src[:, 208], src[:, 209] = d & 0xFF, d >> 8
    s = _dev(src.reshape(-1))
    copies = 16
    C_ = [torch.empty(N * K, dtype=torch.int8, device="cuda") for _ in range(copies)]
    S_ = [torch.empty(N * K // 16, dtype=torch.float32, device="cuda") for _ in range(copies)]
    for c, sc in zip(C_, S_):
        qg.qg_repack_gguf_q8a16("q6_k", s, N, K, c, sc, None)
    X = _dev(synth.normal_as(1601, synth.STREAM_X, K, 0.0, 1.0, "f32").reshape(1, K))
    Y = torch.empty((1, N), device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    step = _bound("qgemv_q8a16", [c.data_ptr() for c in C_], [x.data_ptr() for x in S_], None, X.data_ptr(),
                  qg.QG_X_F32, Y.data_ptr(), N, K, 1, st)
    ms, _ = _timed(step, steps, warmup)
    nbytes = float(N * K + N * K // 16 * 4 + K * 4 + N * 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": "q6_k_gemv_decode", "config": "gguf_q6_k_as_q8a16_no_offsets_N4096_K4096_T1", "mode": "exact",
            "ms_per_step": ms, "us_per_step": ms * 1e3, "dtype": "f32", "kernel": "gemv1_split_kernel",
            "value": gbs, "unit": "GB/s", "bound": "hbm", "peak": PEAK["hbm"], "frac": gbs / PEAK["hbm"],
            "bytes_per_step": nbytes, "gguf_bytes_per_step": float(nsb * 210)}


def measure_q6k_prefill(steps: int, warmup: int) -> dict:
    """The prefill GEMM shape (N = K = 4096, T = 512, f16 X N(0, 0.5)) over a GGUF Q6_K matrix repacked
    on the device into the offset-free Q8A16 layout: fast mode (the decoded f16 tiles), TFLOP/s vs the
    f16 MFMA peak; the exact-mode time of the same call beside it."""
    import torch
    import block_quantized_weight_affine_amd as qg
    import synth
    N = K = 4096
    T = 512
    nsb = N * K // 256
    rng = np.random.default_rng(1701)
    src = rng.integers(0, 256, nsb * 210).astype(np.uint8).reshape(nsb, 210)
    d = synth.f16_uniform(1701, 1, nsb, 0.001, 0.004)
    src[:, 208], src[:, 209] = d & 0xFF, d >> 8
    codes = torch.empty(N * K, dtype=torch.int8, device="cuda")
    scales = torch.empty(N * K // 16, dtype=torch.float32, device="cuda")
    qg.qg_repack_gguf_q8a16("q6_k", _dev(src.reshape(-1)), N, K, codes, scales, None)
    X = _dev(synth.normal_as(1701, synth.STREAM_X, T * K, 0.0, 0.5, "f16").reshape(T, K))
    Y = torch.empty((T, N), device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    fast = _bound("qgemm_q8a16", codes.data_ptr(), scales.data_ptr(), None, X.data_ptr(), qg.QG_X_F16, Y.data_ptr(),
                  N, K, T, qg.QG_FAST, st)
    exact = _bound("qgemm_q8a16", codes.data_ptr(), scales.data_ptr(), None, X.data_ptr(), qg.QG_X_F16,
                   Y.data_ptr(), N, K, T, qg.QG_EXACT, st)
    ms, _ = _timed(fast, steps, warmup)
    ms_exact, _ = _timed(exact, steps, warmup)
    flops = 2.0 * T * N * K
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": "q6_k_prefill_fast", "config": "gguf_q6_k_as_q8a16_no_offsets_N4096_K4096_T512",
            "mode": "fast", "ms_per_step": ms, "us_per_step": ms * 1e3, "us_exact_mode": ms_exact * 1e3,
            "dtype": "f16", "kernel": "gemm_fast_lds_kernel", "value": tf, "unit": "TFLOP/s", "bound": "mfma",
            "peak": PEAK["f16"], "frac": tf / PEAK["f16"], "flops_per_step": flops}


def measure_q8_prefill(mode: str, steps: int, warmup: int) -> dict:
    """The prefill GEMM shape with Q8 weights (N = K = 4096, T = 512, f16 X N(0, 0.5)) in the two
    fast modes: "fast" rounds each decoded weight q d to f16; "fast_wexact" keeps the codes exact in
    f16 and applies the f32 block scale to each 32-k block's f32 partial.  TFLOP/s vs the f16 MFMA
    peak."""
    import torch
    import block_quantized_weight_affine_amd as qg
    import synth
    N = K = 4096
    T = 512
    w = synth.make_dense("q8", N, K, T, "f16", 0.5, 1402)
    C_, S_ = _dev(w["codes"]), _dev(w["scales"])
    X = _dev(w["X"])
    Y = torch.empty((T, N), device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    step = _bound("qgemm_q8", C_.data_ptr(), S_.data_ptr(), X.data_ptr(), qg.QG_X_F16, Y.data_ptr(), N, K, T,
                  qg.MODE[mode], st)
    ms, _ = _timed(step, steps, warmup)
    tf = 2.0 * T * N * K / (ms * 1e-3) / 1e12
    return {"workload": f"q8_prefill_{mode}", "config": "q8_prefill_N4096_K4096_T512", "mode": mode,
            "ms_per_step": ms, "us_per_step": ms * 1e3, "dtype": "f16", "kernel": "gemm_fast_kz_kernel",
            "value": tf, "unit": "TFLOP/s", "bound": "mfma", "peak": PEAK["f16"], "frac": tf / PEAK["f16"]}


def measure_conv(steps: int, warmup: int) -> dict:
    """A 3 x 3 convolution over a 64 x 64 image with 256 input and 256 output channels, Q4 weights
    (N(0, 1) f32 input, group norm over 32 groups with SiLU on the gathered input, exact mode): one step
    is the normalisation statistics (qg_conv_stats) and the implicit-GEMM convolution (qg_conv2d).
    TFLOP/s of the convolution's 2 * pixels * n_out * K flop against the f32 MFMA peak."""
    import torch
    import block_quantized_weight_affine_amd as qg
    import synth
    H = W = 64
    cin, n_out, ksz, groups = 256, 256, 3, 32
    K = ksz * ksz * cin
    w = synth.make_dense("q4", n_out, K, 1, "f32", 1.0, 1501)
    X = _dev(synth.normal_as(1501, synth.STREAM_X, H * W * cin, 0.0, 1.0, "f32"))
    gb = _dev(np.concatenate([np.ones(cin, np.float32), np.zeros(cin, np.float32)]))
    C_, S_ = _dev(w["codes"]), _dev(w["scales"])
    st_buf = torch.empty((groups, 2), device="cuda")
    Y = torch.empty((H * W, n_out), device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    stats = _bound("qg_conv_stats", X.data_ptr(), H * W, cin, groups, 1e-5, st_buf.data_ptr(), st)
    conv = _bound("qg_conv2d", qg.QG_FMT_Q4, C_.data_ptr(), S_.data_ptr(), X.data_ptr(), H, W, cin, ksz, 1, n_out, 1,
                  groups, st_buf.data_ptr(), gb.data_ptr(), 1, Y.data_ptr(), qg.QG_EXACT, st)

    def step(i):
        stats(i)
        conv(i)
    ms, _ = _timed(step, steps, warmup)
    ms_conv, _ = _timed(conv, steps, warmup)
    flops = 2.0 * H * W * n_out * K
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": "conv3x3_q4_gn_silu", "config": "conv_q4_H64_W64_cin256_k3_nout256_group32_silu",
            "mode": "exact", "ms_per_step": ms, "us_per_step": ms * 1e3, "us_conv_only": ms_conv * 1e3,
            "dtype": "f32", "kernel": "gemm_exact_kernel (tap gather)", "value": tf, "unit": "TFLOP/s",
            "bound": "mfma", "peak": PEAK["f32"], "frac": tf / PEAK["f32"], "flops_per_step": flops}


def measure_repack(steps: int, warmup: int) -> dict:
    """GGUF Q4_0 -> split-layout repack of a 4096 x 4096 matrix (an upload-time step): GB/s of the
    bytes it reads (18 per block) and writes (16 code bytes and a 2-byte scale per block)."""
    import torch
    import block_quantized_weight_affine_amd as qg
    N = K = 4096
    nb = N * K // 32
    rng = np.random.default_rng(3)
    src = rng.integers(0, 256, nb * 18).astype(np.uint8).reshape(nb, 18)
    src[:, 0], src[:, 1] = 0x00, 0x24                      # f16 scale 0.015625
    s = _dev(src.reshape(-1))
    codes = torch.empty(N * K // 2, dtype=torch.uint8, device="cuda")
    scales = torch.empty(nb, dtype=torch.int16, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    step = _bound("qg_repack_gguf", qg.QG_GGUF_Q4_0, s.data_ptr(), N, K, codes.data_ptr(), scales.data_ptr(), st)
    ms, _ = _timed(step, steps, warmup)
    nbytes = float(nb * (18 + 16 + 2))
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": "gguf_q4_0_repack", "config": "gguf_q4_0_repack_N4096_K4096", "mode": "exact",
            "ms_per_step": ms, "us_per_step": ms * 1e3, "dtype": "u8", "kernel": "repack_gguf_kernel",
            "value": gbs, "unit": "GB/s", "bound": "hbm", "peak": PEAK["hbm"], "frac": gbs / PEAK["hbm"],
            "bytes_per_step": nbytes}


def measure(name: str, steps: int, warmup: int) -> dict:
    step, info = setup(name)
    ms, wall = _timed(step, steps, warmup)
    c = info["cfg"]
    out = {"workload": name, "config": info["name"], "mode": info["mode"], "ms_per_step": ms,
           "us_per_step": ms * 1e3, "dtype": info["dtype"], "kernel": info["kernel"]}
    if c.index in (1, 4):
        gbs = info["bytes"] / (ms * 1e-3) / 1e9
        out.update({"value": gbs, "unit": "GB/s", "bound": "hbm", "peak": PEAK["hbm"], "frac": gbs / PEAK["hbm"],
                    "bytes_per_step": info["bytes"]})
        if c.index == 4:
            out.update({"used_experts": info["used_experts"], "plan_host_ms": info["plan_host_ms"],
                        "plan_device_us": info["plan_device_us"],
                        "tflops": info["flops"] / (ms * 1e-3) / 1e12})
    else:
        tf = info["flops"] / (ms * 1e-3) / 1e12
        pk = PEAK["f32"] if info["mode"] == "exact" else PEAK[c.xtype]
        out.update({"value": tf, "unit": "TFLOP/s", "bound": "mfma", "peak": pk, "frac": tf / pk,
                    "flops_per_step": info["flops"]})
    out["_info"] = info
    return out


# ---------------------------------------------------------------------------------------------------
def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_run(c, w, threads):
    import oracle
    _, _, used = oracle.gemm(c.fmt, w["codes"], w["scales"], w.get("offsets"), c.group, c.N, c.K,
                             w["X"].view(np.uint16) if c.xtype != "f32" else w["X"], c.xtype, c.T, threads=threads)
    return used


def _oracle_median(c, w, threads, budget_s):
    """Median over 3 timed batches of repeats of the whole workload, each batch about budget_s / 3 s."""
    t0 = time.perf_counter()
    used = _oracle_run(c, w, threads)
    one = time.perf_counter() - t0
    reps = max(1, min(5000, int(budget_s / 3 / max(one, 1e-4))))
    per = []
    for _ in range(3):
        t0 = time.perf_counter()
        for _ in range(reps):
            _oracle_run(c, w, threads)
        per.append((time.perf_counter() - t0) / reps)
    return float(np.median(per)), reps, int(used)


def cpu_baseline(info: dict, budget_s: float = 12.0) -> dict:
    """The CPU oracle (plain C, f64) as it stands, timed on this host: threaded over output rows with
    the process's CPU share (oracle.default_threads), the median of 3 timed batches; for the tiny Q4
    and the Q8 decode workloads also single-threaded.  Reports the host's core count and CPU model
    beside the thread count used."""
    import oracle
    import synth
    c = info["cfg"]
    w = info["weights"]
    dt, reps, used = _oracle_median(c, w, oracle.default_threads(), budget_s)

    def rate(cfg, seconds, nbytes, flops):
        if cfg.index == 1:
            return nbytes / seconds / 1e9, "GB/s"
        return flops / seconds / 1e12, "TFLOP/s"

    value, unit = rate(c, dt, info["bytes"], info["flops"])
    single = []
    for ci in (0, 1):
        cc = synth.CONFIGS[ci]
        ww = w if ci == c.index else synth.make_dense(cc.fmt, cc.N, cc.K, cc.T, cc.xtype, cc.x_sigma, cc.seed,
                                                      group=cc.group)
        d1, r1, _ = _oracle_median(cc, ww, 1, 3.0)
        nbytes = float(ww["codes"].nbytes + ww["scales"].nbytes + ww["X"].nbytes + cc.T * cc.N * 4)
        v1, u1 = rate(cc, d1, nbytes, 2.0 * cc.T * cc.N * cc.K)
        single.append({"workload": cc.name, "value": v1, "unit": u1, "ms": d1 * 1e3, "threads": 1,
                       "gflops_f64": 2.0 * cc.T * cc.N * cc.K / d1 / 1e9, "repeats": 3 * r1})
    return {"value": value, "unit": unit, "cores": used, "kind": "oracle",
            "sample": f"the whole workload ({c.N} rows x K {c.K}, T {c.T}); median of 3 batches of {reps} "
                      f"repeats, {dt * 1e3:.2f} ms each",
            "threads": used, "host_cores": os.cpu_count(), "cpu_model": _cpu_model(),
            "gflops_f64": info["flops"] / dt / 1e9, "single_thread": single}


def traffic_for(name: str, info: dict, ms: float) -> float | None:
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE / WRITE_SIZE summaries, if they were
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    try:
        t = json.load(open(path))
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash(name):
        return None
    return float(t["hbm_bytes_per_launch"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS))
    ap.add_argument("--no-also", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="calibration only: run a plain device copy of this many bytes --steps times and exit "
                         "(the reference kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.copy_bytes:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda").fill_(7)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "copies": args.steps}))
        return

    head = measure(args.workload, args.steps, args.warmup)
    info = head.pop("_info")
    roofline = {"bound": head["bound"], "achieved": head["value"], "peak": head["peak"],
                "unit": head["unit"], "frac": head["frac"], "traffic": traffic_for(args.workload, info,
                                                                                 head["ms_per_step"]),
                "kernel": head["kernel"], "per_launch": (info["bytes"] if head["unit"] == "GB/s" else info["flops"]),
                # one launch per step: the timed region's mean step is the mean launch duration
                "launch_us_timed": head["ms_per_step"] * 1e3}
    cpu = None
    if not args.no_cpu and info["cfg"].index != 4:
        cpu = cpu_baseline(info)
    also = []
    if not args.no_also:
        for name in WORKLOADS:
            if name == args.workload:
                continue
            st = 128 if "moe" in name or "prefill" in name or "upproj" in name else 512
            r = measure(name, st, 20)
            r_info = r.pop("_info")
            if r["unit"] == "GB/s":
                r["traffic"] = traffic_for(name, r_info, r["ms_per_step"])
            also.append({k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()})
            torch.cuda.empty_cache()
        r = measure_repack(256, 20)
        also.append({k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()})
        r = measure_conv(128, 20)
        also.append({k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()})
        r = measure_batch(512, 50)
        r.pop("keep")
        also.append({k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()})
        for fmt, T in (("q8", 4), ("q4", 1), ("q4", 4)):
            r = measure_gemv_t(T, 512, 50, fmt)
            also.append({k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()})
        r = measure_q6k_decode(512, 50)
        also.append({k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()})
        r = measure_q6k_prefill(128, 20)
        also.append({k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()})
        for mode in ("fast", "fast_wexact"):
            r = measure_q8_prefill(mode, 128, 20)
            also.append({k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()})
    c = info["cfg"]
    line = {
        "metric": "TFLOP/s (prefill qgemm) & HBM GB/s (T=1 qgemv), as % of MI355X roofline",
        "value": round(head["value"], 3), "unit": head["unit"], "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(head["ms_per_step"], 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": head["dtype"], "data": "synthetic",
        "config": {"workload": head["config"], "format": c.fmt, "mode": head["mode"], "N": c.N, "K": c.K,
                   "T": c.T, "x_dtype": c.xtype, "weight_copies": info["copies"], "parallelism": "single GPU"},
        "roofline": {k: (round(v, 5) if isinstance(v, float) else v) for k, v in roofline.items()},
        "cpu_baseline": cpu,
        "also": also,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
