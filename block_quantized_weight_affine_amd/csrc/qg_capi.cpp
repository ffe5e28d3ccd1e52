// qg_capi.cpp -- the C ABI declared in include/qgemm.h: argument validation (on the host, before
// any HIP call), kernel selection and launch, the host routing planner and the MoE chain.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <numeric>
#include <vector>

#include "qgemm.h"
#include "qg_internal.hpp"

using qg::GemmParams;

namespace {

constexpr int kMaxN = 1 << 24;
constexpr int kMaxK = 1 << 20;
constexpr int kMaxT = 1 << 21;
constexpr int kMaxGridY = 65535;

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool fmt_ok(int f) {
    return f == QG_FMT_Q4 || f == QG_FMT_Q4A || f == QG_FMT_Q8 || f == QG_FMT_Q8A || f == QG_FMT_Q8A16;
}
// formats of the grouped (MoE) entry points
bool grouped_fmt_ok(int f) { return f == QG_FMT_Q4 || f == QG_FMT_Q4A || f == QG_FMT_Q8; }
// formats with per-block offsets, and the alignment of those offsets
bool has_offs(int f) { return f == QG_FMT_Q4A || f == QG_FMT_Q8A || f == QG_FMT_Q8A16; }
size_t offs_bytes(int f) { return f == QG_FMT_Q4A ? 2 : 4; }
bool xt_ok(int x) { return x == QG_X_F32 || x == QG_X_F16 || x == QG_X_BF16; }
bool mode_ok(int m) { return m == QG_EXACT || m == QG_FAST || m == QG_FAST_WEXACT; }
size_t scale_bytes(int fmt) { return fmt == QG_FMT_Q4 || fmt == QG_FMT_Q4A ? 2 : 4; }

// Shared checks of the dense matmul / GEMV entry points.
qg_status check_dense(int fmt, const void* codes, const void* scales, const uint16_t* offs, int group,
                      const void* X, int xt, const float* Y, int N, int K, int T, int mode) {
    if (!fmt_ok(fmt) || !xt_ok(xt) || !mode_ok(mode)) return QG_EINVAL;
    if (N < 1 || N > kMaxN || K < 32 || K > kMaxK || (K % 32) != 0 || T < 0 || T > kMaxT) return QG_ESHAPE;
    if (fmt == QG_FMT_Q4A && (group < 32 || (group % 32) != 0 || (K % group) != 0)) return QG_ESHAPE;
    if (T == 0) return QG_OK;
    // Q8A16 offsets are optional (NULL: no offset term)
    if (!codes || !scales || !X || !Y || (has_offs(fmt) && fmt != QG_FMT_Q8A16 && !offs)) return QG_EINVAL;
    if (!aligned(codes, 16) || !aligned(X, 16) || !aligned(Y, 4) || !aligned(scales, scale_bytes(fmt)) ||
        (has_offs(fmt) && offs && !aligned(offs, offs_bytes(fmt))))
        return QG_EALIGN;
    return QG_OK;
}

GemmParams dense_params(const void* codes, const void* scales, const uint16_t* offs, int group, const void* X,
                        float* Y, int N, int K, int T) {
    GemmParams p{};
    p.codes = codes;
    p.scales = scales;
    p.offs = offs;
    p.group = group > 0 ? group : 64;
    p.X = X;
    p.Y = Y;
    p.N = N;
    p.K = K;
    p.R = T;
    p.E = 1;
    p.x_rows = T;
    return p;
}

qg_status launched(hipError_t e) { return e == hipSuccess ? QG_OK : QG_ELAUNCH; }

qg_status run_dense(int fmt, const void* codes, const void* scales, const uint16_t* offs, int group, const void* X,
                    int xt, float* Y, int N, int K, int T, int mode, bool gemv_only, hipStream_t s) {
    qg_status st = check_dense(fmt, codes, scales, offs, group, X, xt, Y, N, K, T, mode);
    if (st != QG_OK) return st;
    if (gemv_only && T > 8) return QG_ESHAPE;
    if (T == 0) return QG_OK;
    GemmParams p = dense_params(codes, scales, offs, group, X, Y, N, K, T);
    if (mode == QG_FAST_WEXACT && ((fmt != QG_FMT_Q4 && fmt != QG_FMT_Q8) || xt != QG_X_F16)) return QG_EUNSUPPORTED;
    if (T <= 8) return launched(qg::launch_gemv(fmt, xt, p, false, s));
    // 16-element blocks with f32 X in fast mode: the exact kernel (its result is well inside the fast
    // tolerance)
    if (mode == QG_EXACT || (fmt == QG_FMT_Q8A16 && xt == QG_X_F32))
        return launched(qg::launch_gemm_exact(fmt, xt, p, false, s));
    if (mode == QG_FAST_WEXACT) return launched(qg::launch_gemm_fast_wexact(fmt, p, s));
    if (xt == QG_X_F32) return QG_EUNSUPPORTED;
    return launched(qg::launch_gemm_fast(fmt, xt, p, false, s));
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

const char* qg_strerror(qg_status s) {
    switch (s) {
        case QG_OK: return "ok";
        case QG_EINVAL: return "invalid argument (null pointer, unknown enum value or inconsistent sizes)";
        case QG_EALIGN: return "misaligned pointer";
        case QG_ESHAPE: return "unsupported shape";
        case QG_EUNSUPPORTED: return "unsupported mode / activation type combination";
        case QG_ELAUNCH: return "kernel launch failed";
        case QG_EPLAN: return "invalid routing plan input";
        case QG_EWORKSPACE: return "workspace too small";
        case QG_ESCRATCH: return "the call needs more than the fixed scratch of the no-allocation entry point";
    }
    return "unknown status";
}

int qg_abi_version(void) { return QG_ABI_VERSION; }

qg_status qgemm_q4(const uint8_t* codes, const uint16_t* scales_f16, const void* X, qg_xtype xt, float* Y, int N,
                   int K, int T, qg_mode mode, hipStream_t stream) {
    return run_dense(QG_FMT_Q4, codes, scales_f16, nullptr, 64, X, xt, Y, N, K, T, mode, false, stream);
}

qg_status qgemm_q4a(const uint8_t* codes, const uint16_t* scales_f16, const uint16_t* offsets_bf16, int group,
                    const void* X, qg_xtype xt, float* Y, int N, int K, int T, qg_mode mode, hipStream_t stream) {
    return run_dense(QG_FMT_Q4A, codes, scales_f16, offsets_bf16, group, X, xt, Y, N, K, T, mode, false, stream);
}

qg_status qgemm_q8(const int8_t* codes, const float* scales_f32, const void* X, qg_xtype xt, float* Y, int N, int K,
                   int T, qg_mode mode, hipStream_t stream) {
    return run_dense(QG_FMT_Q8, codes, scales_f32, nullptr, 64, X, xt, Y, N, K, T, mode, false, stream);
}

qg_status qgemm_q8a(const int8_t* codes, const float* scales_f32, const float* offsets_f32, const void* X,
                    qg_xtype xt, float* Y, int N, int K, int T, qg_mode mode, hipStream_t stream) {
    return run_dense(QG_FMT_Q8A, codes, scales_f32, (const uint16_t*)(const void*)offsets_f32, 64, X, xt, Y, N, K, T,
                     mode, false, stream);
}

qg_status qgemm_q8a16(const int8_t* codes, const float* scales_f32, const float* offsets_f32, const void* X,
                      qg_xtype xt, float* Y, int N, int K, int T, qg_mode mode, hipStream_t stream) {
    return run_dense(QG_FMT_Q8A16, codes, scales_f32, (const uint16_t*)(const void*)offsets_f32, 64, X, xt, Y, N, K,
                     T, mode, false, stream);
}

qg_status qgemv_q8a16(const int8_t* codes, const float* scales_f32, const float* offsets_f32, const void* X,
                      qg_xtype xt, float* Y, int N, int K, int T, hipStream_t stream) {
    return run_dense(QG_FMT_Q8A16, codes, scales_f32, (const uint16_t*)(const void*)offsets_f32, 64, X, xt, Y, N, K,
                     T, QG_EXACT, true, stream);
}

qg_status qgemv_q4(const uint8_t* codes, const uint16_t* scales_f16, const void* X, qg_xtype xt, float* Y, int N,
                   int K, int T, hipStream_t stream) {
    return run_dense(QG_FMT_Q4, codes, scales_f16, nullptr, 64, X, xt, Y, N, K, T, QG_EXACT, true, stream);
}

qg_status qgemv_q4a(const uint8_t* codes, const uint16_t* scales_f16, const uint16_t* offsets_bf16, int group,
                    const void* X, qg_xtype xt, float* Y, int N, int K, int T, hipStream_t stream) {
    return run_dense(QG_FMT_Q4A, codes, scales_f16, offsets_bf16, group, X, xt, Y, N, K, T, QG_EXACT, true, stream);
}

qg_status qgemv_q8(const int8_t* codes, const float* scales_f32, const void* X, qg_xtype xt, float* Y, int N, int K,
                   int T, hipStream_t stream) {
    return run_dense(QG_FMT_Q8, codes, scales_f32, nullptr, 64, X, xt, Y, N, K, T, QG_EXACT, true, stream);
}

qg_status qgemv_q8a(const int8_t* codes, const float* scales_f32, const float* offsets_f32, const void* X,
                    qg_xtype xt, float* Y, int N, int K, int T, hipStream_t stream) {
    return run_dense(QG_FMT_Q8A, codes, scales_f32, (const uint16_t*)(const void*)offsets_f32, 64, X, xt, Y, N, K, T,
                     QG_EXACT, true, stream);
}

qg_status qg_dequant_dump(qg_format fmt, const void* codes, const void* scales, const uint16_t* offsets_bf16,
                          int group, int N, int K, int n0, int k0, int rows, int cols, qg_xtype staged, void* out,
                          hipStream_t stream) {
    if (!fmt_ok(fmt) || !xt_ok(staged)) return QG_EINVAL;
    if (N < 1 || N > kMaxN || K < 32 || K > kMaxK || (K % 32) != 0) return QG_ESHAPE;
    if (fmt == QG_FMT_Q4A && (group < 32 || (group % 32) != 0 || (K % group) != 0)) return QG_ESHAPE;
    if (rows < 1 || cols < 32 || (cols % 32) != 0 || (k0 % 32) != 0 || n0 < 0 || k0 < 0 || n0 + rows > N ||
        k0 + cols > K)
        return QG_ESHAPE;
    if (!codes || !scales || !out || (has_offs(fmt) && fmt != QG_FMT_Q8A16 && !offsets_bf16)) return QG_EINVAL;
    if (!aligned(codes, 16) || !aligned(out, 16) || !aligned(scales, scale_bytes(fmt)) ||
        (has_offs(fmt) && offsets_bf16 && !aligned(offsets_bf16, offs_bytes(fmt))))
        return QG_EALIGN;
    return launched(qg::launch_dequant_dump(fmt, codes, scales, offsets_bf16, group, N, K, n0, k0, rows, cols,
                                            staged, out, stream));
}

// ---- routing plan (host) ---------------------------------------------------------------------------
qg_status qg_moe_plan_host(const float* logits, int T, int E, int k, int32_t* seg_off, int32_t* row_src,
                           int32_t* slot_row, float* slot_w, int32_t* slot_expert) {
    if (!logits || !seg_off || !row_src || !slot_row || !slot_w) return QG_EINVAL;
    if (T < 1 || E < 1 || E > 4096 || k < 1 || k > E || (long)T * k > (1L << 30)) return QG_ESHAPE;
    for (long i = 0; i < (long)T * E; i++)
        if (std::isnan(logits[i])) return QG_EPLAN;
    std::vector<int> idx(E), top((size_t)T * k);
    for (int t = 0; t < T; t++) {
        const float* row = logits + (size_t)t * E;
        std::iota(idx.begin(), idx.end(), 0);
        // descending logit; equal logits: lower expert index first
        std::partial_sort(idx.begin(), idx.begin() + k, idx.end(), [row](int a, int b) {
            return row[a] > row[b] || (row[a] == row[b] && a < b);
        });
        const double lmax = row[idx[0]];
        double sum = 0.0;
        for (int j = 0; j < k; j++) sum += std::exp((double)row[idx[j]] - lmax);
        for (int j = 0; j < k; j++) {
            top[(size_t)t * k + j] = idx[j];
            slot_w[(size_t)t * k + j] = (float)(std::exp((double)row[idx[j]] - lmax) / sum);
            if (slot_expert) slot_expert[(size_t)t * k + j] = idx[j];
        }
    }
    std::vector<int32_t> fill(E, 0);
    for (int e = 0; e <= E; e++) seg_off[e] = 0;
    for (size_t i = 0; i < top.size(); i++) seg_off[top[i] + 1]++;
    for (int e = 0; e < E; e++) seg_off[e + 1] += seg_off[e];
    for (int e = 0; e < E; e++) fill[e] = seg_off[e];
    for (int t = 0; t < T; t++)
        for (int j = 0; j < k; j++) {
            const int e = top[(size_t)t * k + j];
            const int r = fill[e]++;
            row_src[r] = t;
            slot_row[(size_t)t * k + j] = r;
        }
    return QG_OK;
}

qg_status qgemm_batch(qg_format fmt, int group, const qg_job* jobs, int J, const void* X, qg_xtype xt, int K,
                      int T, qg_mode mode, hipStream_t stream) {
    if (!jobs) return QG_EINVAL;
    if (J < 1 || J > 64) return QG_ESHAPE;
    if (fmt == QG_FMT_Q8A16) return QG_EUNSUPPORTED;
    for (int j = 0; j < J; j++) {
        const qg_job& b = jobs[j];
        const qg_status st = check_dense(fmt, b.codes, b.scales, b.offsets, group, X, xt, b.Y, b.N, K, T, mode);
        if (st != QG_OK) return st;
    }
    if (T == 0) return QG_OK;
    if (T > 8 && mode == QG_FAST && xt == QG_X_F32) return QG_EUNSUPPORTED;
    if (mode == QG_FAST_WEXACT && ((fmt != QG_FMT_Q4 && fmt != QG_FMT_Q8) || xt != QG_X_F16)) return QG_EUNSUPPORTED;
    if (T <= 8) {
        // T = 1: the streaming GEMV; T = 2..8: the K-split GEMV with one launch column per job
        bool all = true;
        for (int j0 = 0; j0 < J && all; j0 += qg::kMaxBatchJobs) {
            qg::BatchJobs bj{};
            bj.J = std::min(qg::kMaxBatchJobs, J - j0);
            for (int i = 0; i < bj.J; i++) {
                const qg_job& b = jobs[j0 + i];
                bj.start[i + 1] = bj.start[i] + b.N;
                bj.codes[i] = b.codes;
                bj.scales[i] = b.scales;
                bj.offs[i] = b.offsets;
                bj.Y[i] = b.Y;
            }
            GemmParams p = dense_params(nullptr, nullptr, nullptr, group, X, nullptr, bj.start[bj.J], K, T);
            hipError_t err = hipSuccess;
            const bool ok = T == 1 ? qg::launch_gemv1_batch(fmt, xt, p, bj, stream, err)
                                   : qg::launch_gemv_batch(fmt, xt, p, bj, stream, err);
            if (!ok) {
                all = false;  // K beyond the batched kernel: nothing was launched for this group
                for (int j = j0; j < J; j++) {
                    const qg_job& b = jobs[j];
                    const qg_status st = run_dense(fmt, b.codes, b.scales, b.offsets, group, X, xt, b.Y, b.N, K, T,
                                                   mode, false, stream);
                    if (st != QG_OK) return st;
                }
            } else if (err != hipSuccess) {
                return QG_ELAUNCH;
            }
        }
        return QG_OK;
    }
    for (int j = 0; j < J; j++) {
        const qg_job& b = jobs[j];
        const qg_status st = run_dense(fmt, b.codes, b.scales, b.offsets, group, X, xt, b.Y, b.N, K, T, mode, false,
                                       stream);
        if (st != QG_OK) return st;
    }
    return QG_OK;
}

qg_status qg_repack_gguf(qg_gguf_type type, const void* src, int N, int K, void* codes, void* scales,
                         hipStream_t stream) {
    if (type != QG_GGUF_Q4_0 && type != QG_GGUF_Q8_0) return QG_EINVAL;
    if (N < 1 || N > kMaxN || K < 32 || K > kMaxK || (K % 32) != 0) return QG_ESHAPE;
    if (!src || !codes || !scales) return QG_EINVAL;
    const bool q8 = type == QG_GGUF_Q8_0;
    if (!aligned(src, 2) || !aligned(codes, 16) || !aligned(scales, q8 ? 4 : 2)) return QG_EALIGN;
    const size_t nblocks = (size_t)N * (size_t)(K / 32);
    return launched(qg::launch_repack_gguf(q8 ? 1 : 0, src, nblocks, codes, scales, stream));
}

qg_status qg_repack_gguf_q8a(qg_gguf_type type, const void* src, int N, int K, int8_t* codes, float* scales_f32,
                             float* offsets_f32, hipStream_t stream) {
    if (type != QG_GGUF_Q4_1 && type != QG_GGUF_Q5_0 && type != QG_GGUF_Q5_1 && type != QG_GGUF_Q4_K &&
        type != QG_GGUF_Q5_K)
        return QG_EINVAL;
    const bool kq = type == QG_GGUF_Q4_K || type == QG_GGUF_Q5_K;  // 256-element super-blocks
    if (N < 1 || N > kMaxN || K < 32 || K > kMaxK || (K % 32) != 0 || (kq && (K % 256) != 0)) return QG_ESHAPE;
    if (!src || !codes || !scales_f32 || !offsets_f32) return QG_EINVAL;
    if (!aligned(src, 2) || !aligned(codes, 16) || !aligned(scales_f32, 4) || !aligned(offsets_f32, 4))
        return QG_EALIGN;
    const size_t nblocks = (size_t)N * (size_t)(K / 32);
    return launched(qg::launch_repack_gguf_q8a(type, src, nblocks, codes, scales_f32, offsets_f32, stream));
}

qg_status qg_repack_gguf_q8a16(qg_gguf_type type, const void* src, int N, int K, int8_t* codes,
                               float* scales_f32, float* offsets_f32, hipStream_t stream) {
    if (type != QG_GGUF_Q6_K && type != QG_GGUF_Q3_K && type != QG_GGUF_Q2_K) return QG_EINVAL;
    if (N < 1 || N > kMaxN || K < 256 || K > kMaxK || (K % 256) != 0) return QG_ESHAPE;
    // offsets may be omitted for Q6_K and Q3_K (all -0: the offset-free layout)
    if (!src || !codes || !scales_f32 || (!offsets_f32 && type == QG_GGUF_Q2_K)) return QG_EINVAL;
    if (!aligned(src, 2) || !aligned(codes, 16) || !aligned(scales_f32, 4) ||
        (offsets_f32 && !aligned(offsets_f32, 4)))
        return QG_EALIGN;
    const size_t nblk16 = (size_t)N * (size_t)(K / 16);
    return launched(qg::launch_repack_gguf_q8a16(type, src, nblk16, codes, scales_f32, offsets_f32, stream));
}

qg_status qg_repack_q8f(const void* blob, int N, int K, int has_col, float* scales, float* col, hipStream_t stream) {
    if (N < 1 || N > kMaxN || K < 32 || K > kMaxK || (K % 32) != 0) return QG_ESHAPE;
    if (!blob || !scales || (has_col && !col)) return QG_EINVAL;
    if (!aligned(blob, 16) || !aligned(scales, 4) || (has_col && !aligned(col, 16))) return QG_EALIGN;
    return launched(qg::launch_repack_q8f(blob, N, K, has_col != 0, scales, has_col ? col : nullptr, stream));
}

qg_status qg_col_scale(const void* X, qg_xtype xt, int T, int K, const float* col, void* Xs, qg_xtype st,
                       hipStream_t stream) {
    if (!xt_ok(xt) || !xt_ok(st)) return QG_EINVAL;
    if (T < 0 || T > kMaxT || K < 8 || K > kMaxK || (K % 8) != 0) return QG_ESHAPE;
    if (T == 0) return QG_OK;
    if (!X || !col || !Xs) return QG_EINVAL;
    if (!aligned(X, 16) || !aligned(col, 16) || !aligned(Xs, 16)) return QG_EALIGN;
    return launched(qg::launch_col_scale(X, (int)xt, T, K, col, Xs, (int)st, stream));
}

qg_status qg_conv_stats(const float* X, int npix, int cin, int groups, float eps, float* stats, hipStream_t stream) {
    if (npix < 1 || npix > (1 << 26) || cin < 1 || cin > kMaxK || groups < 0 || groups > kMaxGridY ||
        (groups > 0 && (cin % groups) != 0) || (int64_t)npix * cin >= ((int64_t)1 << 31))
        return QG_ESHAPE;
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return QG_EINVAL;
    if (!X || !stats) return QG_EINVAL;
    if (!aligned(X, 4) || !aligned(stats, 4)) return QG_EALIGN;
    return launched(qg::launch_conv_stats(X, npix, cin, groups, eps, stats, stream));
}

qg_status qg_conv2d(qg_format fmt, const void* codes, const void* scales, const float* X, int H, int W, int cin,
                    int ksize, int stride, int n_out, int norm, int groups, const float* stats,
                    const float* gamma_beta, int silu, float* Y, qg_mode mode, hipStream_t stream) {
    if (!fmt_ok(fmt) || !mode_ok(mode) || norm < 0 || norm > 2 || (silu != 0 && silu != 1)) return QG_EINVAL;
    if (silu && norm == 0) return QG_EINVAL;
    if ((fmt != QG_FMT_Q4 && fmt != QG_FMT_Q8) || mode != QG_EXACT) return QG_EUNSUPPORTED;
    if (H < 1 || W < 1 || (int64_t)H * W > ((int64_t)1 << 26) || cin < 32 || (cin % 32) != 0 || ksize < 1 ||
        ksize > 64 || stride < 1 || n_out < 1 || n_out > kMaxN || (int64_t)H * W * cin >= ((int64_t)1 << 31))
        return QG_ESHAPE;
    const int64_t K = (int64_t)ksize * ksize * cin;
    if (K > kMaxK) return QG_ESHAPE;
    const int pad = ksize / 2;
    const int oh = (H + 2 * pad - ksize) / stride + 1, ow = (W + 2 * pad - ksize) / stride + 1;
    const int64_t R = (int64_t)oh * ow;
    if (R > kMaxT || (R + 31) / 32 > kMaxGridY) return QG_ESHAPE;
    if (norm == 1 && (groups < 1 || (cin % groups) != 0)) return QG_ESHAPE;
    if (!codes || !scales || !X || !Y || (norm && (!stats || !gamma_beta))) return QG_EINVAL;
    if (!aligned(codes, 16) || !aligned(scales, scale_bytes(fmt)) || !aligned(X, 16) || !aligned(Y, 4) ||
        (norm && (!aligned(stats, 4) || !aligned(gamma_beta, 4))))
        return QG_EALIGN;
    GemmParams p = dense_params(codes, scales, nullptr, 64, X, Y, n_out, (int)K, (int)R);
    qg::ConvParams cv{};
    cv.H = H;
    cv.W = W;
    cv.cin = cin;
    cv.ksz = ksize;
    cv.stride = stride;
    cv.pad = pad;
    cv.ow = ow;
    cv.norm = norm;
    cv.cpg = norm == 1 ? cin / groups : 1;
    cv.silu = silu;
    cv.stats = stats;
    cv.gb = gamma_beta;
    return launched(qg::launch_conv_exact(fmt, p, cv, stream));
}

qg_status qg_moe_plan(const float* logits, int T, int E, int k, int32_t* seg_off, int32_t* row_src,
                      int32_t* slot_row, float* slot_w, int32_t* slot_expert, int32_t* status, hipStream_t stream) {
    if (T < 1 || E < 1 || E > 1024 || k < 1 || k > E || k > 32 || (long)T * k > 16384) return QG_ESHAPE;
    if (!logits || !seg_off || !row_src || !slot_row || !slot_w) return QG_EINVAL;
    if (!aligned(logits, 4) || !aligned(seg_off, 4) || !aligned(row_src, 4) || !aligned(slot_row, 4) ||
        !aligned(slot_w, 4) || (slot_expert && !aligned(slot_expert, 4)) || (status && !aligned(status, 4)))
        return QG_EALIGN;
    return launched(qg::launch_moe_plan(logits, T, E, k, seg_off, row_src, slot_row, slot_w, slot_expert, status,
                                        QG_EPLAN, stream));
}

qg_status qg_x_half(const float* X, int x_rows, const int32_t* row_src, int R, int K, uint16_t* Xh, float* rs,
                    hipStream_t stream) {
    if (R < 0 || R > kMaxT || K < 8 || K > kMaxK || (K % 8) != 0 || x_rows < 0) return QG_ESHAPE;
    if (R == 0) return QG_OK;
    if (!X || !Xh || !rs) return QG_EINVAL;
    if (!aligned(X, 16) || !aligned(Xh, 16) || !aligned(rs, 4) || (row_src && !aligned(row_src, 4)))
        return QG_EALIGN;
    return launched(qg::launch_x_half(X, x_rows, row_src, R, K, -1, Xh, rs, stream));
}

qg_status qg_x_half_guard(const float* X, int x_rows, const int32_t* row_src, int R, int K, int shift, uint16_t* Xh,
                          float* rs, hipStream_t stream) {
    if (shift < 0 || shift > 14) return QG_EINVAL;
    if (R < 0 || R > kMaxT || K < 8 || K > kMaxK || (K % 8) != 0 || x_rows < 0) return QG_ESHAPE;
    if (R == 0) return QG_OK;
    if (!X || !Xh) return QG_EINVAL;
    if (!aligned(X, 16) || !aligned(Xh, 16) || (rs && !aligned(rs, 4)) || (row_src && !aligned(row_src, 4)))
        return QG_EALIGN;
    return launched(qg::launch_x_half(X, x_rows, row_src, R, K, shift, Xh, rs, stream));
}

qg_status qgemm_moe_grouped(qg_format fmt, const qg_expert* experts, int group, const int32_t* seg_off,
                            const int32_t* row_src, int x_rows, const void* X, qg_xtype xt, const float* rs,
                            float* Y, int N, int K, int R, int E, qg_mode mode, hipStream_t stream) {
    if (!fmt_ok(fmt) || !xt_ok(xt) || !mode_ok(mode)) return QG_EINVAL;
    if (mode == QG_FAST_WEXACT || !grouped_fmt_ok(fmt)) return QG_EUNSUPPORTED;
    if (N < 1 || N > kMaxN || K < 32 || K > kMaxK || (K % 32) != 0 || R < 0 || R > kMaxT || E < 1 ||
        E > kMaxGridY || x_rows < 0)
        return QG_ESHAPE;
    if (fmt == QG_FMT_Q4A && (group < 32 || (group % 32) != 0 || (K % group) != 0)) return QG_ESHAPE;
    if ((mode == QG_FAST || R > 8 * E) && (R + 31) / 32 + std::min(E, R) > kMaxGridY) return QG_ESHAPE;
    if (R == 0) return QG_OK;
    if (!experts || !seg_off || !X || !Y) return QG_EINVAL;
    if (!aligned(experts, 8) || !aligned(seg_off, 4) || !aligned(X, 16) || !aligned(Y, 4) ||
        (row_src && !aligned(row_src, 4)) || (rs && !aligned(rs, 4)))
        return QG_EALIGN;
    // fast mode with f32 X: the rows are scaled to f16 inside the expert-row kernel, which takes K up
    // to 2048 (Q4, Q4A) or 1024 (Q8)
    if (mode == QG_FAST && xt == QG_X_F32 && !qg::grouped_rows_fits(fmt, K, N, 0)) return QG_EUNSUPPORTED;
    GemmParams p{};
    p.experts = (const qg::ExpertPtr*)experts;
    p.seg_off = seg_off;
    p.row_src = row_src;
    p.x_rows = row_src ? x_rows : R;
    p.X = X;
    p.rs = rs;
    p.Y = Y;
    p.group = group > 0 ? group : 64;
    p.N = N;
    p.K = K;
    p.R = R;
    p.E = E;
    // Short segments (at most 8 rows per expert on average) stream each expert's weights once
    // through the expert-row kernel (f32 arithmetic; fast mode with f16 or f32 X: f16 X through
    // v_dot2), or the K-split GEMV where K is past that kernel's limit; longer segments would
    // re-read the weights for every 4 rows, so they take the MFMA tile kernels.
    const bool fast = mode == QG_FAST;
    if (fast && xt == QG_X_F32) return launched(qg::launch_grouped_rows(fmt, xt, true, 0, p, stream));
    if (R <= 8 * E) {
        if (qg::grouped_rows_fits(fmt, K, N, 0)) return launched(qg::launch_grouped_rows(fmt, xt, fast, 0, p, stream));
        if (!fast) return launched(qg::launch_gemv(fmt, xt, p, true, stream));
    }
    if (!fast) return launched(qg::launch_gemm_exact(fmt, xt, p, true, stream));
    return launched(qg::launch_gemm_fast(fmt, xt, p, true, stream));
}

qg_status qg_swiglu(const float* GU, int R, int I, void* A, qg_xtype at, float* rs, hipStream_t stream) {
    if (at != QG_X_F32 && at != QG_X_F16) return xt_ok(at) ? QG_EUNSUPPORTED : QG_EINVAL;
    if (R < 0 || R > kMaxT || I < 8 || (I % 8) != 0 || I > kMaxK) return QG_ESHAPE;
    if (R == 0) return QG_OK;
    if (!GU || !A || (at == QG_X_F16 && !rs)) return QG_EINVAL;
    if (!aligned(GU, 16) || !aligned(A, 16) || (rs && !aligned(rs, 4))) return QG_EALIGN;
    return launched(qg::launch_swiglu(GU, R, I, A, at, rs, stream));
}

qg_status qg_moe_combine(const float* O, int R, const int32_t* slot_row, const float* slot_w, float* Y, int H,
                         int T, int k, int accumulate, hipStream_t stream) {
    if (R < 0 || H < 4 || (H % 4) != 0 || H > kMaxK || T < 0 || T > kMaxGridY || k < 1 || k > 4096)
        return QG_ESHAPE;
    if (T == 0) return QG_OK;
    if (!O || !slot_row || !slot_w || !Y) return QG_EINVAL;
    if (!aligned(O, 16) || !aligned(Y, 16) || !aligned(slot_row, 4) || !aligned(slot_w, 4)) return QG_EALIGN;
    return launched(qg::launch_moe_combine(O, R, slot_row, slot_w, Y, H, T, k, accumulate ? 1 : 0, stream));
}

size_t qg_moe_ffn_workspace(int H, int I, int T, int k, qg_mode mode) {
    if (H < 1 || I < 1 || T < 0 || k < 1) return 0;
    const size_t R = (size_t)T * (size_t)k;
    size_t b = align256(R * 2 * I * 4) + align256(R * H * 4);  // GU, O
    if (mode == QG_FAST)
        b += align256(R * H * 2) + 2 * align256(R * 4) + align256(R * I * 2);  // Xh, rs1, rs2, A f16
    else
        b += align256(R * I * 4);  // A f32
    return b;
}

}  // extern "C"

namespace {

// Every check of the expert block's arguments except the workspace, before any HIP call (the stage
// entry points check again what they need; with these passed, none of them can fail after an
// earlier stage was launched).
qg_status check_ffn(int fmt, const qg_expert* gate_up, const qg_expert* down, int group, int E, int H, int I,
                    const float* X, int T, int k, const int32_t* seg_off, const int32_t* row_src,
                    const int32_t* slot_row, const float* slot_w, const float* Y, int mode) {
    if (!fmt_ok(fmt) || !mode_ok(mode)) return QG_EINVAL;
    if (mode == QG_FAST_WEXACT || !grouped_fmt_ok(fmt)) return QG_EUNSUPPORTED;
    if (E < 1 || E > kMaxGridY || H < 32 || (H % 32) != 0 || H > kMaxK || I < 32 || (I % 32) != 0 || I > kMaxK ||
        T < 0 || T > kMaxGridY || k < 1 || k > E || (int64_t)T * k > kMaxT)
        return QG_ESHAPE;
    if (fmt == QG_FMT_Q4A && (group < 32 || (group % 32) != 0 || (H % group) != 0 || (I % group) != 0))
        return QG_ESHAPE;
    const int R = T * k;
    if ((mode == QG_FAST || R > 8 * E) && (R + 31) / 32 + std::min(E, R) > kMaxGridY) return QG_ESHAPE;
    if (T == 0) return QG_OK;
    if (!gate_up || !down || !X || !seg_off || !row_src || !slot_row || !slot_w || !Y) return QG_EINVAL;
    if (!aligned(gate_up, 8) || !aligned(down, 8) || !aligned(X, 16) || !aligned(Y, 16) || !aligned(seg_off, 4) ||
        !aligned(row_src, 4) || !aligned(slot_row, 4) || !aligned(slot_w, 4))
        return QG_EALIGN;
    return QG_OK;
}

}  // namespace

extern "C" {

qg_status qg_moe_ffn(qg_format fmt, const qg_expert* gate_up, const qg_expert* down, int group, int E, int H, int I,
                     const float* X, int T, int k, const int32_t* seg_off, const int32_t* row_src,
                     const int32_t* slot_row, const float* slot_w, float* Y, int accumulate, qg_mode mode,
                     void* workspace, size_t ws_bytes, hipStream_t stream) {
    qg_status st = check_ffn(fmt, gate_up, down, group, E, H, I, X, T, k, seg_off, row_src, slot_row, slot_w, Y,
                             mode);
    if (st != QG_OK || T == 0) return st;
    if (!workspace) return QG_EINVAL;
    if (!aligned(workspace, 256)) return QG_EALIGN;
    if (ws_bytes < qg_moe_ffn_workspace(H, I, T, k, mode)) return QG_EWORKSPACE;
    const int R = T * k;
    char* w = (char*)workspace;
    if (R <= 8 * E && qg::grouped_rows_fits(fmt, H, 2 * I, 1) && qg::grouped_rows_fits(fmt, I, H, 0)) {
        // Short segments: gate|up with SwiGLU in its epilogue (A f32), then down, then the combine;
        // fast mode scales the f32 rows of X and of A to f16 inside the two matmuls.
        const bool fast = mode == QG_FAST;
        float* A = (float*)w;
        float* O = (float*)(w + align256((size_t)R * I * 4));
        GemmParams p{};
        p.experts = (const qg::ExpertPtr*)gate_up;
        p.seg_off = seg_off;
        p.row_src = row_src;
        p.x_rows = T;
        p.X = X;
        p.Y = A;
        p.group = group > 0 ? group : 64;
        p.N = 2 * I;
        p.K = H;
        p.R = R;
        p.E = E;
        if ((st = launched(qg::launch_grouped_rows(fmt, QG_X_F32, fast, 1, p, stream))) != QG_OK) return st;
        p.experts = (const qg::ExpertPtr*)down;
        p.row_src = nullptr;
        p.x_rows = R;
        p.X = A;
        p.Y = O;
        p.N = H;
        p.K = I;
        if ((st = launched(qg::launch_grouped_rows(fmt, QG_X_F32, fast, 0, p, stream))) != QG_OK) return st;
        return qg_moe_combine(O, R, slot_row, slot_w, Y, H, T, k, accumulate, stream);
    }
    float* GU = (float*)w;
    w += align256((size_t)R * 2 * I * 4);
    float* O = (float*)w;
    w += align256((size_t)R * H * 4);
    if (mode == QG_FAST) {
        uint16_t* Xh = (uint16_t*)w;
        w += align256((size_t)R * H * 2);
        float* rs1 = (float*)w;
        w += align256((size_t)R * 4);
        float* rs2 = (float*)w;
        w += align256((size_t)R * 4);
        uint16_t* A = (uint16_t*)w;
        if ((st = qg_x_half(X, T, row_src, R, H, Xh, rs1, stream)) != QG_OK) return st;
        if ((st = qgemm_moe_grouped(fmt, gate_up, group, seg_off, nullptr, R, Xh, QG_X_F16, rs1, GU, 2 * I, H, R, E,
                                    QG_FAST, stream)) != QG_OK)
            return st;
        if ((st = qg_swiglu(GU, R, I, A, QG_X_F16, rs2, stream)) != QG_OK) return st;
        if ((st = qgemm_moe_grouped(fmt, down, group, seg_off, nullptr, R, A, QG_X_F16, rs2, O, H, I, R, E, QG_FAST,
                                    stream)) != QG_OK)
            return st;
    } else {
        float* A = (float*)w;
        if ((st = qgemm_moe_grouped(fmt, gate_up, group, seg_off, row_src, T, X, QG_X_F32, nullptr, GU, 2 * I, H, R,
                                    E, QG_EXACT, stream)) != QG_OK)
            return st;
        if ((st = qg_swiglu(GU, R, I, A, QG_X_F32, nullptr, stream)) != QG_OK) return st;
        if ((st = qgemm_moe_grouped(fmt, down, group, seg_off, nullptr, R, A, QG_X_F32, nullptr, O, H, I, R, E,
                                    QG_EXACT, stream)) != QG_OK)
            return st;
    }
    return qg_moe_combine(O, R, slot_row, slot_w, Y, H, T, k, accumulate, stream);
}

qg_status qg_moe_ffn_noalloc(qg_format fmt, const qg_expert* gate_up, const qg_expert* down, int group, int E,
                             int H, int I, const float* X, int T, int k, const int32_t* seg_off,
                             const int32_t* row_src, const int32_t* slot_row, const float* slot_w, float* Y,
                             int accumulate, qg_mode mode, hipStream_t stream) {
    qg_status st = check_ffn(fmt, gate_up, down, group, E, H, I, X, T, k, seg_off, row_src, slot_row, slot_w, Y,
                             mode);
    if (st != QG_OK || T == 0) return st;
    if (qg_moe_ffn_workspace(H, I, T, k, mode) > (size_t)QG_NOALLOC_SCRATCH_BYTES) return QG_ESCRATCH;
    void* ws = nullptr;
    if (qg::noalloc_scratch(&ws) != hipSuccess) return QG_ELAUNCH;
    return qg_moe_ffn(fmt, gate_up, down, group, E, H, I, X, T, k, seg_off, row_src, slot_row, slot_w, Y, accumulate,
                      mode, ws, QG_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
