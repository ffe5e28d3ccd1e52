// qg_gemv.hip -- wavefront-reduction GEMV for T <= 8 rows of X, exact f32 arithmetic.
//
// Prior art: page "cortiq-engine 0.8.41 src/gpu_metal/clover.rs", q4rows (a narrow kernel that
// takes at most 8 rows per dispatch, measured faster than tile GEMMs for expert panels) and the
// memory-bound-decode notes of "oxinfer 0.0.5 src/metal.rs" (module notes).  The layout here:
//
//  * A wavefront owns RW consecutive weight rows and walks K in steps of 64 "units" of 16
//    elements, one unit per lane per row: Q4 / Q4A unit u is the 8 code bytes 8u..8u+7 of the
//    row (half of block u/2: low nibbles are elements 32b+8h..+7, high nibbles 32b+16+8h..+7 with
//    b = u/2, h = u%2); Q8 unit u is the 16 code bytes 16u..16u+15.  Consecutive lanes read
//    consecutive bytes, so every load instruction of a wavefront is one contiguous 512 B (Q4) or
//    1 KiB (Q8) run of the row.
//  * The lane's slice of each X row (16 values per unit) is loaded once per step and reused by
//    all RW rows; loads of U steps are issued before any arithmetic.
//  * Q4 / Q8: the f32 partial sum of (nibble - 8) * x (or q * x) over the unit is multiplied by the
//    block scale once (the block scale applied to the f32 partial).  Q4A: each weight is decoded
//    to its f32 value (nibble - 8) * d + m first.
//  * After K, each accumulator is reduced across the 64 lanes with xor-shuffles.
//  * Grouped launches (exact-mode MoE): blockIdx.y is the expert; the block walks the expert's
//    row segment in chunks of at most 8 rows.
#include "qg_device.hpp"
#include "qg_internal.hpp"

namespace qg {

constexpr int kGemvThreads = 256;

template <int FMT>
struct Unit;
template <>
struct Unit<FMT_Q4> {
    uint2 q;
    float d, m;
};
template <>
struct Unit<FMT_Q4A> {
    uint2 q;
    float d, m;
};
template <>
struct Unit<FMT_Q8> {
    uint4 q;
    float d, m;
};

template <int FMT>
__device__ __forceinline__ Unit<FMT> load_unit(const void* codes, const void* scales, const uint16_t* offs,
                                               int group, int K, int n, int u) {
    Unit<FMT> r;
    const size_t bi = (size_t)n * (size_t)(K >> 5) + (size_t)(u >> 1);
    if constexpr (FMT == FMT_Q8) {
        const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)((const int8_t*)codes + (size_t)n * K + (size_t)u * 16));
        r.q = make_uint4(v.x, v.y, v.z, v.w);
        r.d = ((const float*)scales)[bi];
        r.m = 0.f;
    } else {
        const u32x2_t v = __builtin_nontemporal_load((const u32x2_t*)((const uint8_t*)codes + (size_t)n * (K >> 1) + (size_t)u * 8));
        r.q = make_uint2(v.x, v.y);
        r.d = f16_to_f32(((const uint16_t*)scales)[bi]);
        r.m = FMT == FMT_Q4A ? bf16_to_f32(offs[(size_t)n * (size_t)(K / group) + (size_t)((u >> 1) * 32 / group)]) : 0.f;
    }
    return r;
}

// Element offsets of unit u's 16 values: two runs of 8 starting at k0 and k1.
template <int FMT>
__device__ __forceinline__ void unit_runs(int u, int& k0, int& k1) {
    if constexpr (FMT == FMT_Q8) {
        k0 = 16 * u;
        k1 = 16 * u + 8;
    } else {
        const int b = u >> 1, h = u & 1;
        k0 = 32 * b + 8 * h;
        k1 = 32 * b + 16 + 8 * h;
    }
}

// Sum over the unit of w(i) * x[i] with x[0..7] at run k0 and x[8..15] at run k1.
template <int FMT>
__device__ __forceinline__ float unit_dot(const Unit<FMT>& w, const float (&x)[16]) {
    if constexpr (FMT == FMT_Q8) {
        const uint32_t ws[4] = {w.q.x, w.q.y, w.q.z, w.q.w};
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int q = (int)(int8_t)((ws[i >> 2] >> (8 * (i & 3))) & 0xFFu);
            p = fmaf((float)q, x[i], p);
        }
        return p * w.d;
    } else if constexpr (FMT == FMT_Q4) {
        const uint32_t ws[2] = {w.q.x, w.q.y};
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t byte = (ws[i >> 2] >> (8 * (i & 3))) & 0xFFu;
            p = fmaf((float)(byte & 15u) - 8.0f, x[i], p);
            p = fmaf((float)(byte >> 4) - 8.0f, x[8 + i], p);
        }
        return p * w.d;
    } else {
        const uint32_t ws[2] = {w.q.x, w.q.y};
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t byte = (ws[i >> 2] >> (8 * (i & 3))) & 0xFFu;
            const float lo = fmaf((float)(byte & 15u) - 8.0f, w.d, w.m);
            const float hi = fmaf((float)(byte >> 4) - 8.0f, w.d, w.m);
            p = fmaf(lo, x[i], p);
            p = fmaf(hi, x[8 + i], p);
        }
        return p;
    }
}

// RW weight rows starting at nrow0, NT X rows (xrow[t], -1 = zero row), outputs at Y rows yrow0 + t.
template <int FMT, int XT, int RW, int NT>
__device__ __forceinline__ void gemv_rows(const GemmParams& p, const void* codes, const void* scales,
                                          const uint16_t* offs, int nrow0, int yrow0, const int* xrow) {
    constexpr int U = NT == 1 ? 4 : (NT == 2 ? 2 : 1);
    const int lane = threadIdx.x & 63;
    const int K = p.K, units = K >> 4;
    int rows[RW];
#pragma unroll
    for (int r = 0; r < RW; r++) rows[r] = min(nrow0 + r, p.N - 1);
    float acc[RW][NT];
#pragma unroll
    for (int r = 0; r < RW; r++)
#pragma unroll
        for (int t = 0; t < NT; t++) acc[r][t] = 0.f;

    for (int u0 = 0; u0 < units; u0 += 64 * U) {
        Unit<FMT> w[U][RW];
        float x[U][NT][16];
        bool ok[U];
#pragma unroll
        for (int j = 0; j < U; j++) {
            const int u = u0 + 64 * j + lane;
            ok[j] = u < units;
            const int uc = ok[j] ? u : units - 1;
#pragma unroll
            for (int r = 0; r < RW; r++) w[j][r] = load_unit<FMT>(codes, scales, offs, p.group, K, rows[r], uc);
            int k0, k1;
            unit_runs<FMT>(uc, k0, k1);
#pragma unroll
            for (int t = 0; t < NT; t++) {
                if (xrow[t] >= 0 && ok[j]) {
                    float a[8], b[8];
                    x_load8<XT>(p.X, (size_t)xrow[t] * K + k0, a);
                    x_load8<XT>(p.X, (size_t)xrow[t] * K + k1, b);
#pragma unroll
                    for (int i = 0; i < 8; i++) {
                        x[j][t][i] = a[i];
                        x[j][t][8 + i] = b[i];
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 16; i++) x[j][t][i] = 0.f;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < U; j++)
#pragma unroll
            for (int r = 0; r < RW; r++)
#pragma unroll
                for (int t = 0; t < NT; t++) acc[r][t] += unit_dot<FMT>(w[j][r], x[j][t]);
    }

#pragma unroll
    for (int r = 0; r < RW; r++)
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const float v = wave_sum(acc[r][t]);
            const int n = nrow0 + r;
            float sc = 1.f;
            if (p.rs) sc = p.rs[yrow0 + t];
            if (lane == ((r * NT + t) & 63) && n < p.N) p.Y[(size_t)(yrow0 + t) * p.N + n] = v * sc;
        }
}

template <int FMT, int XT, int RW, int NT>
__device__ __forceinline__ void gemv_chunk(const GemmParams& p, const void* codes, const void* scales,
                                           const uint16_t* offs, int nrow0, int c) {
    int xrow[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) {
        const int r = c + t;
        int s = r;
        if (p.row_src) {
            s = p.row_src[r];
            if (s < 0 || s >= p.x_rows) s = -1;
        }
        xrow[t] = s;
    }
    gemv_rows<FMT, XT, RW, NT>(p, codes, scales, offs, nrow0, c, xrow);
}

template <int FMT, int XT, int RW>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(GemmParams p, bool grouped) {
    const int wave = threadIdx.x >> 6;
    const int nrow0 = (blockIdx.x * 4 + wave) * RW;
    int r0 = 0, r1 = p.R;
    const void* codes = p.codes;
    const void* scales = p.scales;
    const uint16_t* offs = p.offs;
    if (grouped) {
        const int e = blockIdx.y;
        r0 = min(max(p.seg_off[e], 0), p.R);
        r1 = min(max(p.seg_off[e + 1], r0), p.R);
        codes = p.experts[e].codes;
        scales = p.experts[e].scales;
        offs = p.experts[e].offsets;
    }
    if (nrow0 >= p.N) return;  // whole wavefront beyond N (no barriers in this kernel)
    for (int c = r0; c < r1; c += 8) {
        switch (min(8, r1 - c)) {
            case 1: gemv_chunk<FMT, XT, RW, 1>(p, codes, scales, offs, nrow0, c); break;
            case 2: gemv_chunk<FMT, XT, RW, 2>(p, codes, scales, offs, nrow0, c); break;
            case 3: gemv_chunk<FMT, XT, RW, 3>(p, codes, scales, offs, nrow0, c); break;
            case 4: gemv_chunk<FMT, XT, RW, 4>(p, codes, scales, offs, nrow0, c); break;
            case 5: gemv_chunk<FMT, XT, RW, 5>(p, codes, scales, offs, nrow0, c); break;
            case 6: gemv_chunk<FMT, XT, RW, 6>(p, codes, scales, offs, nrow0, c); break;
            case 7: gemv_chunk<FMT, XT, RW, 7>(p, codes, scales, offs, nrow0, c); break;
            default: gemv_chunk<FMT, XT, RW, 8>(p, codes, scales, offs, nrow0, c); break;
        }
    }
}

template <int FMT, int XT>
static void gemv_launch(const GemmParams& p, bool grouped, hipStream_t s) {
    constexpr int RW = 2;
    dim3 grid((p.N + 4 * RW - 1) / (4 * RW), grouped ? p.E : 1);
    hipLaunchKernelGGL((gemv_kernel<FMT, XT, RW>), grid, dim3(kGemvThreads), 0, s, p, grouped);
}

template <int FMT>
static void gemv_xt(int xt, const GemmParams& p, bool grouped, hipStream_t s) {
    if (xt == XT_F32) gemv_launch<FMT, XT_F32>(p, grouped, s);
    else if (xt == XT_F16) gemv_launch<FMT, XT_F16>(p, grouped, s);
    else gemv_launch<FMT, XT_BF16>(p, grouped, s);
}

hipError_t launch_gemv(int fmt, int xt, const GemmParams& p, bool grouped, hipStream_t s) {
    if (fmt == FMT_Q4) gemv_xt<FMT_Q4>(xt, p, grouped, s);
    else if (fmt == FMT_Q4A) gemv_xt<FMT_Q4A>(xt, p, grouped, s);
    else gemv_xt<FMT_Q8>(xt, p, grouped, s);
    return hipGetLastError();
}

}  // namespace qg
