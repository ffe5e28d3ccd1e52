// qg_gemv.hip -- wavefront-reduction GEMV for at most 8 rows of X, exact f32 arithmetic.
//
// Prior art: page "cortiq-engine 0.8.41 src/gpu_metal/clover.rs", q4rows (a narrow kernel that
// takes at most 8 rows per dispatch, measured faster than tile GEMMs for expert panels) and the
// memory-bound-decode notes of "oxinfer 0.0.5 src/metal.rs" (module notes).  The layout here:
//
//  * A workgroup is 4 wavefronts; wavefront w owns RW consecutive weight rows.  K is walked in
//    steps of 64 "units" of 16 elements, one unit per lane per row: Q4 / Q4A unit u is the 8 code
//    bytes 8u..8u+7 of the row (half of block u/2: low nibbles are elements 32b+8h..+7, high
//    nibbles 32b+16+8h..+7 with b = u/2, h = u%2); Q8 unit u is the 16 code bytes 16u..16u+15.
//    Consecutive lanes read consecutive bytes, so each load instruction of a wavefront is one
//    contiguous 512 B (Q4) or 1 KiB (Q8) run of a row.
//  * X rows are staged once per workgroup in LDS as f32, in K chunks of at most 16384 values in
//    all; the chunk's X loads are issued first, then every weight load of the chunk, so the X
//    store to LDS waits only for X while the weights stream in.
//  * Per weight row and unit the f32 partial P = sum s_i x_i over signed codes s_i, each a signed
//    byte converted to f32 by one instruction: Q8 s = q; Q4 / Q4A s = 16 (nibble - 8), made by
//    moving the nibble to the byte's high half and flipping its top bit.  Then acc += d P (Q8) or
//    (d / 16) P (Q4), and Q4A adds m Sx with Sx the sum of the unit's 16 x values -- the block
//    scale applied to the f32 partial.
//  * After K, each accumulator is reduced across the 64 lanes with xor shuffles.
//  * Grouped launches (exact-mode MoE): blockIdx.y is the expert; the workgroup walks the expert's
//    row segment in chunks of at most 4 rows.
//
// Kernels: gemv1_split_kernel (one X row: K split over the workgroup, each lane one 16-byte code
// chunk of every weight row, its X values in registers; also the batched launch of several matrices),
// gemv_ksplit_kernel / gemv_ksplit_grouped_kernel (2..8 X rows or an expert's segment chunk: K split
// over the wavefronts in the unit layout above, each lane's X unit in registers, DPP row sums), and
// gemv_kernel (the chunked LDS kernel above, for K beyond the K-split limits).
#include <algorithm>

#include "qg_device.hpp"
#include "qg_internal.hpp"

namespace qg {

constexpr int kGemvThreads = 256;   // workgroup size of the multi-row and grouped launches
constexpr int kGemv1Threads = 512;  // single X row: 8 wavefronts of 2 weight rows share one X copy

template <int NT>
struct GemvChunk {
    static constexpr int steps = NT <= 4 ? 4 : 2;  // 1024-element steps per chunk
    static constexpr int kc = 1024 * steps;        // NT * kc <= 16384 f32 values (64 KiB of LDS)
};

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
template <>
struct Unit<FMT_Q8A> {
    uint4 q;
    float d, m;
};
// a unit of 16 Q8 values is exactly one 16-element block
template <>
struct Unit<FMT_Q8A16> {
    uint4 q;
    float d, m;
};
// formats with an offset term (the partial then needs the unit's x sum)
template <int FMT>
constexpr bool has_offs = FMT == FMT_Q4A || FMT == FMT_Q8A || FMT == FMT_Q8A16;

template <int FMT>
__device__ __forceinline__ Unit<FMT> load_unit(const void* codes, const void* scales, const uint16_t* offs,
                                               int group, int K, int n, int u) {
    Unit<FMT> r;
    const size_t bi = blk16<FMT> ? (size_t)n * (size_t)(K >> 4) + (size_t)u : (size_t)n * (size_t)(K >> 5) + (size_t)(u >> 1);
    if constexpr (q8_layout<FMT>) {
        const u32x4_t v =
            __builtin_nontemporal_load((const u32x4_t*)((const int8_t*)codes + (size_t)n * K + (size_t)u * 16));
        r.q = make_uint4(v.x, v.y, v.z, v.w);
        r.d = ((const float*)scales)[bi];
        if constexpr (blk16<FMT>) r.m = offs ? ((const float*)(const void*)offs)[bi] : -0.0f;  // NULL: none
        else r.m = has_offs<FMT> ? ((const float*)(const void*)offs)[bi] : 0.f;
    } else {
        const u32x2_t v =
            __builtin_nontemporal_load((const u32x2_t*)((const uint8_t*)codes + (size_t)n * (K >> 1) + (size_t)u * 8));
        r.q = make_uint2(v.x, v.y);
        r.d = f16_to_f32(((const uint16_t*)scales)[bi]);
        r.m = FMT == FMT_Q4A ? bf16_to_f32(offs[(size_t)n * (size_t)(K / group) + (size_t)((u >> 1) * 32 / group)])
                             : 0.f;
    }
    return r;
}

// Element offsets (within the row) of unit u's two runs of 8 values.
template <int FMT>
__device__ __forceinline__ void unit_runs(int u, int& k0, int& k1) {
    if constexpr (q8_layout<FMT>) {
        k0 = 16 * u;
        k1 = 16 * u + 8;
    } else {
        const int b = u >> 1, h = u & 1;
        k0 = 32 * b + 8 * h;
        k1 = 32 * b + 16 + 8 * h;
    }
}

__device__ __forceinline__ float sbyte_f32(uint32_t word, int i) { return (float)(int8_t)(word >> (8 * i)); }

// sum_i s_i x_i over the unit's 16 signed codes (x[0..7] and x[8..15] the unit's two runs): Q8
// s = q; Q4 / Q4A s = 16 (nibble - 8), the byte (nibble << 4) ^ 0x80 read as signed.
template <int FMT>
__device__ __forceinline__ float unit_partial(const Unit<FMT>& w, const float (&x)[16]) {
    float p = 0.f;
    if constexpr (q8_layout<FMT>) {
        const uint32_t ws[4] = {w.q.x, w.q.y, w.q.z, w.q.w};
#pragma unroll
        for (int i = 0; i < 16; i++) p = fmaf(sbyte_f32(ws[i >> 2], i & 3), x[i], p);
    } else {
        const uint32_t lo[2] = {((w.q.x << 4) & 0xF0F0F0F0u) ^ 0x80808080u, ((w.q.y << 4) & 0xF0F0F0F0u) ^ 0x80808080u};
        const uint32_t hi[2] = {(w.q.x & 0xF0F0F0F0u) ^ 0x80808080u, (w.q.y & 0xF0F0F0F0u) ^ 0x80808080u};
#pragma unroll
        for (int i = 0; i < 8; i++) p = fmaf(sbyte_f32(lo[i >> 2], i & 3), x[i], p);
#pragma unroll
        for (int i = 0; i < 8; i++) p = fmaf(sbyte_f32(hi[i >> 2], i & 3), x[8 + i], p);
    }
    return p;
}

// The unit's 16 signed codes as f32 (the factors unit_partial multiplies x by), for reuse across
// several X rows.
template <int FMT>
__device__ __forceinline__ void unit_codes(const Unit<FMT>& w, float (&c)[16]) {
    if constexpr (q8_layout<FMT>) {
        const uint32_t ws[4] = {w.q.x, w.q.y, w.q.z, w.q.w};
#pragma unroll
        for (int i = 0; i < 16; i++) c[i] = sbyte_f32(ws[i >> 2], i & 3);
    } else {
        const uint32_t lo[2] = {((w.q.x << 4) & 0xF0F0F0F0u) ^ 0x80808080u, ((w.q.y << 4) & 0xF0F0F0F0u) ^ 0x80808080u};
        const uint32_t hi[2] = {(w.q.x & 0xF0F0F0F0u) ^ 0x80808080u, (w.q.y & 0xF0F0F0F0u) ^ 0x80808080u};
#pragma unroll
        for (int i = 0; i < 8; i++) c[i] = sbyte_f32(lo[i >> 2], i & 3);
#pragma unroll
        for (int i = 0; i < 8; i++) c[8 + i] = sbyte_f32(hi[i >> 2], i & 3);
    }
}

// Contribution of one unit: the block scale (and offset) applied to the f32 partial; sx (the sum
// of the unit's x values) is used by Q4A only.
template <int FMT>
__device__ __forceinline__ float unit_value(const Unit<FMT>& w, float p, float sx) {
    if constexpr (FMT == FMT_Q8)
        return w.d * p;
    else if constexpr (FMT == FMT_Q8A || FMT == FMT_Q8A16)
        return fmaf(w.d, p, w.m * sx);
    else if constexpr (FMT == FMT_Q4)
        return (0.0625f * w.d) * p;
    else
        return fmaf(0.0625f * w.d, p, w.m * sx);
}

// RW weight rows starting at nrow0; NT X rows (xrow[t], -1 = zero row) -> Y rows yrow0 + t.
// TH threads per workgroup stage each X chunk together.  SOV > 0 sets the chunk to SOV 1024-value
// steps.  DMA (f32 X only): X goes from memory straight into LDS (buffer_load ... lds, 16 bytes per
// lane, lanes past the chunk masked off, rows outside X read as zero), which holds no registers.
template <int FMT, int XT, int RW, int NT, int TH, int SOV = 0, bool DMA = false>
__device__ __forceinline__ void gemv_rows(const GemmParams& p, const void* codes, const void* scales,
                                          const uint16_t* offs, int nrow0, int yrow0, const int* xrow, float* xs) {
    static_assert(!DMA || XT == XT_F32, "direct staging copies f32 rows");
    constexpr int S = SOV > 0 ? SOV : GemvChunk<NT>::steps;
    constexpr int KC = 1024 * S;
    constexpr int G = (16 / RW) < S ? (16 / RW) : S;                     // steps whose loads are in flight together
    constexpr int XV = (XT == XT_F32) ? 4 : 8;                          // X values per 16-byte load
    constexpr int XL = (KC / XV + TH - 1) / TH;  // X loads per thread per X row and chunk
    const int lane = threadIdx.x & 63;
    const int K = p.K, units = K >> 4;
    const int KS = min(K, KC);  // LDS row stride of the staged X chunk
    int rows[RW];
#pragma unroll
    for (int r = 0; r < RW; r++) rows[r] = min(nrow0 + r, p.N - 1);
    float acc[RW][NT];
#pragma unroll
    for (int r = 0; r < RW; r++)
#pragma unroll
        for (int t = 0; t < NT; t++) acc[r][t] = 0.f;

    for (int k0 = 0; k0 < K; k0 += KC) {
        const int kn = min(KC, K - k0);
        const int u0 = k0 >> 4;
        const int nsteps = (kn + 1023) >> 10;
        // 1. X loads of the chunk, 16 bytes each: load (t, i) covers values [e, e + XV) of X row t of
        //    the chunk with e = XV * (tid + i * threads).
        if constexpr (DMA) {
            // the whole X matrix as one buffer (its size fits 31 bits: checked by the launcher)
            const __amdgpu_buffer_rsrc_t xr =
                __builtin_amdgcn_make_buffer_rsrc((void*)p.X, 0, p.x_rows * K * 4, 0x00020000);
            const int wave = threadIdx.x >> 6;
#pragma unroll
            for (int t = 0; t < NT; t++)
#pragma unroll
                for (int i = 0; i < XL; i++) {
                    const int e = XV * (int)(threadIdx.x + i * TH);
                    const int off = xrow[t] >= 0 ? (xrow[t] * K + k0 + e) * 4 : 0x7FFFFFF0;
                    if (e < kn) buffer_copy16_lds(xr, xs + t * KS + XV * (64 * wave + i * TH), off);
                }
        }
        uint4 xl[DMA ? 1 : NT][DMA ? 1 : XL];
#pragma unroll
        for (int t = 0; t < (DMA ? 0 : NT); t++)
#pragma unroll
            for (int i = 0; i < XL; i++) {
                const int e = XV * (int)(threadIdx.x + i * TH);
                xl[t][i] = make_uint4(0, 0, 0, 0);
                if (e < kn && xrow[t] >= 0) {
                    if constexpr (XT == XT_F32)
                        xl[t][i] = *(const uint4*)((const float*)p.X + (size_t)xrow[t] * K + k0 + e);
                    else
                        xl[t][i] = *(const uint4*)((const uint16_t*)p.X + (size_t)xrow[t] * K + k0 + e);
                }
            }
        for (int g0 = 0; g0 < nsteps; g0 += G) {
            // 2. the weight loads of G steps
            Unit<FMT> w[G][RW];
#pragma unroll
            for (int j = 0; j < G; j++) {
                const int u = min(u0 + 64 * (g0 + j) + lane, units - 1);
#pragma unroll
                for (int r = 0; r < RW; r++) w[j][r] = load_unit<FMT>(codes, scales, offs, p.group, K, rows[r], u);
            }
            if (g0 == 0) {
                // 3. X to LDS as f32: X row t of the chunk at xs[t * KS + e]
#pragma unroll
                for (int t = 0; t < (DMA ? 0 : NT); t++)
#pragma unroll
                    for (int i = 0; i < XL; i++) {
                        const int e = XV * (int)(threadIdx.x + i * TH);
                        if (e < kn) {
                            float4* d = (float4*)(xs + t * KS + e);
                            const uint4 q4 = xl[t][i];
                            if constexpr (XT == XT_F32) {
                                d[0] = make_float4(__uint_as_float(q4.x), __uint_as_float(q4.y), __uint_as_float(q4.z),
                                                   __uint_as_float(q4.w));
                            } else {
                                const uint32_t q[4] = {q4.x, q4.y, q4.z, q4.w};
                                float v[8];
#pragma unroll
                                for (int h = 0; h < 4; h++) {
                                    if constexpr (XT == XT_F16) {
                                        v[2 * h] = f16_to_f32((uint16_t)(q[h] & 0xFFFFu));
                                        v[2 * h + 1] = f16_to_f32((uint16_t)(q[h] >> 16));
                                    } else {
                                        v[2 * h] = __uint_as_float(q[h] << 16);
                                        v[2 * h + 1] = __uint_as_float(q[h] & 0xFFFF0000u);
                                    }
                                }
                                d[0] = make_float4(v[0], v[1], v[2], v[3]);
                                d[1] = make_float4(v[4], v[5], v[6], v[7]);
                            }
                        }
                    }
                __syncthreads();
            }
            // 4. arithmetic of the G steps
#pragma unroll
            for (int j = 0; j < G; j++) {
                const int u = u0 + 64 * (g0 + j) + lane;
                if (g0 + j < nsteps && u < units) {
                    int e0, e1;
                    unit_runs<FMT>(u, e0, e1);
                    e0 -= k0;
                    e1 -= k0;
                    // each row's codes are converted once and serve all NT X rows
                    float cv[RW][16];
#pragma unroll
                    for (int r = 0; r < RW; r++) unit_codes<FMT>(w[j][r], cv[r]);
#pragma unroll
                    for (int t = 0; t < NT; t++) {
                        float x[16];
                        const float4* a = (const float4*)(xs + t * KS + e0);
                        const float4* b = (const float4*)(xs + t * KS + e1);
                        const float4 a0 = a[0], a1 = a[1], b0 = b[0], b1 = b[1];
                        x[0] = a0.x; x[1] = a0.y; x[2] = a0.z; x[3] = a0.w;
                        x[4] = a1.x; x[5] = a1.y; x[6] = a1.z; x[7] = a1.w;
                        x[8] = b0.x; x[9] = b0.y; x[10] = b0.z; x[11] = b0.w;
                        x[12] = b1.x; x[13] = b1.y; x[14] = b1.z; x[15] = b1.w;
                        float sx = 0.f;
                        if constexpr (has_offs<FMT>) {
#pragma unroll
                            for (int i = 0; i < 16; i++) sx += x[i];
                        }
#pragma unroll
                        for (int r = 0; r < RW; r++) {
                            float pr = 0.f;
#pragma unroll
                            for (int i = 0; i < 16; i++) pr = fmaf(cv[r][i], x[i], pr);
                            acc[r][t] += unit_value<FMT>(w[j][r], pr, sx);
                        }
                    }
                }
            }
        }
        __syncthreads();  // the next chunk (or the next rows' chunk) overwrites xs
    }

#pragma unroll
    for (int r = 0; r < RW; r++)
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const float v = wave_sum(acc[r][t]);
            const int n = nrow0 + r;
            if (lane == ((r * NT + t) & 63) && n < p.N) {
                const float sc = p.rs ? p.rs[yrow0 + t] : 1.f;
                p.Y[(size_t)(yrow0 + t) * p.N + n] = v * sc;
            }
        }
}

template <int FMT, int XT, int RW, int NT, int TH, int SOV = 0, bool DMA = false>
__device__ __forceinline__ void gemv_chunk(const GemmParams& p, const void* codes, const void* scales,
                                           const uint16_t* offs, int nrow0, int c, float* xs) {
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
    gemv_rows<FMT, XT, RW, NT, TH, SOV, DMA>(p, codes, scales, offs, nrow0, c, xrow, xs);
}

// Grouped launches: the NT (1..NTG) X rows of one chunk of an expert's segment, in K chunks of
// 2048 values; with DMA, f32 X is staged straight into LDS.
constexpr int kGroupedSteps = 2;
template <int FMT, int XT, int RW, int TH, int NTG, bool DMA>
__device__ __forceinline__ void gemv_grouped_chunk(const GemmParams& p, const void* codes, const void* scales,
                                                   const uint16_t* offs, int nrow0, int c, int nt, float* xs) {
    if constexpr (NTG > 1) {
        if (nt < NTG)
            return gemv_grouped_chunk<FMT, XT, RW, TH, NTG - 1, DMA>(p, codes, scales, offs, nrow0, c, nt, xs);
    }
    gemv_chunk<FMT, XT, RW, NTG, TH, kGroupedSteps, DMA>(p, codes, scales, offs, nrow0, c, xs);
}

// NTD > 0: dense call with NTD = T rows of X (T <= 8).  NTD == 0: grouped call; blockIdx.y is the
// expert and the workgroup walks the expert's rows in chunks of at most NTG.  TH threads per
// workgroup, each wavefront owning RW weight rows.
template <int FMT, int XT, int RW, int NTD, int TH, int NTG = 8, bool DMA = false>
__global__ __launch_bounds__(TH) __attribute__((amdgpu_waves_per_eu(DMA ? 3 : 1))) void gemv_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(16))) float xs[];  // gemv_lds_bytes()
    const int wave = threadIdx.x >> 6;
    const int nrow0 = (blockIdx.x * (TH / 64) + wave) * RW;
    // Every wavefront stays to the end (the X chunks are staged by the whole workgroup); rows
    // beyond N are clamped on load and never stored.
    if constexpr (NTD > 0) {
        gemv_chunk<FMT, XT, RW, NTD, TH, 0, DMA>(p, p.codes, p.scales, p.offs, nrow0, 0, xs);
    } else {
        const int e = blockIdx.y;
        const int r0 = min(max(p.seg_off[e], 0), p.R);
        const int r1 = min(max(p.seg_off[e + 1], r0), p.R);
        const void* codes = p.experts[e].codes;
        const void* scales = p.experts[e].scales;
        const uint16_t* offs = p.experts[e].offsets;
        for (int c = r0; c < r1; c += NTG)
            gemv_grouped_chunk<FMT, XT, RW, TH, NTG, DMA>(p, codes, scales, offs, nrow0, c, min(NTG, r1 - c), xs);
    }
}

// ---- single X row: K split over the workgroup --------------------------------------------------
// Lane c of the workgroup owns chunk c of every weight row: its 16 code bytes (Q8: 16 values, half a
// block; Q4 / Q4A: 32 values, one block), so every load instruction of a wavefront is one contiguous
// 1 KiB run of a row, and the chunk's X values stay in registers for the whole launch.  A workgroup
// of W = ceil(chunks / 64) wavefronts takes R consecutive weight rows: it issues the loads of all R
// rows, then per row forms the chunk's f32 partial (block scale on the partial, Q4A offset times the
// chunk's X sum), sums each 16-lane row by DPP, and after one barrier R threads add the W * 4 row
// sums and store Y.
//
// Measured on MI355X, Q8 N = K = 4096, f32 X, 16 rotating weight copies, standalone kernels in one
// process (the figures of one run): this shape with R = 8 5.03-5.07 us per launch; R = 4 5.19-5.32;
// R = 16 (one workgroup per CU) 5.8; the previous kernel (one row per wavefront, X staged in LDS per
// workgroup, 1024 workgroups) 5.43-5.70 through the C ABI.  What the rest is: an empty launch costs
// 1.58 us on the GPU; a kernel issuing the same loads and only folding the bytes takes 4.16-4.19 us;
// the row sums, barrier and Y store add 0.35 us to it (0.25 of that is the store: a kernel that
// leaves output in the L2 caches pays their write-back at its end, whatever the store's scope); the
// decode (16 conversions and 16 FMAs per lane and row) overlaps the loads only in part, because a
// wavefront consumes its loads in issue order.  Tried and slower: each lane owning 2 or 4
// consecutive chunks (a load then covers 2 or 4 KiB with gaps: 5.5-12 us), every load pinned ahead
// of all arithmetic (5.3-5.6), X loaded after the weights (5.6-5.9), per-lane partials summed from
// LDS instead of DPP row sums (5.26), nontemporal Y stores (5.23).
constexpr int kStreamKMax = 16384;  // K limit of the K-split kernels for Q8 (16 wavefronts of 1024 values)

template <int FMT>
struct G1Chunk {
    static constexpr int values = q8_layout<FMT> ? 16 : 32;  // X values per lane chunk (16 code bytes)
};


// BATCH: p.N is the total row count of the jobs in bj; row g belongs to the job j with
// start[j] <= g < start[j+1] (a scan over at most 8 wave-uniform entries).
template <int FMT, int XT, int R, bool BATCH, bool RS>
__global__ __launch_bounds__(1024) void gemv1_split_kernel(GemmParams p, BatchJobs bj) {
    constexpr int V = G1Chunk<FMT>::values;
    __shared__ float part[R * 16 * 4];  // [row][wavefront][4 row sums]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int K = p.K, N = p.N, chunks = K / V;
    const int W = (chunks + 63) >> 6;  // the launch's wavefront count (blockDim.x would be read late)
    const int c = 64 * wave + lane;
    const bool on = c < chunks;
    const int cc = min(c, chunks - 1);
    const int n0 = (int)blockIdx.x * R;
    // What the epilogue needs from the arguments is read here and pinned in scalar registers: the
    // compiler treats argument loads as free to repeat and otherwise reloads them after the barrier,
    // a memory round trip at the end of every workgroup (0.3-0.5 us per launch measured).
    QG_GLOBAL float* Yout = gptr_mut<float>(p.Y);
    int Nout = N;
    asm volatile("" : "+s"(Yout), "+s"(Nout));
    float sc = 1.f;
    if constexpr (RS) sc = p.rs ? p.rs[0] : 1.f;
    __builtin_amdgcn_sched_barrier(0);

    // This lane's X values: Q8 elements 16cc..16cc+15; Q4 / Q4A elements 32cc..32cc+31 (x[0..15]
    // pair with the low nibbles, x[16..31] with the high ones).  Zero for a lane past K.
    float x[V];
    {
        const size_t e0 = (size_t)cc * V;
        if constexpr (XT == XT_F32) {
#pragma unroll
            for (int i = 0; i < V / 4; i++) {
                const float4 a = *(const float4*)((const float*)p.X + e0 + 4 * i);
                x[4 * i] = a.x;
                x[4 * i + 1] = a.y;
                x[4 * i + 2] = a.z;
                x[4 * i + 3] = a.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < V / 8; i++) {
                const uint4 q = *(const uint4*)((const uint16_t*)p.X + e0 + 8 * i);
                const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                for (int h = 0; h < 8; h++) {
                    const uint16_t hv = (uint16_t)(w4[h >> 1] >> (16 * (h & 1)));
                    x[8 * i + h] = (XT == XT_F16) ? f16_to_f32(hv) : bf16_to_f32(hv);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < V; i++) x[i] = on ? x[i] : 0.f;
    }
    float sx = 0.f;
    if constexpr (has_offs<FMT>) {
#pragma unroll
        for (int i = 0; i < V; i++) sx += x[i];
    }

    auto job_of = [&](int g) {
        int j = 0;
        if constexpr (BATCH) {
#pragma unroll
            for (int i = 1; i < kMaxBatchJobs; i++)
                if (i < bj.J && g >= bj.start[i]) j = i;
        }
        return j;
    };
    // Row bases of codes, scales (and offsets) for every row, as wavefront-uniform pointers pinned in
    // scalar registers before any load: each load is then base + the lane's 32-bit offset, with no
    // per-lane 64-bit address arithmetic (left to itself the compiler computes half of them per
    // lane in vector registers; 0.2-0.3 us per launch measured).
    const QG_GLOBAL char* crow[R];
    const QG_GLOBAL char* srow[R];
    const QG_GLOBAL char* orow[R];
#pragma unroll
    for (int r = 0; r < R; r++) {
        int n = min(n0 + r, N - 1);
        const void* codes = p.codes;
        const void* scales = p.scales;
        const uint16_t* offs = p.offs;
        if constexpr (BATCH) {
            const int j = job_of(n);
            codes = bj.codes[j];
            scales = bj.scales[j];
            offs = bj.offs[j];
            n -= bj.start[j];
        }
        crow[r] = uniform_ptr(codes, (uint64_t)n * (uint64_t)(q8_layout<FMT> ? K : K >> 1));
        srow[r] = uniform_ptr(scales, (uint64_t)n * (uint64_t)((K >> (blk16<FMT> ? 4 : 5)) * (q8_layout<FMT> ? 4 : 2)));
        asm volatile("" : "+s"(crow[r]), "+s"(srow[r]));
        if constexpr (has_offs<FMT>) {
            // Q4A: bf16 per group; Q8A / Q8A16: f32 per block, laid out as the scales (Q8A16 offsets
            // may be absent: row 0's base is then never read)
            orow[r] = uniform_ptr(offs, (uint64_t)(blk16<FMT> && !offs ? 0 : n) *
                                            (uint64_t)(FMT == FMT_Q4A ? (K / p.group) * 2 : (K >> (blk16<FMT> ? 4 : 5)) * 4));
            asm volatile("" : "+s"(orow[r]));
        }
    }
    const uint32_t oc = (uint32_t)(cc * 16);
    const uint32_t os = blk16<FMT> ? (uint32_t)(cc * 4) : q8_layout<FMT> ? (uint32_t)((cc >> 1) * 4) : (uint32_t)(cc * 2);
    const uint32_t oo = FMT == FMT_Q4A ? (uint32_t)(((cc * 32) / p.group) * 2) : has_offs<FMT> ? os : 0u;
    u32x4_t q[R];
    float d[R], m[R];
    const bool hm = !blk16<FMT> || p.offs != nullptr;  // Q8A16 without offsets: none read
    auto issue = [&](int r) __attribute__((always_inline)) {
        q[r] = __builtin_nontemporal_load((const QG_GLOBAL u32x4_t*)(crow[r] + oc));
        if constexpr (q8_layout<FMT>) {
            d[r] = *(const QG_GLOBAL float*)(srow[r] + os);
            if constexpr (blk16<FMT>) m[r] = hm ? *(const QG_GLOBAL float*)(orow[r] + oo) : -0.0f;
            else m[r] = has_offs<FMT> ? *(const QG_GLOBAL float*)(orow[r] + oo) : 0.f;
        } else {
            d[r] = 0.0625f * f16_to_f32(*(const QG_GLOBAL uint16_t*)(srow[r] + os));
            m[r] = FMT == FMT_Q4A ? bf16_to_f32(*(const QG_GLOBAL uint16_t*)(orow[r] + oo)) : 0.f;
        }
    };
    auto row = [&](int r) __attribute__((always_inline)) {
        const uint32_t w4[4] = {q[r].x, q[r].y, q[r].z, q[r].w};
        float pr = 0.f;
        if constexpr (q8_layout<FMT>) {
#pragma unroll
            for (int i = 0; i < 16; i++) pr = fmaf(sbyte_f32(w4[i >> 2], i & 3), x[i], pr);
        } else {
            // signed bytes 16 (nibble - 8): the nibble moved to the byte's high half, top bit flipped
#pragma unroll
            for (int i = 0; i < 16; i++) pr = fmaf(sbyte_f32(((w4[i >> 2] << 4) & 0xF0F0F0F0u) ^ 0x80808080u, i & 3), x[i], pr);
#pragma unroll
            for (int i = 0; i < 16; i++) pr = fmaf(sbyte_f32((w4[i >> 2] & 0xF0F0F0F0u) ^ 0x80808080u, i & 3), x[16 + i], pr);
        }
        const float v = row16_sum_dpp(has_offs<FMT> ? fmaf(d[r], pr, m[r] * sx) : d[r] * pr);
        if ((lane & 15) == 15) part[(r * 16 + wave) * 4 + (lane >> 4)] = v;
    };
    // Issue order (pinned by scheduling barriers): X (above), rows [0, A), the arithmetic of row 0,
    // rows [A, R), the arithmetic of the rest.  Measured (Q8 4096 x 4096, R = 8): A = 3 or 4 5.03
    // us, A = 2 5.13, A = 1 5.24, the rest issued before row 0's arithmetic 5.23, and the order the
    // compiler picks by itself 5.05-5.45 depending on the surrounding code.  R = 4 (Q4 4096 x 4096,
    // two wavefronts a row): all four rows first, 5.15-5.23 us against 5.61-5.64 with A = 1.
    constexpr int A = R >= 8 ? 4 : R;
#pragma unroll
    for (int r = 0; r < A; r++) issue(r);
    __builtin_amdgcn_sched_barrier(0);
    row(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = A; r < R; r++) issue(r);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 1; r < R; r++) row(r);
    __syncthreads();
    // Row r's W * 4 partials: thread 16 r + w adds wavefront w's four, then a 16-lane DPP sum
    // (R * 16 <= 64 W threads: R = 8 runs with W >= 4, R = 4 with W >= 1).
    if ((int)threadIdx.x < R * 16) {
        const int r = (int)threadIdx.x >> 4, w = (int)threadIdx.x & 15;
        float sum = 0.f;
        if (w < W) {
            const float4 a = *(const float4*)(part + ((int)threadIdx.x) * 4);
            sum = (a.x + a.y) + (a.z + a.w);
        }
        sum = row16_sum_dpp(sum);
        const int g = n0 + r;
        if (w == 15 && g < Nout) {
            if constexpr (BATCH) {
                const int j = job_of(g);
                bj.Y[j][g - bj.start[j]] = sum * sc;
            } else {
                Yout[g] = sum * sc;
            }
        }
    }
}

// CU count of the current device (cached).
static int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cus[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
        cus[dev] = v;
    }
    return cus[dev];
}

// Single X row: W = ceil(chunks / 64) <= 16 wavefronts (Q8 K <= 16384, Q4 K <= 32768); R = 8 rows per
// workgroup when W >= 4, else 4 (more workgroups for narrow ones).  False (nothing launched) when K
// is past the limit.
template <int FMT, int XT>
static bool gemv1(const GemmParams& p, hipStream_t s, const BatchJobs* bj = nullptr) {
    const int chunks = p.K / G1Chunk<FMT>::values;
    const int W = (chunks + 63) / 64;
    if (W > 16) return false;
    const BatchJobs none{};
    const BatchJobs& b = bj ? *bj : none;
    // variants: rows per workgroup, batched jobs, a row scale (read only when given)
    auto go = [&](auto kern, int rows) { hipLaunchKernelGGL(kern, dim3((p.N + rows - 1) / rows), dim3(64 * W), 0, s, p, b); };
    if (W >= 4) {
        if (bj) go(gemv1_split_kernel<FMT, XT, 8, true, false>, 8);
        else if (p.rs) go(gemv1_split_kernel<FMT, XT, 8, false, true>, 8);
        else go(gemv1_split_kernel<FMT, XT, 8, false, false>, 8);
    } else {
        if (bj) go(gemv1_split_kernel<FMT, XT, 4, true, false>, 4);
        else if (p.rs) go(gemv1_split_kernel<FMT, XT, 4, false, true>, 4);
        else go(gemv1_split_kernel<FMT, XT, 4, false, false>, 4);
    }
    return true;
}

// T = 2..8 rows of X, K <= 16384 (8192 for T > 4): K is split over the workgroup's wavefronts, 64 units (1024
// values) each, so that a lane owns one unit of every weight row and keeps that unit's 16 X values
// of every X row in registers for the whole launch; no X is read from LDS.  Each wavefront takes
// batches of KS_RB weight rows (the next batch's loads issued before the current one is
// computed), reduces each (row, X row) partial within its four 16-lane rows, and the workgroup adds
// those four sums of each wavefront through LDS after one barrier per batch.  Every workgroup reads
// its wavefronts' X slices (T * K values) once, so X traffic falls as workgroups take more batches:
// 16 resident wavefronts per CU for T <= 3, 8 for T = 4.  Measured on the Q8 decode shape (N = K =
// 4096, f32 X, 16 rotating weight copies), against the chunked LDS kernel on the same box: T = 2
// 6.98 us against 7.32, T = 3 8.18 against 9.07, T = 4 10.31 against 10.8 (16 wavefronts per CU at
// T = 4: 10.62).  Full-wavefront xor-shuffle sums instead of the row sums: T = 4 13.9 us.  T > 4
// (152..200 VGPRs, two or three wavefronts per SIMD): T = 5 10.97 us against 12.88, T = 6 11.64
// against 14.61, T = 8 14.05 against 17.94.
constexpr int kSplitRows = 4;  // weight rows per batch

// One pass of the scheme above: NT X rows xrow[t] (-1 = a zero row) against the weight-row batches
// b, b + stride, ... < ceil(N / kSplitRows) of one matrix, into Y rows yrow0 + t.  part: LDS of
// 2 * 16 * kSplitRows * NTS * 4 floats, 16-byte aligned, with a per-wavefront slot of
// kSplitRows * NTS * 4 floats whatever NT is (NT <= NTS): passes of different NT that follow each
// other (the grouped kernel's chunks) then keep the two parities' slots disjoint, so the
// double buffer needs one barrier per batch only.  par: the parity of the workgroup's next batch.
// Every wavefront of the workgroup calls it with the same arguments.
template <int FMT, int XT, int NT, int NTS = NT>
__device__ __forceinline__ void ksplit_pass(const GemmParams& p, const void* codes, const void* scales,
                                            const uint16_t* offs, const int (&xrow)[NT], int yrow0, int b, int stride,
                                            float* part, int& par) {
    static_assert(NT <= NTS, "a pass's partials fit the per-wavefront slot");
    constexpr int RB = kSplitRows;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, W = (int)blockDim.x >> 6;
    const int K = p.K, units = K >> 4, N = p.N;
    const int nb = (N + RB - 1) / RB;
    const int u = 64 * wave + lane;
    const bool on = u < units;
    const int uc = min(u, units - 1);

    // This lane's unit of every X row (zero for a lane past K or a zero row, so its partials are zero).
    float x[NT][16], sx[NT];
    {
        int e0, e1;
        unit_runs<FMT>(uc, e0, e1);
#pragma unroll
        for (int t = 0; t < NT; t++) {
            // a zero row loads X row 0 (the launchers guarantee X holds a row) and discards it: no
            // branch around the loads
            const bool use = on && xrow[t] >= 0;
            const size_t base = (size_t)max(xrow[t], 0) * K;
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const size_t e = base + (h ? e1 : e0);
                if constexpr (XT == XT_F32) {
                    const float4 a = *(const float4*)((const float*)p.X + e);
                    const float4 c = *(const float4*)((const float*)p.X + e + 4);
                    const float v[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
                    for (int i = 0; i < 8; i++) x[t][8 * h + i] = use ? v[i] : 0.f;
                } else {
                    const uint4 q = *(const uint4*)((const uint16_t*)p.X + e);
                    const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                    for (int i = 0; i < 8; i++) {
                        const uint16_t hv = (uint16_t)(w4[i >> 1] >> (16 * (i & 1)));
                        const float v = (XT == XT_F16) ? f16_to_f32(hv) : bf16_to_f32(hv);
                        x[t][8 * h + i] = use ? v : 0.f;
                    }
                }
            }
            sx[t] = 0.f;
            if constexpr (has_offs<FMT>) {
#pragma unroll
                for (int i = 0; i < 16; i++) sx[t] += x[t][i];
            }
        }
    }
    float sc[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) sc[t] = p.rs ? p.rs[yrow0 + t] : 1.f;
    auto load_batch = [&](int bb, Unit<FMT> (&w)[RB]) {
#pragma unroll
        for (int r = 0; r < RB; r++) w[r] = load_unit<FMT>(codes, scales, offs, p.group, K, min(bb * RB + r, N - 1), uc);
    };
    Unit<FMT> wa[RB], wb[RB];
    load_batch(b, wa);

    auto step = [&](const Unit<FMT> (&cu)[RB], Unit<FMT> (&nx)[RB]) __attribute__((always_inline)) {
        const int b2 = b + stride;
        const bool more = b2 < nb;
        if (more) load_batch(b2, nx);
        float* pw = part + (size_t)(par * 16 + wave) * (RB * NTS * 4);
#pragma unroll
        for (int r = 0; r < RB; r++) {
            float c[16];
            unit_codes<FMT>(cu[r], c);
#pragma unroll
            for (int t = 0; t < NT; t++) {
                float pr = 0.f;
#pragma unroll
                for (int i = 0; i < 16; i++) pr = fmaf(c[i], x[t][i], pr);
                const float v = row16_sum_dpp(unit_value<FMT>(cu[r], pr, sx[t]));
                if ((lane & 15) == 15) pw[(r * NT + t) * 4 + (lane >> 4)] = v;
            }
        }
        __syncthreads();
        if ((int)threadIdx.x < RB * NT) {
            const int r = (int)threadIdx.x / NT, t = (int)threadIdx.x % NT, row = b * RB + r;
            if (row < N) {
                float s = 0.f;
                for (int w = 0; w < W; w++) {
                    const float4 q = *(const float4*)(part + ((size_t)(par * 16 + w) * (RB * NTS) + threadIdx.x) * 4);
                    s += (q.x + q.y) + (q.z + q.w);
                }
                p.Y[(size_t)(yrow0 + t) * N + row] = s * sc[t];
            }
        }
        par ^= 1;
        b = b2;
        return more;
    };
    while (step(wa, wb) && step(wb, wa)) {
    }
}

template <int FMT, int XT, int NT>
__global__ __launch_bounds__(NT <= 4 ? 1024 : 512) void gemv_ksplit_kernel(GemmParams p) {
    __shared__ __attribute__((aligned(16))) float part[2 * 16 * kSplitRows * NT * 4];
    if ((int)blockIdx.x * kSplitRows >= p.N) return;  // uniform over the workgroup
    int xrow[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) xrow[t] = t;
    int par = 0;
    ksplit_pass<FMT, XT, NT>(p, p.codes, p.scales, p.offs, xrow, 0, (int)blockIdx.x, (int)gridDim.x, part, par);
}

// Several matrices sharing the NT X rows (qgemm_batch, T = 2..8): blockIdx.y is the job, whose rows
// the workgroups of that column take in batches with stride gridDim.x, as the dense launch does.
template <int FMT, int XT, int NT>
__global__ __launch_bounds__(NT <= 4 ? 1024 : 512) void gemv_ksplit_batch_kernel(GemmParams p, BatchJobs bj) {
    __shared__ __attribute__((aligned(16))) float part[2 * 16 * kSplitRows * NT * 4];
    const int j = blockIdx.y;
    if (j >= bj.J) return;  // uniform over the workgroup
    GemmParams q = p;
    q.codes = bj.codes[j];
    q.scales = bj.scales[j];
    q.offs = bj.offs[j];
    q.Y = bj.Y[j];
    q.N = bj.start[j + 1] - bj.start[j];
    if ((int)blockIdx.x * kSplitRows >= q.N) return;  // uniform over the workgroup
    int xrow[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) xrow[t] = t;
    int par = 0;
    ksplit_pass<FMT, XT, NT>(q, q.codes, q.scales, q.offs, xrow, 0, (int)blockIdx.x, (int)gridDim.x, part, par);
}

// Grouped launches (exact-mode MoE): blockIdx.y is the expert; the workgroup walks the expert's row
// segment in chunks of at most 4 X rows (gathered through row_src when given; ids outside X read as
// zero rows), each chunk one pass over its share of the expert's weight-row batches.
template <int FMT, int XT, int NTC>
__device__ __forceinline__ void ksplit_grouped_chunk(const GemmParams& p, const void* codes, const void* scales,
                                                     const uint16_t* offs, int c, float* part, int& par) {
    int xrow[NTC];
#pragma unroll
    for (int t = 0; t < NTC; t++) {
        int s = c + t;
        if (p.row_src) {
            s = p.row_src[c + t];
            if (s < 0 || s >= p.x_rows) s = -1;
        }
        xrow[t] = s;
    }
    ksplit_pass<FMT, XT, NTC, 4>(p, codes, scales, offs, xrow, c, (int)blockIdx.x, (int)gridDim.x, part, par);
}

template <int FMT, int XT>
__global__ __launch_bounds__(512) void gemv_ksplit_grouped_kernel(GemmParams p) {
    __shared__ __attribute__((aligned(16))) float part[2 * 16 * kSplitRows * 4 * 4];
    const int e = blockIdx.y;
    const int r0 = min(max(p.seg_off[e], 0), p.R);
    const int r1 = min(max(p.seg_off[e + 1], r0), p.R);
    if (r1 <= r0 || (int)blockIdx.x * kSplitRows >= p.N) return;  // uniform over the workgroup
    const void* codes = p.experts[e].codes;
    const void* scales = p.experts[e].scales;
    const uint16_t* offs = p.experts[e].offsets;
    int par = 0;
    for (int c = r0; c < r1; c += 4) {
        const int nt = min(4, r1 - c);
        if (nt == 1) ksplit_grouped_chunk<FMT, XT, 1>(p, codes, scales, offs, c, part, par);
        else if (nt == 2) ksplit_grouped_chunk<FMT, XT, 2>(p, codes, scales, offs, c, part, par);
        else if (nt == 3) ksplit_grouped_chunk<FMT, XT, 3>(p, codes, scales, offs, c, part, par);
        else ksplit_grouped_chunk<FMT, XT, 4>(p, codes, scales, offs, c, part, par);
    }
}

template <int FMT, int XT, int NT>
static bool gemv_ksplit(const GemmParams& p, hipStream_t s) {
    // T > 4: X takes 16 T registers per lane, so workgroups of at most 8 wavefronts (K <= 8192)
    if (p.R != NT || p.row_src || p.K > (NT <= 4 ? kStreamKMax : kStreamKMax / 2)) return false;
    const int W = (p.K / 16 + 63) / 64;  // 1..16 wavefronts
    const int nb = (p.N + kSplitRows - 1) / kSplitRows;
    const int per_cu = std::max(1, (NT >= 4 ? 8 : 16) / W);
    const int grid = std::max(1, std::min(nb, device_cus() * per_cu));
    hipLaunchKernelGGL((gemv_ksplit_kernel<FMT, XT, NT>), dim3(grid), dim3(64 * W), 0, s, p);
    return true;
}

// LDS bytes for the X chunks: the largest NT * min(K, chunk(NT)) over the row counts NT a chunk of
// output rows can have (dense: T; grouped: 1..8).
template <int NT>
static size_t chunk_floats(int K) {
    return (size_t)NT * (size_t)std::min(K, GemvChunk<NT>::kc);
}
static size_t gemv_lds_bytes(int K, int nt_lo, int nt_hi) {
    const size_t f[8] = {chunk_floats<1>(K), chunk_floats<2>(K), chunk_floats<3>(K), chunk_floats<4>(K),
                         chunk_floats<5>(K), chunk_floats<6>(K), chunk_floats<7>(K), chunk_floats<8>(K)};
    size_t m = 0;
    for (int i = nt_lo - 1; i < nt_hi; i++) m = std::max(m, f[i]);
    return 4 * m;
}

// Rows per workgroup: a single X row uses 8 wavefronts of 2 weight rows (one X copy in LDS serves
// 16 rows, and each X value read from LDS serves 2); more X rows use 4 wavefronts of 2 or 4 rows,
// so that the X staged per workgroup stays small next to the weights it serves.
template <int FMT, int XT, int NT, int RWX, int THX>
static void gemv_dense_dma(const GemmParams& p, hipStream_t s) {
    constexpr int ROWS = RWX * THX / 64;
    dim3 grid((p.N + ROWS - 1) / ROWS);
    hipLaunchKernelGGL((gemv_kernel<FMT, XT, RWX, NT, THX, 8, true>), grid, dim3(THX), gemv_lds_bytes(p.K, NT, NT), s, p);
}

template <int FMT, int XT, int NT>
static void gemv_dense(const GemmParams& p, hipStream_t s) {
    // 3..8 f32 X rows: X staged straight into LDS, 2 weight rows per wavefront (twice the
    // workgroups of 4 rows), three wavefronts per SIMD.  Measured on the Q8 decode shape (N = K =
    // 4096): T = 4 10.9 us against 12.6 (4 rows per wavefront through registers), T = 8 17.8
    // against 19.7; at T = 2 both run 7.3-7.5 us, and 1 row per wavefront is slower.
    if constexpr (NT >= 2) {
        if (gemv_ksplit<FMT, XT, NT>(p, s)) return;
    }
    if constexpr (XT == XT_F32 && NT > 2) {
        if ((size_t)p.x_rows * (size_t)p.K * 4 <= 0x7FFFFFF0u) return gemv_dense_dma<FMT, XT, NT, 2, 256>(p, s);
    }
    constexpr int RW = NT == 1 ? 2 : NT == 2 ? 2 : 4;
    constexpr int TH = NT == 1 ? kGemv1Threads : kGemvThreads;
    constexpr int ROWS = RW * TH / 64;
    dim3 grid((p.N + ROWS - 1) / ROWS);
    hipLaunchKernelGGL((gemv_kernel<FMT, XT, RW, NT, TH>), grid, dim3(TH), gemv_lds_bytes(p.K, NT, NT), s, p);
}

template <int FMT, int XT>
static void gemv_pick(const GemmParams& p, bool grouped, hipStream_t s) {
    if (grouped) {
        if (p.K <= kStreamKMax / 2 && p.x_rows >= 1) {
            // K split over at most 8 wavefronts, X rows of each segment chunk in registers; about four
            // resident rounds of workgroups if every expert has rows.  Its zero rows read X row 0, so
            // an X without rows goes to the chunked kernel, whose X loads are range-checked.  Exact MoE block (128 experts,
            // top 8, 32 tokens): 377 us at one round, 314 at two, 271 at four, 273 at eight, 292 at
            // sixteen; the chunked LDS kernel it replaces ran 345 us.  512-thread bounds (no spills,
            // two or three wavefronts per SIMD) against 1024 (128 VGPRs, 24-49 spilled): 309.5 against
            // 312.3 us at two rounds.
            const int W = (p.K / 16 + 63) / 64;
            const int nb = (p.N + kSplitRows - 1) / kSplitRows;
            const int per_cu = std::max(1, 16 / W);
            const int gx = std::max(1, std::min(nb, (4 * device_cus() * per_cu + p.E - 1) / p.E));
            hipLaunchKernelGGL((gemv_ksplit_grouped_kernel<FMT, XT>), dim3(gx, p.E), dim3(64 * W), 0, s, p);
            return;
        }
        // Chunks of at most 4 segment rows and 2048 values of K, LDS sized for them; segments longer
        // than 4 rows (a few percent of the routed experts) read their weights once per chunk.  f32
        // X is staged straight into LDS (no staging registers), which brings the kernel to 168
        // VGPRs and three wavefronts per SIMD (a 36-byte spill).  Measured on the exact MoE block
        // (128 experts, top 8, 32 tokens): 517 us with 8-row chunks through registers (two
        // wavefronts per SIMD); 487 us with 4-row chunks; 439 us adding the direct staging and
        // 2048-value chunks; 354 us at three wavefronts per SIMD; 760 us forced to four (spills).
        dim3 grid((p.N + 15) / 16, p.E);
        const size_t lds = 4 * 4 * (size_t)std::min(p.K, 1024 * kGroupedSteps);  // 4 rows of one K chunk
        if constexpr (XT == XT_F32) {
            // direct staging addresses X through one buffer range of 31 bits
            if ((size_t)p.x_rows * (size_t)p.K * 4 <= 0x7FFFFFF0u) {
                hipLaunchKernelGGL((gemv_kernel<FMT, XT, 4, 0, kGemvThreads, 4, true>), grid, dim3(kGemvThreads), lds,
                                   s, p);
                return;
            }
        }
        hipLaunchKernelGGL((gemv_kernel<FMT, XT, 4, 0, kGemvThreads, 4>), grid, dim3(kGemvThreads), lds, s, p);
        return;
    }
    switch (p.R) {
        case 1:
            if (gemv1<FMT, XT>(p, s)) return;
            return gemv_dense<FMT, XT, 1>(p, s);
        case 2: return gemv_dense<FMT, XT, 2>(p, s);
        case 3: return gemv_dense<FMT, XT, 3>(p, s);
        case 4: return gemv_dense<FMT, XT, 4>(p, s);
        case 5: return gemv_dense<FMT, XT, 5>(p, s);
        case 6: return gemv_dense<FMT, XT, 6>(p, s);
        case 7: return gemv_dense<FMT, XT, 7>(p, s);
        default: return gemv_dense<FMT, XT, 8>(p, s);
    }
}

template <int FMT>
static void gemv_xt(int xt, const GemmParams& p, bool grouped, hipStream_t s) {
    if (xt == XT_F32) gemv_pick<FMT, XT_F32>(p, grouped, s);
    else if (xt == XT_F16) gemv_pick<FMT, XT_F16>(p, grouped, s);
    else gemv_pick<FMT, XT_BF16>(p, grouped, s);
}

template <int FMT>
static bool gemv1_batch_xt(int xt, const GemmParams& p, const BatchJobs& bj, hipStream_t s) {
    if (xt == XT_F32) return gemv1<FMT, XT_F32>(p, s, &bj);
    if (xt == XT_F16) return gemv1<FMT, XT_F16>(p, s, &bj);
    return gemv1<FMT, XT_BF16>(p, s, &bj);
}

// T = 2..8 X rows, every job of bj in one launch: the K-split kernel with blockIdx.y the job and the
// column count sized like the dense launch's resident round, shared out in proportion to the largest
// job's rows (smaller jobs' extra workgroups exit at once).  False when K is past the kernel's limit.
template <int FMT, int XT, int NT>
static bool gemv_ksplit_batch(const GemmParams& p, const BatchJobs& bj, hipStream_t s) {
    if (p.K > (NT <= 4 ? kStreamKMax : kStreamKMax / 2)) return false;
    const int W = (p.K / 16 + 63) / 64;
    int nb_max = 1;
    long nb_tot = 0;
    for (int j = 0; j < bj.J; j++) {
        const int nb = (bj.start[j + 1] - bj.start[j] + kSplitRows - 1) / kSplitRows;
        nb_max = std::max(nb_max, nb);
        nb_tot += nb;
    }
    const int per_cu = std::max(1, (NT >= 4 ? 8 : 16) / W);
    const long round = (long)device_cus() * per_cu;
    const int gx = (int)std::max(1L, std::min((long)nb_max, (round * nb_max + nb_tot - 1) / std::max(1L, nb_tot)));
    hipLaunchKernelGGL((gemv_ksplit_batch_kernel<FMT, XT, NT>), dim3(gx, bj.J), dim3(64 * W), 0, s, p, bj);
    return true;
}

template <int FMT, int XT>
static bool gemv_batch_t(const GemmParams& p, const BatchJobs& bj, hipStream_t s) {
    switch (p.R) {
        case 2: return gemv_ksplit_batch<FMT, XT, 2>(p, bj, s);
        case 3: return gemv_ksplit_batch<FMT, XT, 3>(p, bj, s);
        case 4: return gemv_ksplit_batch<FMT, XT, 4>(p, bj, s);
        case 5: return gemv_ksplit_batch<FMT, XT, 5>(p, bj, s);
        case 6: return gemv_ksplit_batch<FMT, XT, 6>(p, bj, s);
        case 7: return gemv_ksplit_batch<FMT, XT, 7>(p, bj, s);
        case 8: return gemv_ksplit_batch<FMT, XT, 8>(p, bj, s);
        default: return false;
    }
}

template <int FMT>
static bool gemv_batch_xt(int xt, const GemmParams& p, const BatchJobs& bj, hipStream_t s) {
    if (xt == XT_F32) return gemv_batch_t<FMT, XT_F32>(p, bj, s);
    if (xt == XT_F16) return gemv_batch_t<FMT, XT_F16>(p, bj, s);
    return gemv_batch_t<FMT, XT_BF16>(p, bj, s);
}

bool launch_gemv_batch(int fmt, int xt, const GemmParams& p, const BatchJobs& bj, hipStream_t s, hipError_t& err) {
    bool ok;
    if (fmt == FMT_Q4) ok = gemv_batch_xt<FMT_Q4>(xt, p, bj, s);
    else if (fmt == FMT_Q4A) ok = gemv_batch_xt<FMT_Q4A>(xt, p, bj, s);
    else if (fmt == FMT_Q8A) ok = gemv_batch_xt<FMT_Q8A>(xt, p, bj, s);
    else ok = gemv_batch_xt<FMT_Q8>(xt, p, bj, s);
    err = ok ? hipGetLastError() : hipSuccess;
    return ok;
}

bool launch_gemv1_batch(int fmt, int xt, const GemmParams& p, const BatchJobs& bj, hipStream_t s, hipError_t& err) {
    bool ok;
    if (fmt == FMT_Q4) ok = gemv1_batch_xt<FMT_Q4>(xt, p, bj, s);
    else if (fmt == FMT_Q4A) ok = gemv1_batch_xt<FMT_Q4A>(xt, p, bj, s);
    else if (fmt == FMT_Q8A) ok = gemv1_batch_xt<FMT_Q8A>(xt, p, bj, s);
    else ok = gemv1_batch_xt<FMT_Q8>(xt, p, bj, s);
    err = ok ? hipGetLastError() : hipSuccess;
    return ok;
}

hipError_t launch_gemv(int fmt, int xt, const GemmParams& p, bool grouped, hipStream_t s) {
    if (fmt == FMT_Q4) gemv_xt<FMT_Q4>(xt, p, grouped, s);
    else if (fmt == FMT_Q4A) gemv_xt<FMT_Q4A>(xt, p, grouped, s);
    else if (fmt == FMT_Q8A) gemv_xt<FMT_Q8A>(xt, p, grouped, s);
    else if (fmt == FMT_Q8A16 && !grouped) gemv_xt<FMT_Q8A16>(xt, p, false, s);
    else if (fmt == FMT_Q8A16) return hipErrorInvalidValue;
    else gemv_xt<FMT_Q8>(xt, p, grouped, s);
    return hipGetLastError();
}

}  // namespace qg
