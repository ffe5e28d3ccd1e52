// qg_gemm.hip -- MFMA tile kernels of the block-quantized matmul Y = X . dequant(W)^T (gfx950).
//
// Prior art: page "oxinfer 0.0.5 src/metal.rs", SHADER_SRC gemm_body (f32 tile, weights
// dequantized per 32-k block) and MMA_SHADER_SRC mma_tile / MMAG (half operands, f32 accumulation,
// grouped tiles over experts).  The tiling here is CDNA4's own:
//
//  * A workgroup is 4 wavefronts and owns BT rows of X (tokens) by BN = 4 * 32 * MN weight rows.
//    Wavefront w owns weight rows [w*32*MN, (w+1)*32*MN) of the tile and every token row, so each
//    weight element is decoded exactly once per token tile.
//  * Weights never pass through LDS: in each 64-k stage, lane (row n = lane % 32, g = lane / 32)
//    loads the 16 code bytes of block 2s+g of its row (one coalesced 128-bit load), decodes them in
//    registers and feeds them straight into the MFMA B operand.  Lane group g supplies the k values
//    of block 2s+g to every MFMA of the stage; the A operand (X) uses the same assignment, so the
//    contraction covers every k of the stage exactly once.
//  * X is staged through LDS, double-buffered, one barrier per stage; rows padded by 16 bytes.
//  * Fast mode: v_mfma_f32_32x32x16_{f16,bf16}, 4 MFMAs per 32x32 tile per stage (MFMA j takes
//    elements 8j..8j+7 of each lane group's block).  Exact mode: v_mfma_f32_32x32x2_f32, 32 MFMAs
//    per tile per stage (MFMA j takes element j).
//  * Grouped (MoE) launches: blockIdx.y enumerates the row tiles of all experts' segments; each
//    workgroup finds its (expert, first row) by a wavefront prefix scan over seg_off.
//  * Rows beyond the tile's valid range and weight rows beyond N are clamped on load and never
//    stored; a K tail of one block (K % 64 == 32) zeroes both operands of the missing block.
#include "qg_device.hpp"
#include "qg_internal.hpp"

namespace qg {

constexpr int kThreads = 256;

// Finds the row tile of blockIdx.y.  Dense: rows [y*BT, min(R, y*BT+BT)) of the single matrix.
// Grouped: tiles of BT rows over every expert's segment, experts ascending.  Returns false when the
// workgroup has no tile (grouped launches are sized for the worst case).
template <int BT>
__device__ __forceinline__ bool find_tile(const GemmParams& p, bool grouped, int& e_out, int& r0, int& r1) {
    if (!grouped) {
        e_out = 0;
        r0 = blockIdx.y * BT;
        r1 = min(p.R, r0 + BT);
        return r0 < p.R;
    }
    __shared__ int s_tile[3];
    const int lane = threadIdx.x & 63;
    if (threadIdx.x < 64) {
        if (lane == 0) s_tile[0] = -1;
        int before = 0;
        const int y = blockIdx.y;
        for (int base = 0; base < p.E; base += 64) {
            const int e = base + lane;
            int a = 0, b = 0, cnt = 0;
            if (e < p.E) {
                a = min(max(p.seg_off[e], 0), p.R);
                b = min(max(p.seg_off[e + 1], a), p.R);
                cnt = (b - a + BT - 1) / BT;
            }
            int incl = cnt;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int v = __shfl_up(incl, o, 64);
                if (lane >= o) incl += v;
            }
            const int excl = before + incl - cnt;
            if (cnt > 0 && y >= excl && y < excl + cnt) {
                s_tile[0] = e;
                s_tile[1] = a + (y - excl) * BT;
                s_tile[2] = b;
            }
            before += __shfl(incl, 63, 64);
        }
    }
    __syncthreads();
    e_out = s_tile[0];
    if (e_out < 0) return false;
    r0 = s_tile[1];
    r1 = min(s_tile[2], r0 + BT);
    return true;
}

// X row of output row r; -1 means a zero row.
__device__ __forceinline__ int x_row_of(const GemmParams& p, int r) {
    if (!p.row_src) return r;
    const int s = p.row_src[r];
    return (s >= 0 && s < p.x_rows) ? s : -1;
}

// ================================================================================================
// Fast mode: f16 / bf16 MFMA, f32 accumulation.  X is f16 (ST = XT_F16) or bf16 (ST = XT_BF16).
// Software pipeline per wavefront: while the MFMAs of stage s run on fragments decoded earlier,
// the raw blocks of stage s+1 are decoded (independent instructions the scheduler can interleave
// with the MFMAs), the blocks of stage s+2 and the X chunk of stage s+1 are in flight.
template <int FMT, int ST, int MT, int MN>
__global__ __launch_bounds__(kThreads, 1) void gemm_fast_kernel(GemmParams p, bool grouped) {
    constexpr int BT = 32 * MT;
    constexpr int BN = 4 * 32 * MN;
    constexpr int PITCH = 72;  // halves per LDS row: 64 + 8 (16-byte pad)
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][BT * PITCH];

    int e, r0, r1;
    if (!find_tile<BT>(p, grouped, e, r0, r1)) return;
    const void* codes = p.codes;
    const void* scales = p.scales;
    const uint16_t* offs = p.offs;
    if (grouped) {
        codes = p.experts[e].codes;
        scales = p.experts[e].scales;
        offs = p.experts[e].offsets;
    }
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n_base = blockIdx.x * BN + wave * 32 * MN;
    const int g = lane >> 5, li = lane & 31;
    const int K = p.K, nblk = K >> 5, nstage = (K + 63) >> 6;
    const uint16_t* X = (const uint16_t*)p.X;

    // X staging: chunk c (16 bytes = 8 halves) -> tile row c / 8, column 8 * (c % 8).
    constexpr int XCH = BT * 8 / kThreads;  // chunks per thread
    int xrow[XCH];
#pragma unroll
    for (int i = 0; i < XCH; i++) {
        const int c = tid + i * kThreads;
        xrow[i] = x_row_of(p, min(r0 + c / 8, r1 - 1));
    }
    auto load_x = [&](int st, uint4 (&v)[XCH]) {
#pragma unroll
        for (int i = 0; i < XCH; i++) {
            const int c = tid + i * kThreads;
            const int k = st * 64 + 8 * (c & 7);
            if (xrow[i] >= 0 && k < K)
                v[i] = *(const uint4*)(X + (size_t)xrow[i] * K + k);
            else
                v[i] = make_uint4(0, 0, 0, 0);
        }
    };
    auto store_x = [&](int buf, const uint4 (&v)[XCH]) {
#pragma unroll
        for (int i = 0; i < XCH; i++) {
            const int c = tid + i * kThreads;
            *(uint4*)(&xs[buf][(c >> 3) * PITCH + 8 * (c & 7)]) = v[i];
        }
    };
    int wrow[MN];
#pragma unroll
    for (int mn = 0; mn < MN; mn++) wrow[mn] = min(n_base + 32 * mn + li, p.N - 1);
    auto load_w = [&](int st, RawBlock<FMT> (&w)[MN]) {
        const int b = min(2 * st + g, nblk - 1);
#pragma unroll
        for (int mn = 0; mn < MN; mn++) w[mn] = load_block<FMT>(codes, scales, offs, p.group, K, wrow[mn], b);
    };
    // B fragments of stage st (zero for a block beyond K, i.e. K % 64 == 32 at the last stage).
    auto decode = [&](int st, const RawBlock<FMT> (&w)[MN], short8_t (&bf)[MN][4]) {
        const bool valid = 2 * st + g < nblk;
#pragma unroll
        for (int mn = 0; mn < MN; mn++) {
            block_to_frags16<FMT, ST>(w[mn], bf[mn]);
            if (!valid)
#pragma unroll
                for (int j = 0; j < 4; j++) bf[mn][j] = short8_t{0, 0, 0, 0, 0, 0, 0, 0};
        }
    };

    f32x16_t acc[MT][MN];
#pragma unroll
    for (int a = 0; a < MT; a++)
#pragma unroll
        for (int b = 0; b < MN; b++)
#pragma unroll
            for (int i = 0; i < 16; i++) acc[a][b][i] = 0.f;

    uint4 xv[XCH];
    RawBlock<FMT> w1[MN];
    short8_t fc[MN][4];
    {
        RawBlock<FMT> w0[MN];
        load_x(0, xv);
        load_w(0, w0);
        if (nstage > 1) load_w(1, w1);
        store_x(0, xv);
        decode(0, w0, fc);
    }
    __syncthreads();

    for (int s = 0; s < nstage; s++) {
        const int buf = s & 1;
        const bool more = s + 1 < nstage;
        RawBlock<FMT> w2[MN];
        if (s + 2 < nstage) load_w(s + 2, w2);
        if (more) load_x(s + 1, xv);
        short8_t fn[MN][4];
        if (more) decode(s + 1, w1, fn);
#pragma unroll
        for (int j = 0; j < 4; j++) {
#pragma unroll
            for (int mt = 0; mt < MT; mt++) {
                const short8_t a = *(const short8_t*)(&xs[buf][(mt * 32 + li) * PITCH + 32 * g + 8 * j]);
#pragma unroll
                for (int mn = 0; mn < MN; mn++) {
                    if constexpr (ST == XT_F16)
                        acc[mt][mn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            __builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, fc[mn][j]), acc[mt][mn], 0, 0, 0);
                    else
                        acc[mt][mn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, fc[mn][j]), acc[mt][mn], 0, 0,
                            0);
                }
            }
        }
        if (more) {
            store_x(buf ^ 1, xv);
#pragma unroll
            for (int mn = 0; mn < MN; mn++) {
#pragma unroll
                for (int j = 0; j < 4; j++) fc[mn][j] = fn[mn][j];
                w1[mn] = w2[mn];
            }
        }
        __syncthreads();
    }

    // Epilogue: D[row][col] with col = lane % 32 (weight row), row = 8*(i/4) + 4*(lane/32) + i%4 (token).
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int mn = 0; mn < MN; mn++) {
            const int n = n_base + 32 * mn + li;
            if (n >= p.N) continue;
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int r = r0 + mt * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
                if (r < r1) {
                    float v = acc[mt][mn][i];
                    if (p.rs) v *= p.rs[r];
                    p.Y[(size_t)r * p.N + n] = v;
                }
            }
        }
}

// ================================================================================================
// Exact mode: f32 MFMA (v_mfma_f32_32x32x2_f32), f32 accumulation; X f32, f16 or bf16 widened.
template <int FMT, int XT, int MT, int MN>
__global__ __launch_bounds__(kThreads) void gemm_exact_kernel(GemmParams p, bool grouped) {
    constexpr int BT = 32 * MT;
    constexpr int BN = 4 * 32 * MN;
    constexpr int PITCH = 68;  // floats per LDS row: 64 + 4 (16-byte pad)
    __shared__ __attribute__((aligned(16))) float xs[2][BT * PITCH];

    int e, r0, r1;
    if (!find_tile<BT>(p, grouped, e, r0, r1)) return;
    const void* codes = p.codes;
    const void* scales = p.scales;
    const uint16_t* offs = p.offs;
    if (grouped) {
        codes = p.experts[e].codes;
        scales = p.experts[e].scales;
        offs = p.experts[e].offsets;
    }
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n_base = blockIdx.x * BN + wave * 32 * MN;
    const int g = lane >> 5, li = lane & 31;
    const int K = p.K, nblk = K >> 5, nstage = (K + 63) >> 6;

    // X staging in 8-element chunks: chunk c -> tile row c / 8, columns 8 * (c % 8) .. +7.
    constexpr int XCH = BT * 8 / kThreads;
    int xrow[XCH];
#pragma unroll
    for (int i = 0; i < XCH; i++) {
        const int c = tid + i * kThreads;
        xrow[i] = x_row_of(p, min(r0 + c / 8, r1 - 1));
    }
    auto load_x = [&](int s, float (&v)[XCH][8]) {
#pragma unroll
        for (int i = 0; i < XCH; i++) {
            const int c = tid + i * kThreads;
            const int k = s * 64 + 8 * (c & 7);
            if (xrow[i] >= 0 && k < K)
                x_load8<XT>(p.X, (size_t)xrow[i] * K + k, v[i]);
            else
#pragma unroll
                for (int j = 0; j < 8; j++) v[i][j] = 0.f;
        }
    };
    auto store_x = [&](int buf, const float (&v)[XCH][8]) {
#pragma unroll
        for (int i = 0; i < XCH; i++) {
            const int c = tid + i * kThreads;
            float4* d = (float4*)(&xs[buf][(c >> 3) * PITCH + 8 * (c & 7)]);
            d[0] = make_float4(v[i][0], v[i][1], v[i][2], v[i][3]);
            d[1] = make_float4(v[i][4], v[i][5], v[i][6], v[i][7]);
        }
    };
    int wrow[MN];
#pragma unroll
    for (int mn = 0; mn < MN; mn++) wrow[mn] = min(n_base + 32 * mn + li, p.N - 1);
    auto load_w = [&](int s, RawBlock<FMT> (&w)[MN]) {
        const int b = min(2 * s + g, nblk - 1);
#pragma unroll
        for (int mn = 0; mn < MN; mn++) w[mn] = load_block<FMT>(codes, scales, offs, p.group, K, wrow[mn], b);
    };

    f32x16_t acc[MT][MN];
#pragma unroll
    for (int a = 0; a < MT; a++)
#pragma unroll
        for (int b = 0; b < MN; b++)
#pragma unroll
            for (int i = 0; i < 16; i++) acc[a][b][i] = 0.f;

    float xv[XCH][8];
    RawBlock<FMT> wr[MN];
    load_x(0, xv);
    load_w(0, wr);
    store_x(0, xv);
    __syncthreads();

    for (int s = 0; s < nstage; s++) {
        const int buf = s & 1;
        const bool more = s + 1 < nstage;
        RawBlock<FMT> wn[MN];
        if (more) {
            load_x(s + 1, xv);
            load_w(s + 1, wn);
        }
        const bool valid = 2 * s + g < nblk;
        float wv[MN][32];
#pragma unroll
        for (int mn = 0; mn < MN; mn++) {
            block_to_f32<FMT>(wr[mn], wv[mn]);
            if (!valid)
#pragma unroll
                for (int j = 0; j < 32; j++) wv[mn][j] = 0.f;
        }
#pragma unroll
        for (int q = 0; q < 8; q++) {
#pragma unroll
            for (int mt = 0; mt < MT; mt++) {
                const float4 a = *(const float4*)(&xs[buf][(mt * 32 + li) * PITCH + 32 * g + 4 * q]);
                const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                for (int jj = 0; jj < 4; jj++)
#pragma unroll
                    for (int mn = 0; mn < MN; mn++)
                        acc[mt][mn] =
                            __builtin_amdgcn_mfma_f32_32x32x2f32(av[jj], wv[mn][4 * q + jj], acc[mt][mn], 0, 0, 0);
            }
        }
        if (more) {
            store_x(buf ^ 1, xv);
#pragma unroll
            for (int mn = 0; mn < MN; mn++) wr[mn] = wn[mn];
        }
        __syncthreads();
    }

#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int mn = 0; mn < MN; mn++) {
            const int n = n_base + 32 * mn + li;
            if (n >= p.N) continue;
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int r = r0 + mt * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
                if (r < r1) {
                    float v = acc[mt][mn][i];
                    if (p.rs) v *= p.rs[r];
                    p.Y[(size_t)r * p.N + n] = v;
                }
            }
        }
}

// ================================================================================================
// Launchers.  Tile choice: the largest tile that still gives at least one workgroup per CU.
static int grid_rows(const GemmParams& p, bool grouped, int BT) {
    if (!grouped) return (p.R + BT - 1) / BT;
    return (p.R + BT - 1) / BT + min(p.E, p.R);
}

template <int FMT, int ST, int MT, int MN>
static void fast_launch(const GemmParams& p, bool grouped, hipStream_t s) {
    dim3 grid((p.N + 128 * MN - 1) / (128 * MN), grid_rows(p, grouped, 32 * MT));
    hipLaunchKernelGGL((gemm_fast_kernel<FMT, ST, MT, MN>), grid, dim3(kThreads), 0, s, p, grouped);
}

template <int FMT, int ST>
static void fast_pick(const GemmParams& p, bool grouped, hipStream_t s) {
    if (grouped) return fast_launch<FMT, ST, 1, 2>(p, grouped, s);
    // The largest tile that still gives about one workgroup per CU: big tiles amortize each
    // decoded weight over more tokens and each staged X row over more weight rows.
    auto wgs = [&](int bt, int bn) { return (long)((p.N + bn - 1) / bn) * ((p.R + bt - 1) / bt); };
    if (wgs(256, 256) >= 200) return fast_launch<FMT, ST, 8, 2>(p, grouped, s);
    if (wgs(128, 256) >= 200) return fast_launch<FMT, ST, 4, 2>(p, grouped, s);
    if (wgs(128, 128) >= 200) return fast_launch<FMT, ST, 4, 1>(p, grouped, s);
    return fast_launch<FMT, ST, 2, 1>(p, grouped, s);
}

hipError_t launch_gemm_fast(int fmt, int st, const GemmParams& p, bool grouped, hipStream_t s) {
    if (st == XT_F16) {
        if (fmt == FMT_Q4) fast_pick<FMT_Q4, XT_F16>(p, grouped, s);
        else if (fmt == FMT_Q4A) fast_pick<FMT_Q4A, XT_F16>(p, grouped, s);
        else fast_pick<FMT_Q8, XT_F16>(p, grouped, s);
    } else {
        if (fmt == FMT_Q4) fast_pick<FMT_Q4, XT_BF16>(p, grouped, s);
        else if (fmt == FMT_Q4A) fast_pick<FMT_Q4A, XT_BF16>(p, grouped, s);
        else fast_pick<FMT_Q8, XT_BF16>(p, grouped, s);
    }
    return hipGetLastError();
}

template <int FMT, int XT, int MT, int MN>
static void exact_launch(const GemmParams& p, bool grouped, hipStream_t s) {
    dim3 grid((p.N + 128 * MN - 1) / (128 * MN), grid_rows(p, grouped, 32 * MT));
    hipLaunchKernelGGL((gemm_exact_kernel<FMT, XT, MT, MN>), grid, dim3(kThreads), 0, s, p, grouped);
}

template <int FMT, int XT>
static void exact_pick(const GemmParams& p, bool grouped, hipStream_t s) {
    if (grouped) return exact_launch<FMT, XT, 1, 1>(p, grouped, s);
    const long mid = (long)((p.N + 127) / 128) * ((p.R + 63) / 64);
    if (mid >= 200) return exact_launch<FMT, XT, 2, 1>(p, grouped, s);
    return exact_launch<FMT, XT, 1, 1>(p, grouped, s);
}

template <int FMT>
static void exact_xt(int xt, const GemmParams& p, bool grouped, hipStream_t s) {
    if (xt == XT_F32) exact_pick<FMT, XT_F32>(p, grouped, s);
    else if (xt == XT_F16) exact_pick<FMT, XT_F16>(p, grouped, s);
    else exact_pick<FMT, XT_BF16>(p, grouped, s);
}

hipError_t launch_gemm_exact(int fmt, int xt, const GemmParams& p, bool grouped, hipStream_t s) {
    if (fmt == FMT_Q4) exact_xt<FMT_Q4>(xt, p, grouped, s);
    else if (fmt == FMT_Q4A) exact_xt<FMT_Q4A>(xt, p, grouped, s);
    else exact_xt<FMT_Q8>(xt, p, grouped, s);
    return hipGetLastError();
}

}  // namespace qg
