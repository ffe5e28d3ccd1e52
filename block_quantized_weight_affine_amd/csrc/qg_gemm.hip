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
#include <type_traits>

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
// Weight rows of one lane: row pointers into the codes, scales and offsets of the lane's rows.
template <int FMT, int MN>
struct LaneRows {
    static_assert(!blk16<FMT>, "16-element blocks: exact kernel only");
    const QG_GLOBAL uint8_t* codes[MN];
    const QG_GLOBAL uint8_t* scales[MN];  // f16 (Q4, Q4A) or f32 (Q8) scales of the row
    const QG_GLOBAL uint16_t* offs[MN];   // Q4A offsets of the row (Q8A: f32, per block)
    int group;

    __device__ __forceinline__ void init(const void* c, const void* sc, const uint16_t* of, int grp, int K, int N,
                                         int row0) {
        group = grp;
#pragma unroll
        for (int mn = 0; mn < MN; mn++) {
            const size_t n = (size_t)min(row0 + 32 * mn, N - 1);
            const size_t row_bytes = q8_layout<FMT> ? (size_t)K : (size_t)(K >> 1);
            codes[mn] = gptr<uint8_t>((const uint8_t*)c + n * row_bytes);
            scales[mn] = gptr<uint8_t>((const uint8_t*)sc + n * (size_t)(K >> 5) * (q8_layout<FMT> ? 4 : 2));
            offs[mn] = FMT == FMT_Q4A ? gptr<uint16_t>(of + n * (size_t)(K / grp))
                       : FMT == FMT_Q8A ? gptr<uint16_t>((const float*)(const void*)of + n * (size_t)(K >> 5))
                                        : nullptr;
        }
    }
    // Block b (in bounds) of every row.
    __device__ __forceinline__ void load(int b, RawBlock<FMT> (&w)[MN]) const {
#pragma unroll
        for (int mn = 0; mn < MN; mn++) {
            if constexpr (q8_layout<FMT>) {
                const QG_GLOBAL u32x4_t* q = (const QG_GLOBAL u32x4_t*)(codes[mn] + 32 * b);
                const u32x4_t a = q[0], c = q[1];
                w[mn].q0 = make_uint4(a.x, a.y, a.z, a.w);
                w[mn].q1 = make_uint4(c.x, c.y, c.z, c.w);
                w[mn].d = ((const QG_GLOBAL float*)scales[mn])[b];
                w[mn].m = FMT == FMT_Q8A ? ((const QG_GLOBAL float*)offs[mn])[b] : 0.f;
                w[mn].dh = 0;
            } else {
                const u32x4_t a = *(const QG_GLOBAL u32x4_t*)(codes[mn] + 16 * b);
                w[mn].q = make_uint4(a.x, a.y, a.z, a.w);
                w[mn].dh = ((const QG_GLOBAL uint16_t*)scales[mn])[b];
                w[mn].d = f16_to_f32((uint16_t)w[mn].dh);
                w[mn].m = FMT == FMT_Q4A ? bf16_to_f32(offs[mn][(32 * b) / group]) : 0.f;
            }
        }
    }
};

// Fast mode: f16 / bf16 MFMA, f32 accumulation.  X is f16 (ST = XT_F16) or bf16 (ST = XT_BF16).
// Software pipeline per wavefront: while the MFMAs of stage s run on fragments decoded earlier,
// the raw blocks of stage s+1 are decoded (independent instructions the scheduler can interleave
// with the MFMAs), and the blocks of stage s+2 and the X chunk of stage s+1 are in flight.  The
// stage body is one basic block: loads past the end are clamped to valid addresses (and unused),
// a K tail of one block (K % 64 == 32) is handled by zero X columns (the clamped weight block is
// multiplied by zeros), and the rare Q4A re-decode runs as a fix-up after the MFMAs.
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

    // X staging: chunk c = tid + i * threads (16 bytes = 8 halves) -> tile row c / 8, column
    // xcol = 8 * (tid % 8) (the same for every chunk of the thread).
    constexpr int XCH = BT * 8 / kThreads;
    const int xcol = 8 * (tid & 7);
    const QG_GLOBAL u32x4_t* xp[XCH];
    bool xok[XCH];
#pragma unroll
    for (int i = 0; i < XCH; i++) {
        const int c = tid + i * kThreads;
        const int row = x_row_of(p, min(r0 + c / 8, r1 - 1));
        xok[i] = row >= 0;
        xp[i] = gptr<u32x4_t>((const uint16_t*)p.X + (size_t)max(row, 0) * K + xcol);
    }
    // Stage st's chunk: columns st*64 + xcol .. +7 of the thread's rows, zero for a zero row or for
    // columns at or beyond K; the address is clamped to columns K-8 .. K-1 so it stays in bounds.
    auto load_x = [&](int st, uint4 (&v)[XCH]) {
        const bool kin = st * 64 + xcol < K;
        const int off = min(st * 64, K - 8 - xcol) >> 3;  // in 16-byte units from the row's column xcol
#pragma unroll
        for (int i = 0; i < XCH; i++) {
            const u32x4_t t = xp[i][off];
            const bool ok = xok[i] && kin;
            v[i] = make_uint4(ok ? t.x : 0u, ok ? t.y : 0u, ok ? t.z : 0u, ok ? t.w : 0u);
        }
    };
    auto store_x = [&](int buf, const uint4 (&v)[XCH]) {
#pragma unroll
        for (int i = 0; i < XCH; i++) {
            const int c = tid + i * kThreads;
            *(uint4*)(&xs[buf][(c >> 3) * PITCH + xcol]) = v[i];
        }
    };
    LaneRows<FMT, MN> rows;
    rows.init(codes, scales, offs, p.group, K, p.N, n_base + li);
    auto load_w = [&](int st, RawBlock<FMT> (&w)[MN]) { rows.load(min(2 * st + g, nblk - 1), w); };

    f32x16_t acc[MT][MN];
#pragma unroll
    for (int a = 0; a < MT; a++)
#pragma unroll
        for (int b = 0; b < MN; b++)
#pragma unroll
            for (int i = 0; i < 16; i++) acc[a][b][i] = 0.f;

    // MFMAs of one stage; the A fragments of step j+1 are read from LDS before the MFMAs of step j.
    auto mfmas = [&](int buf, const short8_t (&fc)[MN][4]) {
        const uint16_t* xb = &xs[buf][li * PITCH + 32 * g];
        short8_t a[2][MT];
#pragma unroll
        for (int mt = 0; mt < MT; mt++) a[0][mt] = *(const short8_t*)(xb + mt * 32 * PITCH);
#pragma unroll
        for (int j = 0; j < 4; j++) {
            if (j < 3)
#pragma unroll
                for (int mt = 0; mt < MT; mt++) a[(j + 1) & 1][mt] = *(const short8_t*)(xb + mt * 32 * PITCH + 8 * (j + 1));
#pragma unroll
            for (int mt = 0; mt < MT; mt++) {
#pragma unroll
                for (int mn = 0; mn < MN; mn++) {
                    if constexpr (ST == XT_F16)
                        acc[mt][mn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a[j & 1][mt]),
                                                                             __builtin_bit_cast(half8_t, fc[mn][j]),
                                                                             acc[mt][mn], 0, 0, 0);
                    else
                        acc[mt][mn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8_t, a[j & 1][mt]), __builtin_bit_cast(bf16x8_t, fc[mn][j]),
                            acc[mt][mn], 0, 0, 0);
                }
            }
        }
    };

    uint4 xv[XCH];
    RawBlock<FMT> w1[MN];
    short8_t fc[MN][4];
    {
        RawBlock<FMT> w0[MN];
        load_x(0, xv);
        load_w(0, w0);
        load_w(min(1, nstage - 1), w1);
        store_x(0, xv);
#pragma unroll
        for (int mn = 0; mn < MN; mn++) block_to_frags16<FMT, ST>(w0[mn], fc[mn]);
    }
    __syncthreads();

    for (int s = 0; s < nstage; s++) {
        const int buf = s & 1;
        RawBlock<FMT> w2[MN];
        load_w(min(s + 2, nstage - 1), w2);
        load_x(min(s + 1, nstage - 1), xv);
        short8_t fn[MN][4];
#pragma unroll
        for (int mn = 0; mn < MN; mn++) block_to_frags16_fast<FMT, ST>(w1[mn], fn[mn]);
        mfmas(buf, fc);
        store_x(buf ^ 1, xv);
#pragma unroll
        for (int mn = 0; mn < MN; mn++)
            if (frags16_need_fixup<FMT, ST>(w1[mn])) block_frags16_fixup<FMT, ST>(w1[mn], fn[mn]);
        __syncthreads();
#pragma unroll
        for (int mn = 0; mn < MN; mn++) {
#pragma unroll
            for (int j = 0; j < 4; j++) fc[mn][j] = fn[mn][j];
            w1[mn] = w2[mn];
        }
    }

    // Epilogue: D[row][col] with col = lane % 32 (weight row), row = 8*(i/4) + 4*(lane/32) + i%4 (token).
    QG_GLOBAL float* Y = gptr_mut<float>(p.Y);
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
                    Y[(size_t)r * p.N + n] = v;
                }
            }
        }
}

// ================================================================================================
// Dense fast mode through LDS tiles (large token counts).  Per 64-k stage the workgroup decodes the
// weight slab once, cooperatively, into an LDS tile of BN rows (f16 / bf16, 16-byte padded rows,
// natural k order), next to the X slab.  The 4 wavefronts sit in a WM x WN grid; wavefront
// (wm, wn) reads its A fragments (32*MT token rows) and B fragments (32*MN weight rows) from LDS,
// so each fragment read feeds MN or MT MFMAs.  MFMA step j covers k 16j .. 16j+15 of the stage;
// lane group g holds k 16j+8g .. +7 of both operands.
//
// X goes from HBM straight into LDS (buffer_load ... lds, 16 bytes per lane): no registers, and
// chunks past K or past the tile's last row read as zero.  One such load writes 64 consecutive
// 16-byte slots, i.e. 8 whole rows of the slab; the lane for slot p of row r fetches chunk
// p ^ ((r / 2) % 8), so chunk c of row r sits at slot c ^ ((r / 2) % 8).  A fragment read takes
// one chunk from 16 consecutive rows per LDS cycle (16 lanes x 16 bytes over 64 banks): rows of
// one parity land on 8 different slots and the two parities on the two 128-byte halves of the
// bank space, so the 16 lanes hit 16 different bank quads.
//
// Pipeline of stage s (one wavefront per SIMD, so each wavefront keeps its matrix core busy by
// itself): buffers C hold X(s) and W(s), the raw blocks of W(s+1) are in registers.  In one
// straight-line region the wavefront starts the X(s+1) copy into the other X buffer and the raw
// loads of W(s+2) into the second register set, decodes W(s+1) into the other weight buffer and
// runs the 4 * MT * MN MFMAs of stage s, reading the fragments of step j+1 during step j; the
// decode's VALU work is interleaved with the MFMAs (sched_group_barrier), where it runs beside
// the matrix core.  Blocks whose fast decode (1) is not the pages' rounding are re-loaded and
// re-decoded in the pages' order after the MFMAs; one barrier (which waits for all of the stage's
// copies) ends the stage.  The two LDS buffers are separate arrays and the stage loop is unrolled,
// so the compiler can see that the decode's stores and the MFMA reads never alias.
//
// Small tiles (DP = 4) have stages too short to cover a memory round trip with one stage of lead:
// their X chunks load into a ring of 4 register sets 4 stages ahead (buffer loads, zero past K and
// past the tile) and are stored to LDS at the end of the stage before they are used, and the raw
// weight blocks load into 4 register sets, 4 stages ahead.  (A deeper ring of direct LDS copies
// would not help: the stage-end barrier waits for every copy in flight.)
//
// Decode ownership: a stage holds 2 BN blocks = 8 BN fragments of 8 values, FPT = BN / 32 per
// thread; a thread owns FPB = min(FPT, 4) fragments of each of its blocks, so narrow tiles still
// spread the decode over all 256 threads.
// Stages s .. s+U-1 of an unrolled stage loop (stage u of the group gets u as a compile-time index),
// and the at most U-1 stages left after the last whole group.
template <int I, int U, class F>
__device__ __forceinline__ void run_stages(F& f, int s) {
    f(std::integral_constant<int, I>{}, s + I);
    if constexpr (I + 1 < U) run_stages<I + 1, U>(f, s);
}
// f(integral_constant<I>) for I .. U-1
template <int I, int U, class F>
__device__ __forceinline__ void run_stages_c(F& f) {
    if constexpr (I < U) {
        f(std::integral_constant<int, I>{});
        run_stages_c<I + 1, U>(f);
    }
}
template <int I, int U, class F>
__device__ __forceinline__ void run_tail_stages(F& f, int s, int nstage) {
    if constexpr (I < U - 1) {
        if (s + I < nstage) {
            f(std::integral_constant<int, I>{}, s + I);
            run_tail_stages<I + 1, U>(f, s, nstage);
        }
    }
}

template <int FMT, int ST, int WM, int MT, int MN, int DP, bool GR>
__global__ __launch_bounds__(kThreads, 1) void gemm_fast_lds_kernel(GemmParams p) {
    constexpr int WN = 4 / WM;
    constexpr int BT = 32 * MT * WM;
    constexpr int BN = 32 * MN * WN;
    constexpr int PITCH = 72;               // halves per weight-tile row: 64 + 8 (16-byte pad)
    constexpr int FPT = BN / 32;            // 8-value fragments decoded per thread per stage
    constexpr int FPB = FPT < 4 ? FPT : 4;  // fragments of one block a thread decodes
    constexpr int TPB = 4 / FPB;            // threads sharing one block
    constexpr int WB = FPT / FPB;           // blocks per thread per stage
    constexpr int XCH = BT / 32;            // X row-octets copied per wavefront per stage
    static_assert(FPT >= 1 && (FPT == 1 || FPT == 2 || FPT % 4 == 0) && BT % 32 == 0, "tile");
    __shared__ __attribute__((aligned(16))) uint16_t xs0[BT * 64];
    __shared__ __attribute__((aligned(16))) uint16_t xs1[BT * 64];
    // The last row's pad is never touched: leaving it out keeps two 32 x 256 grouped workgroups
    // (and their tile lookup slot) within one CU's 160 KiB.
    __shared__ __attribute__((aligned(16))) uint16_t ws0[BN * PITCH - 8];
    __shared__ __attribute__((aligned(16))) uint16_t ws1[BN * PITCH - 8];

    // Grouped (MoE) launches: blockIdx.y enumerates the row tiles of every expert's segment
    // (find_tile); the tile's weights are its expert's.  X rows are rows r0 .. r1-1 of p.X either way.
    int e = 0, r0 = blockIdx.y * BT, r1 = min(p.R, r0 + BT);
    if constexpr (GR) {
        if (!find_tile<BT>(p, true, e, r0, r1)) return;
    }
    const void* const wcodes = GR ? p.experts[e].codes : p.codes;
    const void* const wscales = GR ? p.experts[e].scales : p.scales;
    const uint16_t* const woffs = GR ? p.experts[e].offsets : p.offs;
    const int n0 = blockIdx.x * BN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int g = lane >> 5, li = lane & 31;
    const int K = p.K, nblk = K >> 5, nstage = (K + 63) >> 6;

    // X rows r0 .. r1-1 as one buffer resource: offsets past its end (rows past the tile) and the
    // offsets used for columns past K read as zero.
    uint16_t* const xbase = (uint16_t*)p.X + (size_t)r0 * K;
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(xbase, 0, (r1 - r0) * K * 2, 0x00020000);
    // DP == 1, X copy i of wavefront w: rows 8 (4 i + w) .. +7 of the slab; this lane's slot is
    // row r = 8 (4 i + w) + lane / 8, position lane % 8, holding chunk xc = (lane % 8) ^ ((r / 2) % 8),
    // where (r / 2) % 8 = 4 (w % 2) + lane / 16.
    // DP > 1, X chunk i of a thread: row r = tid / 8 + 32 i, chunk tid % 8, loaded DP stages ahead
    // into registers and stored at slot (tid % 8) ^ ((r / 2) % 8), where (r / 2) % 8 = (tid / 16) % 8.
    const int xc = DP == 1 ? (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7) : (tid & 7);
    int xoff[XCH];
#pragma unroll
    for (int i = 0; i < XCH; i++)
        xoff[i] = (DP == 1 ? 8 * (4 * i + wave) + (lane >> 3) : (tid >> 3) + 32 * i) * K * 2 + 16 * xc;
    auto xkoff = [&](int st) { return st * 64 + 8 * xc < K ? st * 128 : 0x40000000; };  // 2^30 > any valid offset
    auto copy_x = [&](int st, uint16_t* xs) {
        const int koff = xkoff(st);
#pragma unroll
        for (int i = 0; i < XCH; i++)
            buffer_copy16_lds(xrs, xs + 8 * (4 * i + wave) * 64, xoff[i] + koff);
    };
    auto load_x = [&](int st, u32x4_t (&v)[XCH]) {
        const int koff = xkoff(st);
#pragma unroll
        for (int i = 0; i < XCH; i++) v[i] = __builtin_amdgcn_raw_buffer_load_b128(xrs, xoff[i] + koff, 0, 0);
    };
    auto store_x = [&](uint16_t* xs, const u32x4_t (&v)[XCH]) {
        const int slot = (tid & 7) ^ ((tid >> 4) & 7);
#pragma unroll
        for (int i = 0; i < XCH; i++) *(u32x4_t*)(xs + ((tid >> 3) + 32 * i) * 64 + 8 * slot) = v[i];
    };

    // Weight block i of a thread: q = tid / TPB + i * (threads / TPB) of the stage's 2 BN blocks,
    // tile row q / 2, block 2 st + hsel (hsel = q % 2) of that row, written to columns
    // 32 hsel .. 32 hsel + 31; the thread decodes its fragments fb .. fb + FPB - 1 of it.  Blocks
    // past K are loaded clamped and decoded with zero scale and offset, which gives +0 for every
    // element.
    const int hsel = (tid / TPB) & 1;
    const int fb = (tid % TPB) * FPB;
    auto blk = [&](int i) { return tid / TPB + i * (kThreads / TPB); };
    const QG_GLOBAL uint8_t* wc[WB];
    const QG_GLOBAL uint8_t* wsc[WB];
    const QG_GLOBAL uint16_t* wof[WB];
#pragma unroll
    for (int i = 0; i < WB; i++) {
        const size_t n = (size_t)min(n0 + blk(i) / 2, p.N - 1);
        wc[i] = gptr<uint8_t>((const uint8_t*)wcodes + n * (q8_layout<FMT> ? (size_t)K : (size_t)(K >> 1)));
        wsc[i] = gptr<uint8_t>((const uint8_t*)wscales + n * (size_t)(K >> (blk16<FMT> ? 4 : 5)) * (q8_layout<FMT> ? 4 : 2));
        wof[i] = FMT == FMT_Q4A ? gptr<uint16_t>(woffs + n * (size_t)(K / p.group))
                 : FMT == FMT_Q8A ? gptr<uint16_t>((const float*)(const void*)woffs + n * (size_t)(K >> 5))
                 : (blk16<FMT> && woffs) ? gptr<uint16_t>((const float*)(const void*)woffs + n * (size_t)(K >> 4))
                                  : nullptr;
    }
    auto load_w = [&](int st, RawBlock<FMT> (&w)[WB]) {
        const int b = min(2 * st + hsel, nblk - 1);
#pragma unroll
        for (int i = 0; i < WB; i++) {
            if constexpr (q8_layout<FMT>) {
                const QG_GLOBAL u32x4_t* q = (const QG_GLOBAL u32x4_t*)(wc[i] + 32 * b);
                const u32x4_t a = q[0], c = q[1];
                w[i].q0 = make_uint4(a.x, a.y, a.z, a.w);
                w[i].q1 = make_uint4(c.x, c.y, c.z, c.w);
                w[i].dh = 0;
                if constexpr (blk16<FMT>) {
                    // two (scale, offset) pairs; no offsets (NULL): -0, which changes no value
                    w[i].d = ((const QG_GLOBAL float*)wsc[i])[2 * b];
                    w[i].d2 = ((const QG_GLOBAL float*)wsc[i])[2 * b + 1];
                    w[i].m = woffs ? ((const QG_GLOBAL float*)wof[i])[2 * b] : -0.0f;
                    w[i].m2 = woffs ? ((const QG_GLOBAL float*)wof[i])[2 * b + 1] : -0.0f;
                } else {
                    w[i].d = ((const QG_GLOBAL float*)wsc[i])[b];
                    w[i].m = FMT == FMT_Q8A ? ((const QG_GLOBAL float*)wof[i])[b] : 0.f;
                }
            } else {
                const u32x4_t a = *(const QG_GLOBAL u32x4_t*)(wc[i] + 16 * b);
                w[i].q = make_uint4(a.x, a.y, a.z, a.w);
                w[i].dh = ((const QG_GLOBAL uint16_t*)wsc[i])[b];
                w[i].d = f16_to_f32((uint16_t)w[i].dh);
                w[i].m = FMT == FMT_Q4A ? bf16_to_f32(wof[i][(32 * b) / p.group]) : 0.f;
            }
        }
    };
    auto w_dst = [&](uint16_t* ws, int i) { return ws + (blk(i) >> 1) * PITCH + 32 * hsel; };
    // Q8A / Q8A16 (two roundings per value): every fragment is decoded in the pages' order as it is
    // staged, with no fast pass and no re-decode
    constexpr bool kSlowOnly = FMT == FMT_Q8A || blk16<FMT>;
    // Fast decode (1) of stage st into ws; need is set where a valid block needs the pages' order.
    auto decode_store = [&](int st, uint16_t* ws, const RawBlock<FMT> (&w)[WB], bool& need) {
        const bool valid = 2 * st + hsel < nblk;
#pragma unroll
        for (int i = 0; i < WB; i++) {
            RawBlock<FMT> r = w[i];
            block_clear_if<FMT>(r, valid);
            r.dh = valid ? r.dh : 0u;
            uint16_t* d = w_dst(ws, i);
            if constexpr (kSlowOnly) {
#pragma unroll
                for (int j = 0; j < FPB; j++) *(short8_t*)(d + 8 * (fb + j)) = frag16_slow<FMT, ST>(r, fb + j);
            } else {
                bool fast;
                const float c0 = block_c0<FMT>(r, fast);
                if constexpr (!(FMT == FMT_Q4 && ST == XT_F16)) need = need || (valid && !fast);
#pragma unroll
                for (int j = 0; j < FPB; j++) *(short8_t*)(d + 8 * (fb + j)) = frag16_fast<FMT, ST>(r, c0, fb + j);
            }
        }
    };
    // The pages' order for the blocks of stage st (rare: non-positive scales, inexact m - 8d).
    auto fixup = [&](int st, uint16_t* ws) {
        RawBlock<FMT> w[WB];
        load_w(st, w);
#pragma unroll
        for (int i = 0; i < WB; i++) {
            short8_t f[4];
            block_frags16_fixup<FMT, ST>(w[i], f);
            uint16_t* d = w_dst(ws, i);
#pragma unroll
            for (int j = 0; j < FPB; j++) *(short8_t*)(d + 8 * (fb + j)) = f[fb + j];
        }
    };

    f32x16_t acc[MT][MN];
#pragma unroll
    for (int a = 0; a < MT; a++)
#pragma unroll
        for (int b = 0; b < MN; b++)
#pragma unroll
            for (int i = 0; i < 16; i++) acc[a][b][i] = 0.f;

    // Fragments of MFMA step j: A from the swizzled X slab (row r, chunk 2j + g at slot
    // (2j + g) ^ ((r / 2) % 8), and (r / 2) % 8 = (li / 2) % 8), B from the padded weight tile.
    auto frags_a = [&](const uint16_t* xs, int j, short8_t (&A)[MT]) {
        const uint16_t* xa = xs + (wm * 32 * MT + li) * 64 + 8 * ((2 * j + g) ^ ((li >> 1) & 7));
#pragma unroll
        for (int mt = 0; mt < MT; mt++) A[mt] = *(const short8_t*)(xa + mt * 32 * 64);
    };
    auto frags_b = [&](const uint16_t* ws, int j, short8_t (&B)[MN]) {
        const uint16_t* wb = ws + (wn * 32 * MN + li) * PITCH + 8 * g + 16 * j;
#pragma unroll
        for (int mn = 0; mn < MN; mn++) B[mn] = *(const short8_t*)(wb + mn * 32 * PITCH);
    };
    auto mfma = [&](const short8_t& a, const short8_t& b, f32x16_t& c) {
        if constexpr (ST == XT_F16)
            c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
        else
            c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    };

    // A stage is cut into NCH chunks (CPS per MFMA step), each with MPC of the stage's MFMAs and
    // at most one fragment decode (fragment f of the thread in chunk f * NCH / FPT);
    // sched_barrier keeps every instruction in its chunk, so a decode runs beside the MFMAs of its
    // chunk, and the fragment reads of step j+1, issued in the first chunk of step j, have a whole
    // step of MFMAs to arrive.
    constexpr int CPS = FPT >= 4 ? FPT / 4 : 1;
    constexpr int NCH = 4 * CPS;
    constexpr int MPC = MT * MN / CPS;
    static_assert(MPC * CPS == MT * MN && (CPS == 1 || CPS == 2) && NCH % FPT == 0, "chunking");

    // Raw weights of stage t live in register set (t - 1) % NS and load NS stages ahead; with
    // DP > 1, X of stage t lives in register set t % DP and loads DP stages ahead.  The loop is
    // unrolled by U so every set and buffer index is a compile-time constant.
    constexpr int NS = DP == 1 ? 2 : DP;
    constexpr int U = NS;
    static_assert(U % 2 == 0, "the LDS buffers alternate");
    RawBlock<FMT> wr[NS][WB];
    u32x4_t xr[DP == 1 ? 1 : DP][XCH];

    auto stage = [&](auto uc, int s) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;
        const uint16_t* xc = (u & 1) ? xs1 : xs0;
        const uint16_t* wcur = (u & 1) ? ws1 : ws0;
        uint16_t* xn = (u & 1) ? xs0 : xs1;
        uint16_t* wnx = (u & 1) ? ws0 : ws1;
        short8_t A[2][MT], B[2][MN];
        frags_a(xc, 0, A[0]);
        frags_b(wcur, 0, B[0]);
        if constexpr (DP == 1)
            copy_x(s + 1, xn);
        else
            load_x(s + DP, xr[u % DP]);
        load_w(s + NS, wr[(u + NS - 1) % NS]);
        // Blocks past K decode with zero scale and offset (+0 everywhere).
        const bool valid = 2 * (s + 1) + hsel < nblk;
        RawBlock<FMT> r[WB];
        float c0[WB];
        bool need = false;
#pragma unroll
        for (int i = 0; i < WB; i++) {
            r[i] = wr[u % NS][i];
            block_clear_if<FMT>(r[i], valid);
            r[i].dh = valid ? r[i].dh : 0u;
            c0[i] = 0.f;
            if constexpr (!kSlowOnly) {
                bool fast;
                c0[i] = block_c0<FMT>(r[i], fast);
                if constexpr (!(FMT == FMT_Q4 && ST == XT_F16)) need = need || (valid && !fast);
            }
        }
#pragma unroll
        for (int q = 0; q < NCH; q++) {
            const int j = q / CPS, part = q % CPS;
            if (j < 3 && part == 0) {
                frags_a(xc, j + 1, A[(j + 1) & 1]);
                frags_b(wcur, j + 1, B[(j + 1) & 1]);
            }
#pragma unroll
            for (int m = 0; m < MPC; m++) {
                const int idx = part * MPC + m;
                mfma(A[j & 1][idx / MN], B[j & 1][idx % MN], acc[idx / MN][idx % MN]);
            }
            if (q % (NCH / FPT) == 0) {
                const int f = q / (NCH / FPT);  // fragment index of this thread: block f % WB, fragment f / WB
                const int i = f % WB, jj = fb + f / WB;
                if constexpr (kSlowOnly) *(short8_t*)(w_dst(wnx, i) + 8 * jj) = frag16_slow<FMT, ST>(r[i], jj);
                else *(short8_t*)(w_dst(wnx, i) + 8 * jj) = frag16_fast<FMT, ST>(r[i], c0[i], jj);
            }
            // In-order issue: VALU work only overlaps an MFMA if it sits between MFMAs, so each
            // MFMA is followed by a share of the chunk's fragment reads and decode arithmetic.
#pragma unroll
            for (int m = 0; m < MPC; m++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (j < 3 && part == 0) __builtin_amdgcn_sched_group_barrier(0x100, (MT + MN + MPC - 1) / MPC, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (DP > 1) store_x(xn, xr[(u + 1) % DP]);
        if (need) fixup(s + 1, wnx);
        __syncthreads();
    };

    {
        if constexpr (DP == 1) {
            copy_x(0, xs0);
        } else {
            u32x4_t x0[XCH];
            load_x(0, x0);
#pragma unroll
            for (int t = 1; t < DP; t++) load_x(t, xr[t]);
            store_x(xs0, x0);
        }
        RawBlock<FMT> w0[WB];
        load_w(0, w0);
#pragma unroll
        for (int t = 1; t < NS; t++) load_w(t, wr[t - 1]);
        bool need = false;
        decode_store(0, ws0, w0, need);
        if (need) fixup(0, ws0);
    }
    __syncthreads();
    int s = 0;
    for (; s + U - 1 < nstage; s += U) run_stages<0, U>(stage, s);
    run_tail_stages<0, U>(stage, s, nstage);

    QG_GLOBAL float* Y = gptr_mut<float>(p.Y);
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int mn = 0; mn < MN; mn++) {
            const int n = n0 + wn * 32 * MN + 32 * mn + li;
            if (n >= p.N) continue;
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int r = r0 + wm * 32 * MT + mt * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
                if (r < r1) {
                    if constexpr (GR)  // grouped calls may scale each output row
                        Y[(size_t)r * p.N + n] = p.rs ? acc[mt][mn][i] * p.rs[r] : acc[mt][mn][i];
                    else
                        Y[(size_t)r * p.N + n] = acc[mt][mn][i];
                }
            }
        }
}

// s_waitcnt immediate that waits for at most N outstanding vector-memory loads and leaves the LDS /
// scalar and export counters unconstrained (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8).
template <int N>
constexpr int vmcnt_only() {
    static_assert(N >= 0 && N <= 63, "vmcnt");
    return (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}

// ================================================================================================
// Fast GEMM with K split over the wavefronts (Q4 / Q4A / Q8), for shapes too small for the decoded
// tiles: a workgroup owns a 32 MT-token x 32 MN-row output tile (launched with 128 x 64); each of its 4
// wavefronts computes the whole tile over its own quarter of the 64-k stages, from a ring in LDS that
// only it writes and reads -- X (BT rows x 64 k of the stage; chunk c of row r at position
// c ^ ((r / 2) % 8), so the 16-byte fragment reads of 32 rows hit distinct bank quads) and the raw
// code chunks of its weight rows (chunk c of row n at position c ^ ((n / (16 / CPR)) % CPR)), both
// copied by buffer_load ... lds -- so the main loop has no barrier, and the wait before a stage
// counts only this wavefront's copies.  Each B fragment is decoded once in registers (frag16_words,
// or frag16_codes for W-exact) and serves the MT MFMA row tiles; the four f32 partials are added
// through LDS at the end in wavefront order.
//
// Measured on the Q4 prefill (N = K = 4096, T 512, f16): 31.8-33.4 us at 128 x 64, 39-43 us at
// 64 x 128 (two row tiles per decoded fragment: counters showed 369 VALU instructions per wavefront
// and stage for 32 MFMAs, nearly all decode); the 64 x 128 ring kernel it replaces (X and raw codes
// shared by the 4 wavefronts of a 6-stage ring, one barrier per stage, each wavefront on its own
// 32 rows over every stage) ran 32.5-34.5 us, and its Q8 and W-exact launches 46.9 and 49.5 us
// against 39.2 and 44.7 here.  The 14336-row up-projection keeps the 256 x 256 decoded tiles (236 us
// through this kernel against 129).
// Tile 32 MT tokens x 32 MN weight rows; per wavefront and stage BT x 128 bytes of X and BN x 32 (Q8:
// 64) bytes of codes.
template <int SLOT, int I>
__device__ __forceinline__ uint8_t* kz_slot() {
    __shared__ __attribute__((aligned(16))) uint8_t b[4 * SLOT];
    return b;
}

// WX (W-exact, Q4 and Q8 with f16 X): the fragments hold the codes as exact f16 and each block's two
// MFMA steps accumulate into a partial from zero, which the block scale of the lane's weight row
// multiplies into the accumulator in f32.
template <int FMT, int ST, int MT, int MN, int D, bool WX = false>
__global__ __launch_bounds__(kThreads, 1) void gemm_fast_kz_kernel(GemmParams p) {
    static_assert(FMT == FMT_Q4 || FMT == FMT_Q4A || FMT == FMT_Q8, "Q4 / Q4A / Q8 codes");
    static_assert(!WX || (FMT != FMT_Q4A && ST == XT_F16), "W-exact: Q4 / Q8 codes, f16 X");
    static_assert(D >= 2 && D <= 4, "ring depth");
    constexpr int BT = 32 * MT, BN = 32 * MN;
    constexpr int CPR = FMT == FMT_Q8 ? 4 : 2;  // 16-byte code chunks per row and stage
    constexpr int ESZ = FMT == FMT_Q8 ? 4 : 2;  // scale bytes
    constexpr int XB = BT * 128, WB = BN * CPR * 16, SLOT = XB + WB;  // per wavefront and stage
    static_assert(D * 4 * SLOT <= 160 * 1024, "LDS");
    constexpr int XCH = BT / 8;     // X copies (8 rows each) per stage
    constexpr int WCH = BN * CPR / 64;  // raw-code copies (64 lanes x 16 bytes) per stage
    constexpr int LC = XCH + WCH;   // copies to LDS per stage
    static_assert((D - 1) * LC <= 63, "vmcnt range");
    const int r0 = blockIdx.y * BT, r1 = min(p.R, r0 + BT);
    const int n0 = blockIdx.x * BN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, li = lane & 31;
    const int K = p.K, nblk = K >> 5, nstage = (K + 63) >> 6;
    const int s0 = (wave * nstage) >> 2, s1 = ((wave + 1) * nstage) >> 2;  // this wavefront's stages
    const int rows = min(BN, p.N - n0);

    uint16_t* const xbase = (uint16_t*)p.X + (size_t)r0 * K;
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(xbase, 0, (r1 - r0) * K * 2, 0x00020000);
    // X copy i: rows 8 i .. 8 i + 7; lane at row 8 i + lane / 8, position lane % 8 holding chunk
    // (lane % 8) ^ ((row / 2) % 8) = (lane % 8) ^ ((4 i + lane / 16) % 8)
    int xoff[XCH];
#pragma unroll
    for (int i = 0; i < XCH; i++) {
        const int row = 8 * i + (lane >> 3);
        xoff[i] = row * K * 2 + 16 * ((lane & 7) ^ ((row >> 1) & 7));
    }
    const int rowb = FMT == FMT_Q8 ? K : K >> 1;
    const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint8_t*)p.codes + (size_t)n0 * rowb), 0, rows * rowb, 0x00020000);
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint8_t*)p.scales + (size_t)n0 * nblk * ESZ), 0, rows * nblk * ESZ, 0x00020000);
    const int ngr = FMT == FMT_Q4A ? K / p.group : 1;
    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(FMT == FMT_Q4A ? (const uint8_t*)p.offs + (size_t)n0 * ngr * 2 : (const uint8_t*)p.scales), 0,
        FMT == FMT_Q4A ? rows * ngr * 2 : 0, 0x00020000);
    // raw copy i: slots 64 i + lane -> tile row n = slot / CPR, chunk position cs = slot % CPR, holding
    // the row's chunk cs ^ ((n / (16 / CPR)) % CPR) of the stage
    auto swz = [](int n) { return (n / (16 / CPR)) % CPR; };
    int woff[WCH];
#pragma unroll
    for (int i = 0; i < WCH; i++) {
        const int slot = 64 * i + lane;
        const int n = slot / CPR, cs = slot % CPR;
        woff[i] = n * rowb + 16 * (cs ^ swz(n));
    }
    int soff[MN], ooff[MN];
#pragma unroll
    for (int mn = 0; mn < MN; mn++) {
        soff[mn] = (32 * mn + li) * nblk * ESZ;
        ooff[mn] = (32 * mn + li) * ngr * 2;
    }
    struct Scales {
        uint32_t d[MN][2];
        uint32_t m[MN][2];
    };
    auto issue = [&](auto slotc, int st, Scales& sc) __attribute__((always_inline)) {
        constexpr int sl = decltype(slotc)::value;
        asm volatile("" ::: "memory");
        uint8_t* const xd = kz_slot<SLOT, sl>() + wave * SLOT;
        uint8_t* const wd = xd + XB;
        const int sr = min(st, s1 - 1);  // stages past the wavefront's last repeat it
        const int koff = sr * 64 < K ? sr * 128 : 0x40000000;
#pragma unroll
        for (int i = 0; i < XCH; i++) buffer_copy16_lds(xrs, xd + 1024 * i, xoff[i] + koff);
#pragma unroll
        for (int i = 0; i < WCH; i++) buffer_copy16_lds(crs, wd + 1024 * i, woff[i] + 16 * CPR * sr);
#pragma unroll
        for (int mn = 0; mn < MN; mn++)
#pragma unroll
            for (int b = 0; b < 2; b++) {
                const int blk = 2 * sr + b;
                if constexpr (FMT == FMT_Q8)
                    sc.d[mn][b] = __builtin_amdgcn_raw_buffer_load_b32(srs, soff[mn], 4 * blk, 0);
                else
                    sc.d[mn][b] = __builtin_amdgcn_raw_buffer_load_b16(srs, soff[mn], 2 * blk, 0);
                if constexpr (FMT == FMT_Q4A)
                    sc.m[mn][b] = __builtin_amdgcn_raw_buffer_load_b16(ors, ooff[mn], 2 * ((32 * blk) / p.group), 0);
            }
    };

    f32x16_t acc[MT][MN];
#pragma unroll
    for (int a = 0; a < MT; a++)
#pragma unroll
        for (int b = 0; b < MN; b++)
#pragma unroll
            for (int i = 0; i < 16; i++) acc[a][b][i] = 0.f;

    auto mfma = [&](const short8_t& a, const short8_t& b, f32x16_t& c) {
        if constexpr (ST == XT_F16)
            c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
        else
            c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    };
    Scales scr[D];

    // The four MFMA steps of a stage; step j: X columns 16 j .. 16 j + 15, block j / 2 of every row
    // (Q4 / Q4A: one 16-byte chunk per block, low nibbles for even j, high for odd j; Q8: chunk j).
    auto body = [&](auto uc, auto fastc, int s, const float (&d)[MN][2], const float (&c0)[MN][2],
                    const float (&mm)[MN][2], const uint32_t (&dh)[MN][2]) __attribute__((always_inline)) {
        constexpr bool FAST = decltype(fastc)::value;
        const uint8_t* const xb = kz_slot<SLOT, decltype(uc)::value>() + wave * SLOT;
        const uint16_t* const xsb = (const uint16_t*)xb;
        const uint8_t* const wsb = xb + XB;
        short8_t A[2][MT], B[2][MN];
        uint2 raw[MN];
        f32x16_t part[MT][MN];  // WX: the current block's partial
        auto frags_a = [&](int j, short8_t (&Ao)[MT]) __attribute__((always_inline)) {
            const uint16_t* xa = xsb + li * 64 + 8 * ((2 * j + g) ^ ((li >> 1) & 7));
#pragma unroll
            for (int mt = 0; mt < MT; mt++) Ao[mt] = *(const short8_t*)(xa + mt * 32 * 64);
        };
        auto read_raw = [&](int ch) __attribute__((always_inline)) {
#pragma unroll
            for (int mn = 0; mn < MN; mn++) {
                const int n = 32 * mn + li;
                raw[mn] = *(const uint2*)(wsb + 16 * (CPR * n + (ch ^ swz(n))) + 8 * g);
            }
        };
        auto decode = [&](int q, short8_t (&Bo)[MN]) __attribute__((always_inline)) {
            const int b = q >> 1;
#pragma unroll
            for (int mn = 0; mn < MN; mn++) {
                uint32_t c[2];
                if constexpr (FMT == FMT_Q8) {
                    c[0] = keep_u32(raw[mn].x ^ 0x80808080u);
                    c[1] = keep_u32(raw[mn].y ^ 0x80808080u);
                } else if (q & 1) {
                    c[0] = keep_u32((raw[mn].x >> 4) & 0x0F0F0F0Fu);
                    c[1] = keep_u32((raw[mn].y >> 4) & 0x0F0F0F0Fu);
                } else {
                    c[0] = keep_u32(raw[mn].x & 0x0F0F0F0Fu);
                    c[1] = keep_u32(raw[mn].y & 0x0F0F0F0Fu);
                }
                if constexpr (WX) Bo[mn] = frag16_codes<FMT>(c);
                else if constexpr (FAST) Bo[mn] = frag16_words<FMT, ST>(c, d[mn][b], dh[mn][b], c0[mn][b]);
                else Bo[mn] = frag16_words_slow<FMT, ST>(c, d[mn][b], mm[mn][b]);
            }
        };
        frags_a(0, A[0]);
        read_raw(0);
        decode(0, B[0]);
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int cur = q & 1, nx = cur ^ 1;
            if (q + 1 < 4) {
                frags_a(q + 1, A[nx]);
                if constexpr (FMT == FMT_Q8) read_raw(q + 1);  // each step its own chunk
                else if (q == 1) read_raw(1);                  // the second block's chunks
            }
            if constexpr (WX) {
#pragma unroll
                for (int mt = 0; mt < MT; mt++)
#pragma unroll
                    for (int mn = 0; mn < MN; mn++) {
                        if ((q & 1) == 0) {
                            f32x16_t z;
#pragma unroll
                            for (int i = 0; i < 16; i++) z[i] = 0.f;
                            part[mt][mn] = z;
                        }
                        mfma(A[cur][mt], B[cur][mn], part[mt][mn]);
                        if (q & 1) {
#pragma unroll
                            for (int i = 0; i < 16; i++)
                                acc[mt][mn][i] = fmaf(part[mt][mn][i], d[mn][q >> 1], acc[mt][mn][i]);
                        }
                    }
            } else {
#pragma unroll
                for (int mt = 0; mt < MT; mt++)
#pragma unroll
                    for (int mn = 0; mn < MN; mn++) mfma(A[cur][mt], B[cur][mn], acc[mt][mn]);
            }
            if (q + 1 < 4) decode(q + 1, B[nx]);
        }
    };
    auto stage = [&](auto uc, int s) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;  // (s - s0) % D
        if constexpr (D == 2) {
            // Everything outstanding is this stage's (issued one stage ago): wait for all of it, then
            // issue the next stage.  Issuing first would put the next stage's scale loads into
            // registers behind its copies, and a copy count that is safe with mixed completion order
            // would then wait for part of the stage just issued (measured: 41% of the cycles waiting).
            __builtin_amdgcn_s_waitcnt(vmcnt_only<0>());
            asm volatile("" ::: "memory");
            issue(std::integral_constant<int, (u + 1) % D>{}, s + 1, scr[(u + 1) % D]);
        } else {
            issue(std::integral_constant<int, (u + D - 1) % D>{}, s + D - 1, scr[(u + D - 1) % D]);
            // this stage's copies have landed: D - 1 later stages' copies were issued since (copies to
            // LDS complete in issue order among themselves; the scale loads into registers are not
            // counted)
            __builtin_amdgcn_s_waitcnt(vmcnt_only<(D - 1) * LC>());
            asm volatile("" ::: "memory");
        }
        __builtin_amdgcn_sched_barrier(0);
        float d[MN][2], c0[MN][2], mm[MN][2];
        uint32_t dh[MN][2];
        bool fast = true;
#pragma unroll
        for (int mn = 0; mn < MN; mn++)
#pragma unroll
            for (int b = 0; b < 2; b++) {
                const bool valid = 2 * s + b < nblk;  // a K tail block decodes as zeros
                const uint32_t db = valid ? scr[u].d[mn][b] : 0u;
                dh[mn][b] = db & 0xFFFFu;
                d[mn][b] = FMT == FMT_Q8 ? __uint_as_float(db) : f16_to_f32((uint16_t)db);
                mm[mn][b] = FMT == FMT_Q4A ? (valid ? bf16_to_f32((uint16_t)scr[u].m[mn][b]) : 0.f) : 0.f;
                RawBlock<FMT> rb{};
                rb.d = d[mn][b];
                rb.m = mm[mn][b];
                bool f;
                c0[mn][b] = block_c0<FMT>(rb, f);
                if constexpr (!(FMT == FMT_Q4 && ST == XT_F16)) fast = fast && (f || !valid);
            }
        if constexpr (WX || (FMT == FMT_Q4 && ST == XT_F16)) {
            body(uc, std::true_type{}, s, d, c0, mm, dh);
        } else {
            if (__all(fast)) body(uc, std::true_type{}, s, d, c0, mm, dh);
            else body(uc, std::false_type{}, s, d, c0, mm, dh);
        }
    };
    if (s1 > s0) {
        auto prologue = [&](auto tc) __attribute__((always_inline)) {
            constexpr int t = decltype(tc)::value;
            issue(tc, s0 + t, scr[t]);
        };
        run_stages_c<0, D - 1>(prologue);
        int s = s0;
        for (; s + D <= s1; s += D) run_stages<0, D>(stage, s);
        // the remaining s1 - s < D stages keep their slot numbering (slot (s - s0) % D)
        run_tail_stages<0, D + 1>(stage, s, s1);
    }

    // The four partial tiles added in wavefront order through slot 0, RT accumulator tiles a round:
    // every wavefront writes its partials of the round's tiles, then wavefront w adds and stores the
    // round's tiles t with t % 4 == w.
    __builtin_amdgcn_s_waitcnt(0);  // the ring's last (repeated) copies have landed before slot 0 is reused
    __syncthreads();
    constexpr int NT = MT * MN;
    constexpr int RT = (4 * SLOT) / (4 * 4096) < NT ? (4 * SLOT) / (4 * 4096) : NT;  // 4 KiB per tile and wavefront
    static_assert(RT >= 1, "reduction round");
    float* const red = (float*)kz_slot<SLOT, 0>();
    QG_GLOBAL float* Y = gptr_mut<float>(p.Y);
#pragma unroll
    for (int t0 = 0; t0 < NT; t0 += RT) {
#pragma unroll
        for (int t = t0; t < t0 + RT && t < NT; t++)
#pragma unroll
            for (int i = 0; i < 16; i += 4)
                *(float4*)(red + (((wave * RT + (t - t0)) * 4 + i / 4) * 64 + lane) * 4) =
                    make_float4(acc[t / MN][t % MN][i], acc[t / MN][t % MN][i + 1], acc[t / MN][t % MN][i + 2],
                                acc[t / MN][t % MN][i + 3]);
        __syncthreads();
#pragma unroll
        for (int t = t0; t < t0 + RT && t < NT; t++) {
            if (t % 4 != wave) continue;
            const int mt = t / MN, mn = t % MN;
            const int n = n0 + 32 * mn + li;
#pragma unroll
            for (int i = 0; i < 16; i += 4) {
                float4 v = *(const float4*)(red + (((0 * RT + (t - t0)) * 4 + i / 4) * 64 + lane) * 4);
#pragma unroll
                for (int w = 1; w < 4; w++) {
                    const float4 q = *(const float4*)(red + (((w * RT + (t - t0)) * 4 + i / 4) * 64 + lane) * 4);
                    v.x += q.x;
                    v.y += q.y;
                    v.z += q.z;
                    v.w += q.w;
                }
                const float tv[4] = {v.x, v.y, v.z, v.w};
                if (n < p.N) {
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const int r = r0 + mt * 32 + 8 * ((i + j) >> 2) + 4 * g + ((i + j) & 3);
                        if (r < r1) Y[(size_t)r * p.N + n] = tv[j];
                    }
                }
            }
        }
        __syncthreads();
    }
}

// ================================================================================================
// Exact mode: f32 MFMA (v_mfma_f32_32x32x2_f32), f32 accumulation; X f32, f16 or bf16 widened.
// CV: the convolution (page "oxinfer 0.0.5 src/metal.rs", SHADER_SRC conv_body and norm4): the X tile
// of output pixel r and 8 values of K starting at k is the image's channel slice ci .. ci + 7 of tap
// (ky, kx) = divmod(k / cin, ksz) (cin % 32 == 0, so a slice never crosses a tap) at input pixel
// (oy * stride + ky - pad, ox * stride + kx - pad), zeros outside the image; with normalisation the
// loaded values are normalised (and SiLU applied) when they are stored to LDS, after the stage's
// MFMAs, so the loads keep their latency hidden as in the GEMM.
// Per-channel normalisation parameters of the convolution in LDS (cin <= kConvLdsCin): group norm
// keeps mean_c, rstd_c * gamma_c and beta_c; layer norm gamma_c and beta_c (its (mean, rstd) pair
// is per input pixel and travels with the chunk's loads).
constexpr int kConvLdsCin = 1024;
__device__ __forceinline__ float* conv_norm_lds() {
    __shared__ __attribute__((aligned(16))) float b[3 * kConvLdsCin];
    return b;
}

// SiLU as y / (1 + exp(-y)) with the hardware exponential and reciprocal (a few ulp of the result;
// large negative y give exp = inf and the result -0).
__device__ __forceinline__ float conv_silu(float y) { return y * __builtin_amdgcn_rcpf(1.0f + __expf(-y)); }

template <int FMT, int XT, int MT, int MN, bool CV = false>
__global__ __launch_bounds__(kThreads) void gemm_exact_kernel(GemmParams p, bool grouped, ConvParams cv) {
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
    int cy[XCH], cx[XCH];  // CV: input position of tap (0, 0) for the chunk's output pixel
    int cq[XCH], cc[XCH];  // CV: input pixel and channel of the chunk loaded last (cq < 0: zeros)
    float cm[XCH], cr[XCH];  // CV, layer norm: (mean, rstd) of that input pixel
    // CV: tap (ky, kx) and channel ci of the chunk's k in the stage load_x takes next; load_x runs
    // for stages 0, 1, 2, ... in order, so they advance by 64 channels a call with no division
    int tky[XCH], tkx[XCH], tci[XCH];
#pragma unroll
    for (int i = 0; i < XCH; i++) {
        const int c = tid + i * kThreads;
        xrow[i] = x_row_of(p, min(r0 + c / 8, r1 - 1));
        if constexpr (CV) {
            const int oy = xrow[i] / cv.ow, ox = xrow[i] - oy * cv.ow;
            cy[i] = oy * cv.stride - cv.pad;
            cx[i] = ox * cv.stride - cv.pad;
            const int k0 = 8 * (c & 7), tap = k0 / cv.cin;
            tci[i] = k0 - tap * cv.cin;
            tky[i] = tap / cv.ksz;
            tkx[i] = tap - tky[i] * cv.ksz;
        }
    }
    // CV with normalisation and cin <= kConvLdsCin: the per-channel parameters once per workgroup
    bool norm_lds = false;
    float* nl = nullptr;
    if constexpr (CV) {
        norm_lds = cv.norm != 0 && cv.cin <= kConvLdsCin;
        if (norm_lds) {
            nl = conv_norm_lds();
            for (int ch = tid; ch < cv.cin; ch += kThreads) {
                if (cv.norm == 1) {
                    const int sg = ch / cv.cpg;
                    nl[ch] = cv.stats[2 * sg];
                    nl[kConvLdsCin + ch] = cv.stats[2 * sg + 1] * cv.gb[ch];
                } else {
                    nl[kConvLdsCin + ch] = cv.gb[ch];
                }
                nl[2 * kConvLdsCin + ch] = cv.gb[cv.cin + ch];
            }
            __syncthreads();
        }
    }
    auto load_x = [&](int s, float (&v)[XCH][8]) {
#pragma unroll
        for (int i = 0; i < XCH; i++) {
            const int c = tid + i * kThreads;
            const int k = s * 64 + 8 * (c & 7);
            if constexpr (CV) {
                cq[i] = -1;
                if (xrow[i] >= 0 && k < K) {
                    const int iy = cy[i] + tky[i], ix = cx[i] + tkx[i];
                    if ((unsigned)iy < (unsigned)cv.H && (unsigned)ix < (unsigned)cv.W) {
                        cq[i] = iy * cv.W + ix;
                        cc[i] = tci[i];
                    }
                }
                // the next stage: 64 channels on, past at most two taps (cin >= 32)
                tci[i] += 64;
#pragma unroll
                for (int w = 0; w < 2; w++)
                    if (tci[i] >= cv.cin) {
                        tci[i] -= cv.cin;
                        if (++tkx[i] == cv.ksz) {
                            tkx[i] = 0;
                            ++tky[i];
                        }
                    }
                if (cq[i] >= 0 && cv.norm == 2) {
                    cm[i] = cv.stats[2 * cq[i]];
                    cr[i] = cv.stats[2 * cq[i] + 1];
                }
                if (cq[i] >= 0)
                    x_load8<XT_F32>(p.X, (size_t)cq[i] * cv.cin + cc[i], v[i]);
                else
#pragma unroll
                    for (int j = 0; j < 8; j++) v[i][j] = 0.f;
            } else {
                if (xrow[i] >= 0 && k < K)
                    x_load8<XT>(p.X, (size_t)xrow[i] * K + k, v[i]);
                else
#pragma unroll
                    for (int j = 0; j < 8; j++) v[i][j] = 0.f;
            }
        }
    };
    auto store_x = [&](int buf, float (&v)[XCH][8]) {
#pragma unroll
        for (int i = 0; i < XCH; i++) {
            const int c = tid + i * kThreads;
            if constexpr (CV) {
                // norm4: y = (v - mean) * rstd * gamma + beta, then SiLU; padding taps stay zero
                if (norm_lds && cq[i] >= 0) {
                    const float* pa = nl + kConvLdsCin + cc[i];
                    const float* pb = nl + 2 * kConvLdsCin + cc[i];
                    const float4 a0 = *(const float4*)pa, a1 = *(const float4*)(pa + 4);
                    const float4 b0 = *(const float4*)pb, b1 = *(const float4*)(pb + 4);
                    const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                    const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
                    if (cv.norm == 1) {
                        const float4 m0 = *(const float4*)(nl + cc[i]), m1 = *(const float4*)(nl + cc[i] + 4);
                        const float mv[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
                        for (int j = 0; j < 8; j++) v[i][j] = fmaf(v[i][j] - mv[j], av[j], bv[j]);
                    } else {
#pragma unroll
                        for (int j = 0; j < 8; j++) v[i][j] = fmaf((v[i][j] - cm[i]) * cr[i], av[j], bv[j]);
                    }
                    if (cv.silu)
#pragma unroll
                        for (int j = 0; j < 8; j++) v[i][j] = conv_silu(v[i][j]);
                } else if (cv.norm && cq[i] >= 0) {
                    // cin past the LDS staging: parameters straight from memory
#pragma unroll
                    for (int j = 0; j < 8; j++) {
                        const int ch = cc[i] + j;
                        const int si = cv.norm == 1 ? ch / cv.cpg : cq[i];
                        const float y = fmaf((v[i][j] - cv.stats[2 * si]) * cv.stats[2 * si + 1], cv.gb[ch],
                                             cv.gb[cv.cin + ch]);
                        v[i][j] = cv.silu ? conv_silu(y) : y;
                    }
                }
            }
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

    // Software pipeline: stage s runs its MFMAs on the decoded block wv while the raw block of stage
    // s + 1 (wr) is decoded four values at a time between them and the raw block of stage s + 2
    // loads; blocks past K decode with zero scale and offset (zeros).
    float xv[XCH][8];
    RawBlock<FMT> wr[MN];
    float wv[MN][32];
    load_x(0, xv);
    {
        RawBlock<FMT> w0[MN];
        load_w(0, w0);
        load_w(1, wr);
        const bool valid0 = g < nblk;
#pragma unroll
        for (int mn = 0; mn < MN; mn++) {
            block_clear_if<FMT>(w0[mn], valid0);
            block_to_f32<FMT>(w0[mn], wv[mn]);
        }
    }
    store_x(0, xv);
    __syncthreads();

    for (int s = 0; s < nstage; s++) {
        const int buf = s & 1;
        const bool more = s + 1 < nstage;
        RawBlock<FMT> wn[MN];
        if (more) load_x(s + 1, xv);
        load_w(s + 2, wn);
        const bool valid = 2 * (s + 1) + g < nblk;
        RawBlock<FMT> rn[MN];
#pragma unroll
        for (int mn = 0; mn < MN; mn++) {
            rn[mn] = wr[mn];
            block_clear_if<FMT>(rn[mn], valid);
        }
        float wnv[MN][32];
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
#pragma unroll
            for (int mn = 0; mn < MN; mn++) {
                float t[4];
                block_quad_f32<FMT>(rn[mn], q, t);
#pragma unroll
                for (int b = 0; b < 4; b++) wnv[mn][4 * q + b] = t[b];
            }
        }
        if (more) store_x(buf ^ 1, xv);
#pragma unroll
        for (int mn = 0; mn < MN; mn++) {
            wr[mn] = wn[mn];
#pragma unroll
            for (int j = 0; j < 32; j++) wv[mn][j] = wnv[mn][j];
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

template <int FMT, int ST, int WM, int MT, int MN, int DP, bool GR = false>
static void fast_lds_launch(const GemmParams& p, hipStream_t s) {
    constexpr int BT = 32 * MT * WM, BN = 32 * MN * (4 / WM);
    dim3 grid((p.N + BN - 1) / BN, grid_rows(p, GR, BT));
    hipLaunchKernelGGL((gemm_fast_lds_kernel<FMT, ST, WM, MT, MN, DP, GR>), grid, dim3(kThreads), 0, s, p);
}


template <int FMT, int ST, int MT, int MN, int D, bool WX = false>
static void fast_kz_launch(const GemmParams& p, hipStream_t s) {
    dim3 grid((p.N + 32 * MN - 1) / (32 * MN), (p.R + 32 * MT - 1) / (32 * MT));
    hipLaunchKernelGGL((gemm_fast_kz_kernel<FMT, ST, MT, MN, D, WX>), grid, dim3(kThreads), 0, s, p);
}

template <int FMT, int ST>
static void fast_pick(const GemmParams& p, bool grouped, hipStream_t s) {
    // Grouped launches: 32-row tiles (MoE segments are short), 128 weight rows (three workgroups
    // per CU; measured 13% faster than 256 rows on the MoE block), 4-deep prefetch; gathered X rows
    // (row_src) take the register-direct kernel.
    if constexpr (!blk16<FMT>) {  // 16-element blocks have no grouped calls
        if (grouped) {
            if (p.row_src) return fast_launch<FMT, ST, 1, 2>(p, grouped, s);
            return fast_lds_launch<FMT, ST, 1, 1, 1, 4, true>(p, s);
        }
    }
    // The largest tile that still gives about one workgroup per CU: big tiles amortize each
    // decoded weight over more tokens and each staged X row over more weight rows.
    auto wgs = [&](int bt, int bn) { return (long)((p.N + bn - 1) / bn) * ((p.R + bt - 1) / bt); };
    if (wgs(256, 256) >= 200) return fast_lds_launch<FMT, ST, 2, 4, 4, 1>(p, s);
    if (wgs(128, 256) >= 200) return fast_lds_launch<FMT, ST, 2, 2, 4, 4>(p, s);
    if (wgs(128, 128) >= 200) return fast_lds_launch<FMT, ST, 2, 2, 2, 4>(p, s);
    // Smaller shapes: 128 x 64 tiles with K split over the wavefronts (Q4 prefill N = K = 4096, T 512:
    // 31.8 us; Q8 39.2 us); Q8A (its per-block offsets are not in that kernel's ring) the 128 x 128
    // decoded tiles
    if constexpr (FMT == FMT_Q8A || blk16<FMT>) return fast_lds_launch<FMT, ST, 2, 2, 2, 4>(p, s);
    else return fast_kz_launch<FMT, ST, 4, 2, 2>(p, s);
}

hipError_t launch_gemm_fast_wexact(int fmt, const GemmParams& p, hipStream_t s) {
    // 128 x 64 tiles with K split over the wavefronts, whatever the shape
    if (fmt == FMT_Q4) fast_kz_launch<FMT_Q4, XT_F16, 4, 2, 2, true>(p, s);
    else if (fmt == FMT_Q8) fast_kz_launch<FMT_Q8, XT_F16, 4, 2, 2, true>(p, s);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_gemm_fast(int fmt, int st, const GemmParams& p, bool grouped, hipStream_t s) {
    if (st == XT_F16) {
        if (fmt == FMT_Q4) fast_pick<FMT_Q4, XT_F16>(p, grouped, s);
        else if (fmt == FMT_Q4A) fast_pick<FMT_Q4A, XT_F16>(p, grouped, s);
        else if (fmt == FMT_Q8A) fast_pick<FMT_Q8A, XT_F16>(p, grouped, s);
        else if (fmt == FMT_Q8A16 && !grouped) fast_pick<FMT_Q8A16, XT_F16>(p, false, s);
        else if (fmt == FMT_Q8A16) return hipErrorInvalidValue;
        else fast_pick<FMT_Q8, XT_F16>(p, grouped, s);
    } else {
        if (fmt == FMT_Q4) fast_pick<FMT_Q4, XT_BF16>(p, grouped, s);
        else if (fmt == FMT_Q4A) fast_pick<FMT_Q4A, XT_BF16>(p, grouped, s);
        else if (fmt == FMT_Q8A) fast_pick<FMT_Q8A, XT_BF16>(p, grouped, s);
        else if (fmt == FMT_Q8A16 && !grouped) fast_pick<FMT_Q8A16, XT_BF16>(p, false, s);
        else if (fmt == FMT_Q8A16) return hipErrorInvalidValue;
        else fast_pick<FMT_Q8, XT_BF16>(p, grouped, s);
    }
    return hipGetLastError();
}

template <int FMT, int XT, int MT, int MN>
static void exact_launch(const GemmParams& p, bool grouped, hipStream_t s) {
    dim3 grid((p.N + 128 * MN - 1) / (128 * MN), grid_rows(p, grouped, 32 * MT));
    hipLaunchKernelGGL((gemm_exact_kernel<FMT, XT, MT, MN>), grid, dim3(kThreads), 0, s, p, grouped, ConvParams{});
}

template <int FMT, int XT>
static void exact_pick(const GemmParams& p, bool grouped, hipStream_t s) {
    if (grouped) return exact_launch<FMT, XT, 1, 1>(p, grouped, s);
    // 32-row tiles unless 64-row tiles still give four workgroups per CU: with one workgroup per
    // CU each SIMD holds a single wavefront and every barrier and LDS wait idles its matrix core.
    // Measured on the Q4 prefill (N = K = 4096, T 512): 176 us with 32-row tiles (512 workgroups)
    // against 198 us with 64-row tiles (256).
    const long mid = (long)((p.N + 127) / 128) * ((p.R + 63) / 64);
    if (mid >= 1024) return exact_launch<FMT, XT, 2, 1>(p, grouped, s);
    return exact_launch<FMT, XT, 1, 1>(p, grouped, s);
}

template <int FMT>
static void exact_xt(int xt, const GemmParams& p, bool grouped, hipStream_t s) {
    if (xt == XT_F32) exact_pick<FMT, XT_F32>(p, grouped, s);
    else if (xt == XT_F16) exact_pick<FMT, XT_F16>(p, grouped, s);
    else exact_pick<FMT, XT_BF16>(p, grouped, s);
}

template <int FMT>
static void conv_pick(const GemmParams& p, const ConvParams& cv, hipStream_t s) {
    // the exact kernel's tile rule
    const long mid = (long)((p.N + 127) / 128) * ((p.R + 63) / 64);
    if (mid >= 1024) {
        dim3 grid((p.N + 127) / 128, (p.R + 63) / 64);
        hipLaunchKernelGGL((gemm_exact_kernel<FMT, XT_F32, 2, 1, true>), grid, dim3(kThreads), 0, s, p, false, cv);
    } else {
        dim3 grid((p.N + 127) / 128, (p.R + 31) / 32);
        hipLaunchKernelGGL((gemm_exact_kernel<FMT, XT_F32, 1, 1, true>), grid, dim3(kThreads), 0, s, p, false, cv);
    }
}

hipError_t launch_conv_exact(int fmt, const GemmParams& p, const ConvParams& cv, hipStream_t s) {
    if (fmt == FMT_Q4) conv_pick<FMT_Q4>(p, cv, s);
    else if (fmt == FMT_Q8) conv_pick<FMT_Q8>(p, cv, s);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_gemm_exact(int fmt, int xt, const GemmParams& p, bool grouped, hipStream_t s) {
    if (fmt == FMT_Q4) exact_xt<FMT_Q4>(xt, p, grouped, s);
    else if (fmt == FMT_Q4A) exact_xt<FMT_Q4A>(xt, p, grouped, s);
    else if (fmt == FMT_Q8A) exact_xt<FMT_Q8A>(xt, p, grouped, s);
    else if (fmt == FMT_Q8A16) exact_xt<FMT_Q8A16>(xt, p, grouped, s);
    else exact_xt<FMT_Q8>(xt, p, grouped, s);
    return hipGetLastError();
}

}  // namespace qg
