// qg_moe.hip -- the expert-row streaming kernel of grouped matmuls with short row segments (the
// expert block of a decode step), with the per-row f16 scaling of X and SwiGLU fused in.
//
// Prior art: page "oxinfer 0.0.5 src/metal.rs", Backend::moe (rows of every expert gathered through
// a row map, gate|up, then SiLU(gate) * up, then down, then the weighted combine) and MMA_SHADER_SRC
// (x_half and silu_half: a per-row power-of-two scale before narrowing to f16); page
// "cortiq-engine 0.8.41 src/gpu_metal/clover.rs", q4rows (a narrow kernel of at most 8 rows for
// expert panels).  The layout here:
//
//  * blockIdx.y is the expert e; its X rows are the segment seg_off[e] .. seg_off[e+1] - 1, taken
//    in chunks of at most 4 rows.  Every wavefront owns a contiguous range of the expert's weight
//    rows and streams it on its own, with no barrier: lane c holds byte chunk c of every row, 16
//    bytes (Q4 / Q4A: one 32-value block; Q8: half a block) or, in f32 arithmetic when K is a
//    multiple of 96 up to 1536, 12 bytes (Q4 / Q4A: 24 values over at most two blocks, so that
//    K = 1536 fills all 64 lanes instead of 48), so K <= 64 chunks.  The chunk's X values of each segment row stay in
//    registers for the whole range.
//  * The weight rows go through a per-wavefront ring in LDS, 4 rows a stage, 3 stages: the code bytes
//    (one instruction per row) and the block scales and offsets (one instruction for the stage) are
//    copied by buffer_load ... lds, holding no registers; two stages stay in flight while one is
//    computed.
//  * Arithmetic.  F32: the signed codes as f32, f32 FMA with x, then the block scale times the f32
//    partial (and the Q4A offset times the chunk's x sum).  DOT2 (fast mode with f16 X): two codes
//    per mask instruction as exact f16 subnormals, v_dot2 with pairs of x into an f32 partial, scaled
//    the same way: the weights are never rounded (the W-exact form of the fast path), only X is f16.
//  * The 4 x NT partials of a stage (weight row, X row) are summed over the wavefront at once by a
//    transposing reduction (lane-half and row swaps, then DPP), which leaves each total in its own
//    lanes; SwiGLU and the stores then run once per stage.
//  * Fused X scaling (XH, f32 X in fast mode): each X row is scaled in registers by the x_half rule
//    (the wavefront's maximum over the row, a power of two putting it in [2^13, 2^14)), rounded to
//    f16, and the inverse scale is applied to the outputs -- what x_half followed by the f16-X
//    launch computes, without the f16 copy of X.
//  * In fast mode (Q4 / Q8) each X row of a chunk is converted once per workgroup: wavefront t
//    converts row t into LDS and, after one barrier, every wavefront reads all rows.  Per wavefront
//    this cut the block from 180 to 157 us (the conversion had been repeated by every wavefront of
//    every workgroup of the expert).  A wavefront with no rows of its own still takes part in the
//    barriers.
//  * SwiGLU epilogue (gate|up matrices of 2I rows): the wavefront takes gate row j and up row I + j
//    together and stores a = g / (1 + exp(-g)) * u, so the 2I-wide intermediate is never written.
// Measured on the 128-expert top-8 block (32 tokens, H 2048, I 1536, Q4), whole block in exact / fast
// mode: the K-split GEMV and the MFMA tile kernel it replaces 259 / 228 us; rows through registers
// one batch ahead 234 / 205 us; the LDS ring 217 / 187 us (depth 4) and 214 / 186 (depth 3, kept),
// 221 / 190 at depth 5.  Workgroups per expert: about 4 resident rounds (19 per expert on this block)
// measured best, 207 / 181 us against 211 / 193 at 6 rounds, 220 / 187 at 3.5, 215 / 188 at 4.5 and
// 217 / 193 at 5 (one box, one process each): more workgroups repeat the fused X scaling of every
// segment row in more wavefronts.

#include <algorithm>
#include <type_traits>

#include "qg_device.hpp"
#include "qg_internal.hpp"

namespace qg {

enum { AR_F32 = 0, AR_DOT2 = 1 };
enum { EPI_PLAIN = 0, EPI_SWIGLU = 1 };

constexpr int kRowsWaves = 4;  // wavefronts per workgroup
constexpr int kRowsSeg = 4;    // X rows per segment chunk
constexpr int kRowsBatch = 4;  // weight rows per load batch

constexpr int kRowsRing = 3;   // ring depth (batches in flight per wavefront: kRowsRing - 1)

// f(integral_constant<I>) for I .. U-1
template <int I, int U, class F>
__device__ __forceinline__ void rows_run(F& f) {
    if constexpr (I < U) {
        f(std::integral_constant<int, I>{});
        rows_run<I + 1, U>(f);
    }
}
// f(integral_constant<I>, s + I) for I .. U-1
template <int I, int U, class F>
__device__ __forceinline__ void rows_run_from(F& f, int s) {
    f(std::integral_constant<int, I>{}, s + I);
    if constexpr (I + 1 < U) rows_run_from<I + 1, U>(f, s);
}
// the same for the stages s + I < n only
template <int I, int U, class F>
__device__ __forceinline__ void rows_run_tail(F& f, int s, int n) {
    if (s + I < n) {
        f(std::integral_constant<int, I>{}, s + I);
        if constexpr (I + 1 < U) rows_run_tail<I + 1, U>(f, s, n);
    }
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Lane chunk of CW 4-byte words (CB = 4 CW bytes) of a weight row.  Word i of chunk c starts at row
// byte CB c + 4 i; for Q4 / Q4A it holds the codes of block b_i = (CB c + 4 i) / 16 at in-block
// positions j_i .. j_i + 3 (low nibbles) and 16 + j_i .. 16 + j_i + 3 (high nibbles), j_i =
// (CB c + 4 i) % 16; for Q8 the codes of elements CB c + 4 i .. + 3.  Values are indexed by word:
// value 4 i + j is the low nibble (Q8: the byte) of byte j of word i, value 4 CW + 4 i + j its high
// nibble.  CW = 4: one whole Q4 block (half a Q8 block), values in k order.  CW = 3 (Q4 / Q4A): the
// words span at most two blocks, A = b_0 and B = b_2, word 1 lying in one of them.
template <int FMT, int CW>
struct RowsChunk {
    static_assert(CW == 4 || (CW == 3 && FMT != FMT_Q8), "chunk words");
    static constexpr int CB = 4 * CW;
    static constexpr int V = FMT == FMT_Q8 ? CB : 2 * CB;  // values per chunk
};
// k of value 4 i (the first low-nibble value of word i) of chunk c; its high-nibble values sit 16 on
template <int FMT, int CW>
__device__ __forceinline__ int chunk_word_k(int c, int i) {
    const int o = 4 * CW * c + 4 * i;
    return FMT == FMT_Q8 ? o : 32 * (o >> 4) + (o & 15);
}

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// The chunk's codes as the factors of x (F32 arithmetic): Q4 / Q4A 16 (nibble - 8), the nibble moved
// to the byte's high half with its top bit flipped and read as a signed byte (elements 0..15 from the
// low nibbles, 16..31 from the high ones); Q8 q.
template <int FMT, int CW>
__device__ __forceinline__ void codes_f32(const uint32_t (&w)[CW], float (&c)[RowsChunk<FMT, CW>::V]) {
    if constexpr (FMT == FMT_Q8) {
#pragma unroll
        for (int i = 0; i < 4 * CW; i++) c[i] = (float)(int8_t)(w[i >> 2] >> (8 * (i & 3)));
    } else {
#pragma unroll
        for (int i = 0; i < 4 * CW; i++) {
            c[i] = (float)(int8_t)((((w[i >> 2] << 4) & 0xF0F0F0F0u) ^ 0x80808080u) >> (8 * (i & 3)));
            c[4 * CW + i] = (float)(int8_t)(((w[i >> 2] & 0xF0F0F0F0u) ^ 0x80808080u) >> (8 * (i & 3)));
        }
    }
}

// DOT2 arithmetic: sum_i u_i x_i over the chunk with the codes read as unsigned integers u (Q4 the
// nibble, Q8 q + 128, the byte with its top bit flipped) and x as f16 pairs.  A code is masked in
// place into the low bits of a 16-bit half, which is then the f16 subnormal u * 2^-24 (low nibble, a
// whole Q8 byte) or u * 2^-20 (high nibble) -- exact, with no conversion instruction: one mask makes
// two codes, and v_dot2 multiplies them exactly into an f32 partial per scale, which is scaled back by
// 2^24 / 2^20 (exact).  Pairs: word j of the chunk masked with 0x000F000F (0x00FF00FF for Q8) holds
// the codes of bytes 0 and 2, the word shifted right by 8 those of bytes 1 and 3; x is packed to
// match (rows_chunk: xh[4j..4j+3] = values (4j, 4j+2), (4j+1, 4j+3), (4CW+4j, 4CW+4j+2),
// (4CW+4j+1, 4CW+4j+3) for Q4; xh[2j], xh[2j+1] = (4j, 4j+2), (4j+1, 4j+3) for Q8).  The caller
// subtracts the code offset (8 or 128) times the chunk's x sum.
template <int FMT, int CW>
__device__ __forceinline__ float dot_codes_h2(const uint32_t (&w4)[CW], const uint32_t* xh) {
    float pa = 0.f, pb = 0.f;
#pragma unroll
    for (int j = 0; j < CW; j++) {
        if constexpr (FMT == FMT_Q8) {
            const uint32_t u = w4[j] ^ 0x80808080u, s = u >> 8;
            pa = __builtin_amdgcn_fdot2(as_h2(u & 0x00FF00FFu), as_h2(xh[2 * j]), pa, false);
            pb = __builtin_amdgcn_fdot2(as_h2(s & 0x00FF00FFu), as_h2(xh[2 * j + 1]), pb, false);
        } else {
            const uint32_t w = w4[j], s = w >> 8;
            pa = __builtin_amdgcn_fdot2(as_h2(w & 0x000F000Fu), as_h2(xh[4 * j]), pa, false);
            pa = __builtin_amdgcn_fdot2(as_h2(s & 0x000F000Fu), as_h2(xh[4 * j + 1]), pa, false);
            pb = __builtin_amdgcn_fdot2(as_h2(w & 0x00F000F0u), as_h2(xh[4 * j + 2]), pb, false);
            pb = __builtin_amdgcn_fdot2(as_h2(s & 0x00F000F0u), as_h2(xh[4 * j + 3]), pb, false);
        }
    }
    if constexpr (FMT == FMT_Q8) return (pa + pb) * 16777216.0f;
    else return fmaf(pb, 1048576.0f, pa * 16777216.0f);
}

// Dot products in f32 with two interleaved accumulators (halves the dependency chain).
template <int n>
__device__ __forceinline__ float dot_f32(const float (&c)[n], const float* x) {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int i = 0; i < n; i += 2) {
        a0 = fmaf(c[i], x[i], a0);
        a1 = fmaf(c[i + 1], x[i + 1], a1);
    }
    return a0 + a1;
}
// The same over the 8 values of word I of a CW-word Q4 chunk (values 4I .. 4I+3 and 4CW+4I ..).
template <int CW, int I, int n>
__device__ __forceinline__ float dot_word_f32(const float (&c)[n], const float* x) {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
        a0 = fmaf(c[4 * I + j], x[4 * I + j], a0);
        a1 = fmaf(c[4 * I + j + 1], x[4 * I + j + 1], a1);
        a0 = fmaf(c[4 * CW + 4 * I + j], x[4 * CW + 4 * I + j], a0);
        a1 = fmaf(c[4 * CW + 4 * I + j + 1], x[4 * CW + 4 * I + j + 1], a1);
    }
    return a0 + a1;
}
// Wavefront sums of M values at once, each lane ending with one of the totals (a transposing
// reduction).  Six levels of lane distance 32, 16, 8, 4, 2, 1; while more than one value is left, a
// level adds the values pairwise across the distance so that the lanes on one side keep the sums of
// the first half of the values and the lanes on the other side those of the second half (halving
// the values and the instructions at each level); once one value is left, a level adds it to its
// partner.  Distances 32 and 16 use v_permlane32_swap / v_permlane16_swap (lane halves and rows
// exchanged between two registers), the in-row distances DPP (row rotation by 8, half-row mirror,
// quad permutations).  With M = 2^m, lane l ends with the total of value l >> (6 - m).
template <int L>
__device__ __forceinline__ float tsum_pair(float a, float b, int lane) {
    if constexpr (L == 0) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else if constexpr (L == 1) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else {
        constexpr int ctrl = L == 2 ? 0x128 : L == 3 ? 0x141 : L == 4 ? 0x4E : 0xB1;
        const bool hi = (lane & (32 >> L)) != 0;
        const float send = hi ? a : b, keep = hi ? b : a;
        return keep + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send), ctrl, 0xF, 0xF, false));
    }
}
template <int L, int M>
__device__ __forceinline__ void tsum_levels(float (&v)[16], int lane) {
    if constexpr (L < 6) {
        if constexpr (M >= 2) {
#pragma unroll
            for (int k = 0; k < M / 2; k++) v[k] = tsum_pair<L>(v[k], v[k + M / 2], lane);
            tsum_levels<L + 1, M / 2>(v, lane);
        } else {
            v[0] = tsum_pair<L>(v[0], v[0], lane);
            tsum_levels<L + 1, 1>(v, lane);
        }
    }
}
// s_waitcnt immediate: at most N vector-memory operations outstanding, the other counters
// unconstrained (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
constexpr int rows_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt");
    return (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}
constexpr int pow2_ceil(int n) { return n <= 1 ? 1 : 2 * pow2_ceil((n + 1) / 2); }
constexpr int log2_exact(int n) { return n <= 1 ? 0 : 1 + log2_exact(n / 2); }

struct RowsArgs {
    const char* codes;  // the expert's matrices
    const char* scales;
    const char* offs;
    int u0, u1;  // this wavefront's units (rows; SwiGLU: gate / up row pairs)
    int lane, wave;
};

// Ring slot I as its own LDS array: per wavefront kRowsBatch rows x 1 KiB of code bytes, then the
// rows' block scales and (Q4A) offsets, 640 bytes each (two runs of at most 2 x 128 bytes, or one of
// 4 x 128, each from a 16-byte boundary).
constexpr int kRowsSBytes = 640;
template <int FMT>
constexpr int rows_wave_bytes() { return kRowsBatch * 1024 + (FMT == FMT_Q4A ? 2 : 1) * kRowsSBytes; }
template <int FMT, int I>
__device__ __forceinline__ uint8_t* rows_slot() {
    __shared__ __attribute__((aligned(16))) uint8_t b[kRowsWaves * rows_wave_bytes<FMT>()];
    return b;
}
// X rows of a segment chunk shared by the workgroup's wavefronts (fast mode, Q4 / Q8): row t, word w
// of lane l at [(t * (XHW + 2) + w) * 64 + l]; words XHW and XHW + 1 hold the row's x sum of the
// lane and its output scale.
template <int XHW>
__device__ __forceinline__ uint32_t* rows_xshare() {
    __shared__ __attribute__((aligned(16))) uint32_t b[kRowsSeg * (XHW + 2) * 64];
    return b;
}
// Fast-mode Q4 / Q8 chunks convert each X row once per workgroup (wavefront t converts row t into
// LDS, then every wavefront reads all rows) instead of once per wavefront.
template <int FMT, int AR, int CW>
constexpr bool rows_share_x() { return AR == AR_DOT2 && FMT != FMT_Q4A && CW == 4; }

// One segment chunk: NT X rows starting at gathered row c, against the wavefront's units.
template <int FMT, int XT, int AR, bool XH, int EPI, int NT, int CW>
__device__ __forceinline__ void rows_chunk(const GemmParams& p, const RowsArgs& a, int c) {
    constexpr int V = RowsChunk<FMT, CW>::V, CB = RowsChunk<FMT, CW>::CB;
    // 12-byte chunks take the f32 arithmetic only: with DOT2 the two blocks' separate partials cost
    // more per row than the idle lanes of 16-byte chunks (measured on K = 1536)
    static_assert(CW == 4 || AR == AR_F32, "12-byte chunks: f32 arithmetic");
    constexpr int RU = EPI == EPI_SWIGLU ? 2 : 1;  // weight rows per unit
    constexpr int RB = kRowsBatch / RU;            // units per batch
    constexpr int D = kRowsRing;
    constexpr int XF = AR == AR_F32 ? V : 1;
    constexpr int XHW = AR == AR_DOT2 ? V / 2 : 1;
    const int K = p.K, N = p.N, lane = a.lane;
    const int chunks = K / V;
    const int half_n = N >> 1;  // SwiGLU: I
    const bool on = lane < chunks;
    const int cc = min(lane, chunks - 1);
    // blocks A and B of the chunk's words (the same block for a 16-byte chunk); word 1 lies in A
    // when sel1 (CW = 3)
    const int blkA = FMT == FMT_Q8 ? (cc >> 1) : (CB * cc) >> 4;
    const int blkB = FMT == FMT_Q8 ? blkA : (CB * cc + CB - 4) >> 4;
    const bool sel1 = ((CB * cc + 4) >> 4) == blkA;
    auto in_a = [&](int word) { return CW == 4 || word == 0 || (word == 1 && sel1); };

    // X rows of the chunk: this lane's values of every row (zero past K and for rows outside X).
    float xf[NT][XF];
    uint32_t xh[NT][XHW];
    float sx[NT], sxb[NT];  // x sums over the values of blocks A and B
    float osc[NT];  // output scale per X row: the fused x_half inverse scale times rs
    auto conv_row = [&](int t, float (&xfo)[XF], uint32_t (&xho)[XHW], float& sxo, float& sxbo, float& osco)
                        __attribute__((always_inline)) {
        int s = c + t;
        if (p.row_src) s = p.row_src[c + t];
        const bool valid = s >= 0 && s < p.x_rows;  // uniform over the wavefront
        float v[V];
#pragma unroll
        for (int i = 0; i < V; i++) v[i] = 0.f;
        if (valid && CW != 4) {
            // per word: the low-nibble run of 4 values, and the high-nibble run 16 further on
#pragma unroll
            for (int i = 0; i < CW; i++) {
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const size_t e0 = (size_t)s * K + chunk_word_k<FMT, CW>(cc, i) + 16 * h;
                    float* dst = v + 4 * CW * h + 4 * i;
                    if constexpr (XT == XT_F32) {
                        const f32x4_t q = *(const QG_GLOBAL f32x4_t*)(gptr<float>(p.X) + e0);
                        dst[0] = q.x;
                        dst[1] = q.y;
                        dst[2] = q.z;
                        dst[3] = q.w;
                    } else {
                        const u32x2_t q = *(const QG_GLOBAL u32x2_t*)(gptr<uint16_t>(p.X) + e0);
#pragma unroll
                        for (int j = 0; j < 4; j++) {
                            const uint16_t hv = (uint16_t)((j < 2 ? q.x : q.y) >> (16 * (j & 1)));
                            dst[j] = XT == XT_F16 ? f16_to_f32(hv) : bf16_to_f32(hv);
                        }
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < V; i++) v[i] = on ? v[i] : 0.f;
        } else if (valid) {
            const size_t e0 = (size_t)s * K + (size_t)cc * V;
            if constexpr (XT == XT_F32) {
#pragma unroll
                for (int i = 0; i < V / 4; i++) {
                    const f32x4_t q = *(const QG_GLOBAL f32x4_t*)(gptr<float>(p.X) + e0 + 4 * i);
                    v[4 * i] = q.x;
                    v[4 * i + 1] = q.y;
                    v[4 * i + 2] = q.z;
                    v[4 * i + 3] = q.w;
                }
            } else {
#pragma unroll
                for (int i = 0; i < V / 8; i++) {
                    const u32x4_t q = *(const QG_GLOBAL u32x4_t*)(gptr<uint16_t>(p.X) + e0 + 8 * i);
                    const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                    for (int j = 0; j < 8; j++) {
                        const uint16_t hv = (uint16_t)(w4[j >> 1] >> (16 * (j & 1)));
                        v[8 * i + j] = XT == XT_F16 ? f16_to_f32(hv) : bf16_to_f32(hv);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < V; i++) v[i] = on ? v[i] : 0.f;
        }
        float sc = 1.f, inv = 1.f;
        if constexpr (XH) {
            float m = 0.f;
#pragma unroll
            for (int i = 0; i < V; i++) m = fmaxf(m, fabsf(v[i]));
            const int e = row_scale_exp(wave_max_nonneg(m));
            sc = ldexpf(1.0f, e);
            inv = ldexpf(1.0f, -e);
        }
        osco = inv * (p.rs ? p.rs[c + t] : 1.f);
        sxo = sxbo = 0.f;
        // value i belongs to word (i % (4 CW)) / 4
        if constexpr (AR == AR_F32) {
#pragma unroll
            for (int i = 0; i < V; i++) {
                xfo[i] = v[i];
                if constexpr (FMT == FMT_Q4A) {
                    if (in_a((i % (4 * CW)) >> 2)) sxo += v[i];
                    else sxbo += v[i];
                }
            }
        } else {
            uint16_t hv[V];
#pragma unroll
            for (int i = 0; i < V; i++) {
                // fused scaling: f32 product, then nearest-even narrowing (as x_half does); f16 X: an
                // exact round trip
                hv[i] = XH ? f32_to_f16_bits(keep_f32(v[i] * sc)) : f32_to_f16_bits(v[i]);
                sxo += f16_to_f32(hv[i]);
            }
            auto pk = [&](int i0, int i1) { return (uint32_t)hv[i0] | ((uint32_t)hv[i1] << 16); };
#pragma unroll
            for (int j = 0; j < CW; j++) {
                if constexpr (FMT == FMT_Q8) {
                    xho[2 * j] = pk(4 * j, 4 * j + 2);
                    xho[2 * j + 1] = pk(4 * j + 1, 4 * j + 3);
                } else {
                    xho[4 * j] = pk(4 * j, 4 * j + 2);
                    xho[4 * j + 1] = pk(4 * j + 1, 4 * j + 3);
                    xho[4 * j + 2] = pk(4 * CW + 4 * j, 4 * CW + 4 * j + 2);
                    xho[4 * j + 3] = pk(4 * CW + 4 * j + 1, 4 * CW + 4 * j + 3);
                }
            }
        }
    };
    constexpr bool SHARE = rows_share_x<FMT, AR, CW>();
    if constexpr (SHARE) {
        // wavefront t converts row t; one barrier; every wavefront reads every row
        uint32_t* const xs = rows_xshare<XHW>();
        if (a.wave < NT) {
            float xfr[XF];
            uint32_t xhr[XHW];
            float sxr, sxbr, oscr;
            conv_row(a.wave, xfr, xhr, sxr, sxbr, oscr);
#pragma unroll
            for (int i = 0; i < XHW; i++) xs[(a.wave * (XHW + 2) + i) * 64 + lane] = xhr[i];
            xs[(a.wave * (XHW + 2) + XHW) * 64 + lane] = __float_as_uint(sxr);
            xs[(a.wave * (XHW + 2) + XHW + 1) * 64 + lane] = __float_as_uint(oscr);
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < NT; t++) {
#pragma unroll
            for (int i = 0; i < XHW; i++) xh[t][i] = xs[(t * (XHW + 2) + i) * 64 + lane];
            sx[t] = __uint_as_float(xs[(t * (XHW + 2) + XHW) * 64 + lane]);
            osc[t] = __uint_as_float(xs[(t * (XHW + 2) + XHW + 1) * 64 + lane]);
            sxb[t] = 0.f;
        }
    } else {
#pragma unroll
        for (int t = 0; t < NT; t++) {
            conv_row(t, xf[t], xh[t], sx[t], sxb[t], osc[t]);
            // one X row at a time: its raw values are dead before the next row's loads go out
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Weight rows of the wavefront's batches, all copied by buffer_load ... lds into the wavefront's
    // part of a ring slot: the code bytes of row i of a batch (unit i % RB, gate / up i / RB) to row
    // i (16 bytes per lane, one instruction per row, lanes past the row masked off -- lane 0 always
    // copies, so the instruction is always issued); the block scales (and Q4A offsets) of the batch
    // in one instruction: the RU runs of RB consecutive rows, each from the 16-byte boundary at or
    // below its first byte, RL = 8 RB + 1 lanes of 16 bytes a run.  Every stage issues the same LS
    // copies -- the D - 1 stages issued past the last repeat it (cache hits) -- so that a constant
    // vmcnt wait covers exactly the stage about to be computed.  Only copies to LDS go out here: they
    // complete in issue order among themselves, but not with respect to loads into registers (mixing
    // the two made the wait cover too little, seen as stale slot reads that changed from run to run).
    const int rowb = FMT == FMT_Q8 ? K : K >> 1;
    constexpr int ESZ = FMT == FMT_Q8 ? 4 : 2;
    const int srowb = (K >> 5) * ESZ, orowb = FMT == FMT_Q4A ? (K / p.group) * 2 : 0;
    const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc((void*)a.codes, 0, N * rowb, 0x00020000);
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc((void*)a.scales, 0, N * srowb, 0x00020000);
    const __amdgpu_buffer_rsrc_t ors =
        __builtin_amdgcn_make_buffer_rsrc((void*)(FMT == FMT_Q4A ? a.offs : a.scales), 0, N * orowb, 0x00020000);
    const int os = blkA * ESZ, osb = blkB * ESZ;
    const int oo = FMT == FMT_Q4A ? ((blkA * 32) / p.group) * 2 : 0;
    const int oob = FMT == FMT_Q4A ? ((blkB * 32) / p.group) * 2 : 0;
    const int wbase = a.wave * rows_wave_bytes<FMT>();
    constexpr int SOFF = kRowsBatch * 1024, OOFF = SOFF + kRowsSBytes;  // scale / offset parts
    constexpr int RL = 8 * RB + 1;                                     // lanes per run
    static_assert(RU * RL * 16 <= kRowsSBytes && RB * 128 + 16 <= RL * 16, "scale part");
    constexpr int LS = kRowsBatch + (FMT == FMT_Q4A ? 2 : 1);  // copies per stage
    static_assert((D - 1) * LS <= 63, "vmcnt range");
    const int nstage = (a.u1 - a.u0 + RB - 1) / RB;
    const int lru = lane / RL, lb = 16 * (lane % RL);  // this lane's run and 16-byte piece of it
    auto lds = [](uint8_t* q) { return (__attribute__((address_space(3))) void*)q; };
    auto issue = [&](auto slotc, int st) __attribute__((always_inline)) {
        constexpr int sl = decltype(slotc)::value;
        // the copies into the slot go out after the reads of its previous stage (a compiler
        // memory barrier: the compiler does not see that a copy writes every lane's bytes)
        asm volatile("" ::: "memory");
        uint8_t* const dst = rows_slot<FMT, sl>() + wbase;
        const int sr = min(st, nstage - 1);
#pragma unroll
        for (int i = 0; i < kRowsBatch; i++) {
            const int n = min(a.u0 + sr * RB + i % RB, a.u1 - 1) + (i / RB) * half_n;
            if (on) __builtin_amdgcn_raw_ptr_buffer_load_lds(crs, lds(dst + i * 1024), CB, n * rowb + CB * cc, 0, 0, 0);
        }
        const int n0 = a.u0 + sr * RB + lru * half_n;  // first row of this lane's run
        if (lane < RU * RL) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, lds(dst + SOFF), 16, ((n0 * srowb) & ~15) + lb, 0, 0, 0);
            if constexpr (FMT == FMT_Q4A)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ors, lds(dst + OOFF), 16, ((n0 * orowb) & ~15) + lb, 0, 0, 0);
        }
    };

    QG_GLOBAL float* Y = gptr_mut<float>(p.Y);
    // Epilogue: the J = RB * NT totals of a batch (value j = unit j / NT, X row j % NT; padded to a
    // power of two M) come out of one transposing reduction, lane l holding value l >> (6 - log2 M);
    // SwiGLU and the stores then run once per batch, by the first lane of each value.
    constexpr int J = RB * NT, M = pow2_ceil(J), SH = 6 - log2_exact(M);
    static_assert(M <= 16, "totals per batch");
    const int jv = lane >> SH, jr = jv / NT, jt = jv % NT;
    const bool jlead = (lane & ((1 << SH) - 1)) == 0 && jv < J;
    float oscv = osc[0];
#pragma unroll
    for (int t = 1; t < NT; t++) oscv = jt == t ? osc[t] : oscv;
    const int pitch = EPI == EPI_SWIGLU ? half_n : N;
    auto compute = [&](auto slotc, int st) __attribute__((always_inline)) {
        constexpr int sl = decltype(slotc)::value;
        // this stage's copies have landed: D - 1 later stages (LS loads each) were issued since;
        // loads complete in issue order, and counting the loads only (not the output stores) can
        // only make the wait longer.  The compiler does not see that a copy writes every lane's 16
        // bytes (it models the first lane's), so a memory clobber keeps the slot's reads below the
        // wait.
        __builtin_amdgcn_s_waitcnt(rows_vmcnt<(D - 1) * LS>());
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        // a copy to LDS puts lane l's bytes at 16 l whatever its size (12-byte copies leave 4-byte gaps)
        const uint8_t* const src = rows_slot<FMT, sl>() + wbase + 16 * cc;
        const uint8_t* const ssrc = rows_slot<FMT, sl>() + wbase + SOFF;
        const uint8_t* const osrc = rows_slot<FMT, sl>() + wbase + OOFF;
        int sbase[RU], obase[RU];  // a run's first row within the scale / offset part
#pragma unroll
        for (int ru = 0; ru < RU; ru++) {
            const int n0 = a.u0 + min(st, nstage - 1) * RB + ru * half_n;
            sbase[ru] = ru * RL * 16 + ((n0 * srowb) & 15);
            obase[ru] = ru * RL * 16 + ((n0 * orowb) & 15);
        }
        const int u = a.u0 + st * RB;
        float gvals[16], uvals[16];
#pragma unroll
        for (int j = 0; j < 16; j++) gvals[j] = uvals[j] = 0.f;
#pragma unroll
        for (int r = 0; r < RB; r++) {
            // one unit at a time (a scheduling barrier after each): its codes are decoded once and
            // used for every X row, and only one unit's decoded codes are live
#pragma unroll
            for (int ru = 0; ru < RU; ru++) {
                const int i = ru * RB + r;
                uint32_t w[CW];
                if constexpr (CW == 4) {
                    const u32x4_t q = *(const u32x4_t*)(src + i * 1024);
                    w[0] = q.x;
                    w[1] = q.y;
                    w[2] = q.z;
                    w[3] = q.w;
                } else {
#pragma unroll
                    for (int j = 0; j < CW; j++) w[j] = ((const uint32_t*)(src + i * 1024))[j];
                }
                float d, m = 0.f, db = 0.f, mb = 0.f;
                const int srow = sbase[ru] + r * srowb, orow = obase[ru] + r * orowb;
                if constexpr (FMT == FMT_Q8) {
                    d = *(const float*)(ssrc + srow + os);
                } else {
                    d = f16_to_f32(*(const uint16_t*)(ssrc + srow + os));
                    if constexpr (CW != 4) db = f16_to_f32(*(const uint16_t*)(ssrc + srow + osb));
                    if constexpr (AR == AR_F32) {
                        d *= 0.0625f;
                        db *= 0.0625f;
                    }
                    if constexpr (FMT == FMT_Q4A) {
                        m = bf16_to_f32(*(const uint16_t*)(osrc + orow + oo));
                        if constexpr (CW != 4) mb = bf16_to_f32(*(const uint16_t*)(osrc + orow + oob));
                    }
                }
                float acc[NT];
                if constexpr (AR == AR_F32) {
                    float cw[V];
                    codes_f32<FMT, CW>(w, cw);
#pragma unroll
                    for (int t = 0; t < NT; t++) {
                        if constexpr (CW == 4) {
                            const float pr = dot_f32(cw, xf[t]);
                            acc[t] = FMT == FMT_Q4A ? fmaf(d, pr, m * sx[t]) : d * pr;
                        } else {
                            // words 0 (block A), 2 (block B) and 1 (A when sel1, else B)
                            const float p0 = dot_word_f32<CW, 0>(cw, xf[t]), p1 = dot_word_f32<CW, 1>(cw, xf[t]);
                            const float p2 = dot_word_f32<CW, 2>(cw, xf[t]);
                            const float pa = sel1 ? p0 + p1 : p0, pb = sel1 ? p2 : p1 + p2;
                            const float off = FMT == FMT_Q4A ? fmaf(m, sx[t], mb * sxb[t]) : 0.f;
                            acc[t] = fmaf(d, pa, fmaf(db, pb, off));
                        }
                    }
                } else {
                    // sum (u - off) x = P - off * sum x, off = 8 (Q4, Q4A) or 128 (Q8)
                    const float cofs = m - (FMT == FMT_Q8 ? 128.0f : 8.0f) * d;
#pragma unroll
                    for (int t = 0; t < NT; t++) acc[t] = fmaf(d, dot_codes_h2<FMT, CW>(w, xh[t]), cofs * sx[t]);
                }
#pragma unroll
                for (int t = 0; t < NT; t++) {
                    if (ru == 0) gvals[r * NT + t] = acc[t];
                    else uvals[r * NT + t] = acc[t];
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        tsum_levels<0, M>(gvals, lane);
        if constexpr (EPI == EPI_SWIGLU) tsum_levels<0, M>(uvals, lane);
        if (jlead && u + jr < a.u1) {
            QG_GLOBAL float* dst = Y + (size_t)(c + jt) * pitch + (u + jr);
            if constexpr (EPI == EPI_SWIGLU) *dst = silu_mul(gvals[0] * oscv, uvals[0] * oscv);
            else *dst = gvals[0] * oscv;
        }
    };

    // Ring: stages 0 .. D-2 in flight, then per stage s the copies of stage s + D - 1 (into the slot
    // stage s - 1 used, whose reads are done) go out before stage s is computed.
    auto prologue = [&](auto tc) __attribute__((always_inline)) { issue(tc, decltype(tc)::value); };
    auto stage = [&](auto uc, int st) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;
        issue(std::integral_constant<int, (u + D - 1) % D>{}, st + D - 1);
        compute(uc, st);
    };
    if (a.u0 < a.u1) {  // uniform over the wavefront (an empty range only takes part in the X sharing)
        rows_run<0, D - 1>(prologue);
        int st = 0;
        for (; st + D <= nstage; st += D) rows_run_from<0, D>(stage, st);
        rows_run_tail<0, D>(stage, st, nstage);
    }
    // every wavefront has read the shared X rows before the next chunk writes them
    if constexpr (SHARE) __syncthreads();
}

// Grid: (gx, E) workgroups of kRowsWaves wavefronts; the gx * kRowsWaves wavefronts of expert e split
// its units into equal runs of whole batches.
template <int FMT, int XT, int AR, bool XH, int EPI, int CW>
__global__ __launch_bounds__(64 * kRowsWaves) void grouped_rows_kernel(GemmParams p) {
    const int e = blockIdx.y;
    const int r0 = min(max(p.seg_off[e], 0), p.R);
    const int r1 = min(max(p.seg_off[e + 1], r0), p.R);
    if (r1 <= r0) return;  // uniform over the workgroup
    constexpr int RB = kRowsBatch / (EPI == EPI_SWIGLU ? 2 : 1);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int units = EPI == EPI_SWIGLU ? (p.N >> 1) : p.N;
    const int nb = (units + RB - 1) / RB;
    const int gw = (int)blockIdx.x * kRowsWaves + wave, GW = (int)gridDim.x * kRowsWaves;
    RowsArgs a;
    a.u0 = RB * (int)(((int64_t)nb * gw) / GW);
    a.u1 = min(units, RB * (int)(((int64_t)nb * (gw + 1)) / GW));
    // uniform over the wavefront; with shared X rows it still takes part in every chunk's barriers
    if (a.u0 >= a.u1 && !rows_share_x<FMT, AR, CW>()) return;
    a.lane = threadIdx.x & 63;
    a.wave = wave;
    const Expert ex = ((const Expert*)p.experts)[e];
    a.codes = (const char*)ex.codes;
    a.scales = (const char*)ex.scales;
    a.offs = (const char*)ex.offsets;
    for (int c = r0; c < r1; c += kRowsSeg) {
        const int nt = min(kRowsSeg, r1 - c);
        if (nt == 1) rows_chunk<FMT, XT, AR, XH, EPI, 1, CW>(p, a, c);
        else if (nt == 2) rows_chunk<FMT, XT, AR, XH, EPI, 2, CW>(p, a, c);
        else if (nt == 3) rows_chunk<FMT, XT, AR, XH, EPI, 3, CW>(p, a, c);
        else rows_chunk<FMT, XT, AR, XH, EPI, 4, CW>(p, a, c);
    }
}

// Largest K the kernel takes: one 16-byte chunk per lane (Q4 / Q4A 2048, Q8 1024).  Two chunks per
// lane would hold 256 f32 X values per lane at 4 segment rows.
static int rows_kmax(int fmt) { return 64 * (fmt == FMT_Q8 ? 16 : 32); }

// 12-byte lane chunks (Q4 / Q4A, K a multiple of 96 up to 1536, f32 arithmetic): K / 24 lanes busy
// instead of K / 32.  The 128-expert block's down projection (K 1536): 91.4 -> 84.2 us in exact mode.
static bool rows_chunk12(int fmt, int K) { return fmt != FMT_Q8 && K % 96 == 0 && K <= 1536; }

template <int FMT, int XT, int AR, bool XH, int EPI>
static void rows_launch(const GemmParams& p, int gx, hipStream_t s) {
    if constexpr (FMT != FMT_Q8 && AR == AR_F32) {
        if (rows_chunk12(FMT, p.K)) {
            hipLaunchKernelGGL((grouped_rows_kernel<FMT, XT, AR, XH, EPI, 3>), dim3(gx, p.E), dim3(64 * kRowsWaves), 0,
                               s, p);
            return;
        }
    }
    hipLaunchKernelGGL((grouped_rows_kernel<FMT, XT, AR, XH, EPI, 4>), dim3(gx, p.E), dim3(64 * kRowsWaves), 0, s, p);
}

template <int FMT>
static bool rows_pick(int xt, bool fast, int epi, const GemmParams& p, int gx, hipStream_t s) {
    if (fast && xt == XT_F32) {
        if (epi == EPI_SWIGLU) rows_launch<FMT, XT_F32, AR_DOT2, true, EPI_SWIGLU>(p, gx, s);
        else rows_launch<FMT, XT_F32, AR_DOT2, true, EPI_PLAIN>(p, gx, s);
    } else if (fast && xt == XT_F16) {
        if (epi != EPI_PLAIN) return false;
        rows_launch<FMT, XT_F16, AR_DOT2, false, EPI_PLAIN>(p, gx, s);
    } else if (xt == XT_F32) {
        if (epi == EPI_SWIGLU) rows_launch<FMT, XT_F32, AR_F32, false, EPI_SWIGLU>(p, gx, s);
        else rows_launch<FMT, XT_F32, AR_F32, false, EPI_PLAIN>(p, gx, s);
    } else {
        if (epi != EPI_PLAIN) return false;
        if (xt == XT_F16) rows_launch<FMT, XT_F16, AR_F32, false, EPI_PLAIN>(p, gx, s);
        else rows_launch<FMT, XT_BF16, AR_F32, false, EPI_PLAIN>(p, gx, s);
    }
    return true;
}

bool grouped_rows_fits(int fmt, int K, int N, int epi) {
    // byte offsets into an expert's codes are 31-bit buffer offsets
    // (Q8A is not a grouped format)
    return fmt != FMT_Q8A && K <= rows_kmax(fmt) && (int64_t)N * K < ((int64_t)1 << 31) &&
           (epi == EPI_PLAIN || (N % 2) == 0);
}

hipError_t launch_grouped_rows(int fmt, int xt, bool fast, int epi, const GemmParams& p, hipStream_t s) {
    if (!grouped_rows_fits(fmt, p.K, p.N, epi)) return hipErrorInvalidValue;
    // workgroups per expert: about four rounds of eight resident wavefronts per CU over the experts
    // that have rows
    int cus = 256, dev = 0;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    const int used = std::max(1, std::min(p.E, p.R));
    const int units = epi == EPI_SWIGLU ? p.N / 2 : p.N;
    const int max_gx = std::max(1, (units + kRowsBatch - 1) / kRowsBatch / kRowsWaves);
    const int gx = std::max(1, std::min(max_gx, (4 * cus * 8 / kRowsWaves + used - 1) / used));
    bool ok = false;
    if (fmt == FMT_Q4) ok = rows_pick<FMT_Q4>(xt, fast, epi, p, gx, s);
    else if (fmt == FMT_Q4A) ok = rows_pick<FMT_Q4A>(xt, fast, epi, p, gx, s);
    else if (fmt == FMT_Q8) ok = rows_pick<FMT_Q8>(xt, fast, epi, p, gx, s);
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace qg
