// qg_device.hpp -- device-side types and the block decoders shared by every kernel.
//
// Formats (page "oxinfer 0.0.5 src/metal.rs", SHADER_SRC, the dequantizers Q4W / Q4A / Q8W):
//   Q4   block b of row n = 16 bytes at n*K/2 + 16b; byte j: low nibble -> element j, high nibble
//        -> element j+16; f16 scale d at n*K/32 + b; w = (nibble - 8) * d in f32.
//   Q4A  Q4 plus a bf16 offset m at n*(K/group) + floor(k/group): w = (nibble - 8) * d + m in f32.
//   Q4 products are exact in f32 (4-bit integer times an 11-bit significand), so fusing the
//   multiply and the add of Q4A into one FMA rounds exactly once, as the separate f32 add does.
//   Q8   int8 q at n*K + k, f32 scale d at n*K/32 + floor(k/32): w = float(q) * d in f32.
// Fast mode stages the nearest-even f16 / bf16 rounding of that f32 value (page section
// MMA_SHADER_SRC, mma_tile, where each dequantized value is converted as the tile is written).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

enum { FMT_Q4 = 0, FMT_Q4A = 1, FMT_Q8 = 2, FMT_Q8A = 3, FMT_Q8A16 = 4 };
// Q8 and Q8A share the code layout (one int8 per element) and the f32 block scales; Q8A adds an f32
// offset per 32-element block: value = (float(q) * d) + m, two roundings as written.  Q8A16 is Q8A
// with a scale and an offset per 16-element block (the GGUF K-quants Q6_K, Q3_K, Q2_K repacked).
template <int FMT>
constexpr bool q8_layout = FMT == FMT_Q8 || FMT == FMT_Q8A || FMT == FMT_Q8A16;
// 16-element blocks: scale / offset index n * K / 16 + k / 16
template <int FMT>
constexpr bool blk16 = FMT == FMT_Q8A16;
enum { XT_F32 = 0, XT_F16 = 1, XT_BF16 = 2 };

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Pointers into global memory.  Loads through them compile to global_load_* rather than
// flat_load_*; flat loads also count against the LDS wait counter, so a wait for an LDS read would
// otherwise wait for weight loads issued stages ahead.
#define QG_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ const QG_GLOBAL T* gptr(const void* p) {
    return (const QG_GLOBAL T*)(p);
}
template <typename T>
__device__ __forceinline__ QG_GLOBAL T* gptr_mut(void* p) {
    return (QG_GLOBAL T*)(p);
}

// base + off as a wavefront-uniform pointer held in scalar registers (off must be uniform).
__device__ __forceinline__ const QG_GLOBAL char* uniform_ptr(const void* base, uint64_t off) {
    const uint64_t a = (uint64_t)(uintptr_t)base + off;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a), hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return (const QG_GLOBAL char*)(((uint64_t)hi << 32) | lo);
}

// Same layout as qg_expert in qgemm.h.
struct Expert {
    const void* codes;
    const void* scales;
    const uint16_t* offsets;
};

// ---- scalar conversions -------------------------------------------------------------------------
__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// The staged 16-bit value is the nearest-even rounding of the f32 value.  Keeping the f32 value
// materialised stops the compiler from folding the f32 multiply-add and the narrowing into one
// mixed-precision FMA with a 16-bit result, which rounds the exact result once and so differs
// from the f32-then-narrow sequence on ties.
__device__ __forceinline__ float keep_f32(float v) {
    asm("" : "+v"(v));
    return v;
}
// An opaque copy of an integer: keeps a masked word as is, so each of its bytes converts with one
// v_cvt_f32_ubyteN instead of a re-derived bit-field extract plus an integer conversion.
__device__ __forceinline__ uint32_t keep_u32(uint32_t v) {
    asm("" : "+v"(v));
    return v;
}
template <int ST>
__device__ __forceinline__ uint16_t f32_to_16(float f) {
    return ST == XT_F16 ? f32_to_f16_bits(f) : f32_to_bf16_bits(f);
}

// ---- raw block of one row: the packed bytes and the block's scale (and offset) ------------------
// Q4 / Q4A: 16 code bytes; Q8: 32 code bytes.  dh keeps the f16 scale bits for the packed-f16 path.
template <int FMT>
struct RawBlock;
template <>
struct RawBlock<FMT_Q4> {
    uint4 q;
    float d, m;
    uint32_t dh;
};
template <>
struct RawBlock<FMT_Q4A> {
    uint4 q;
    float d, m;
    uint32_t dh;
};
template <>
struct RawBlock<FMT_Q8> {
    uint4 q0, q1;
    float d, m;
    uint32_t dh;
};
template <>
struct RawBlock<FMT_Q8A> {
    uint4 q0, q1;
    float d, m;
    uint32_t dh;
};
// d, m: elements 0..15; d2, m2: elements 16..31
template <>
struct RawBlock<FMT_Q8A16> {
    uint4 q0, q1;
    float d, m;
    uint32_t dh;
    float d2, m2;
};

// Blocks past K decode to zeros: every scale and offset of the block cleared.
template <int FMT>
__device__ __forceinline__ void block_clear_if(RawBlock<FMT>& r, bool valid) {
    r.d = valid ? r.d : 0.f;
    r.m = valid ? r.m : 0.f;
    if constexpr (blk16<FMT>) {
        r.d2 = valid ? r.d2 : 0.f;
        r.m2 = valid ? r.m2 : 0.f;
    }
}

// Loads block b of row n (all addresses in bounds: the caller clamps n and b).
template <int FMT>
__device__ __forceinline__ RawBlock<FMT> load_block(const void* codes, const void* scales, const uint16_t* offs,
                                                    int group, int K, int n, int b) {
    RawBlock<FMT> r;
    const size_t bi = (size_t)n * (size_t)(K >> 5) + (size_t)b;
    if constexpr (q8_layout<FMT>) {
        const QG_GLOBAL u32x4_t* p = gptr<u32x4_t>((const int8_t*)codes + (size_t)n * (size_t)K + (size_t)b * 32);
        const u32x4_t a = p[0], c = p[1];
        r.q0 = make_uint4(a.x, a.y, a.z, a.w);
        r.q1 = make_uint4(c.x, c.y, c.z, c.w);
        r.dh = 0;
        if constexpr (blk16<FMT>) {
            // no offsets (NULL): -0, which leaves every value, a zero's sign included, unchanged
            const size_t b16 = (size_t)n * (size_t)(K >> 4) + 2 * (size_t)b;
            r.d = gptr<float>(scales)[b16];
            r.m = offs ? gptr<float>((const void*)offs)[b16] : -0.0f;
            r.d2 = gptr<float>(scales)[b16 + 1];
            r.m2 = offs ? gptr<float>((const void*)offs)[b16 + 1] : -0.0f;
        } else {
            r.d = gptr<float>(scales)[bi];
            r.m = FMT == FMT_Q8A ? gptr<float>((const void*)offs)[bi] : 0.f;
        }
    } else {
        const u32x4_t a = *gptr<u32x4_t>((const uint8_t*)codes + (size_t)n * (size_t)(K >> 1) + (size_t)b * 16);
        r.q = make_uint4(a.x, a.y, a.z, a.w);
        r.dh = gptr<uint16_t>(scales)[bi];
        r.d = f16_to_f32((uint16_t)r.dh);
        if constexpr (FMT == FMT_Q4A)
            r.m = bf16_to_f32(gptr<uint16_t>(offs)[(size_t)n * (size_t)(K / group) + (size_t)((b * 32) / group)]);
        else
            r.m = 0.f;
    }
    return r;
}

// The code bytes of a block as "value bytes" c, one per element, in eight 32-bit words: element e
// is byte e % 4 of word e / 4.  Q4: c = nibble (words 0..3 the low nibbles of bytes 0..15, words
// 4..7 the high nibbles); Q8: c = q XOR 0x80 = q + 128.  Every element's f32 value is then
//   w = fma(float(c), d, c0)                                                         (1)
// with c0 = -8d (Q4), -128d (Q8) or m - 8d (Q4A): the exact value c*d + c0 is the pages' value
// ((nibble - 8) d, q d or (nibble - 8) d + m), and one FMA rounds it once to f32 -- the same
// rounding as the pages' f32 decode, since (nibble - 8) d is exact in f32 and q d is their only
// rounding.  (1) is used for a block when its scale is positive (so a zero result has the
// pages' sign) and, for Q4A, when m - 8d is itself exact in f32.  Otherwise (negative scales, or a
// tiny offset next to a large scale) the block takes the pages' order of operations:
// (c - 8) d, (c - 128) d, or fma(c - 8, d, m) -- the product is exact, so the fused add rounds as
// the separate one.  The choice is made for the whole wavefront at once.
template <int FMT>
__device__ __forceinline__ void value_bytes(const RawBlock<FMT>& r, uint32_t (&c)[8]) {
    if constexpr (q8_layout<FMT>) {
        c[0] = keep_u32(r.q0.x ^ 0x80808080u); c[1] = keep_u32(r.q0.y ^ 0x80808080u);
        c[2] = keep_u32(r.q0.z ^ 0x80808080u); c[3] = keep_u32(r.q0.w ^ 0x80808080u);
        c[4] = keep_u32(r.q1.x ^ 0x80808080u); c[5] = keep_u32(r.q1.y ^ 0x80808080u);
        c[6] = keep_u32(r.q1.z ^ 0x80808080u); c[7] = keep_u32(r.q1.w ^ 0x80808080u);
    } else {
        const uint32_t w[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            c[i] = keep_u32(w[i] & 0x0F0F0F0Fu);
            c[4 + i] = keep_u32((w[i] >> 4) & 0x0F0F0F0Fu);
        }
    }
}

// c0 of (1) and whether (1) gives the pages' bits for this block.
template <int FMT>
__device__ __forceinline__ float block_c0(const RawBlock<FMT>& r, bool& fast) {
    fast = r.d > 0.0f;  // zero or negative scales (and NaN) take the pages' order
    if constexpr (FMT == FMT_Q8A || blk16<FMT>) {
        fast = false;  // two roundings (product, then offset): always the written order
        return -128.0f * r.d;
    } else if constexpr (FMT == FMT_Q8) {
        return -128.0f * r.d;
    } else if constexpr (FMT == FMT_Q4) {
        return -8.0f * r.d;
    } else {
        // TwoSum of m and -8d: the rounding error of s = m - 8d is zero iff s is exact.
        const float a = r.m, b = keep_f32(-8.0f * r.d);
        const float s = keep_f32(a + b);
        const float bb = keep_f32(s - a);
        const float err = (a - (s - bb)) + (b - bb);
        fast = fast && err == 0.0f && isfinite(s);
        return s;
    }
}

// The pages' order of operations for one element (value byte as f32).
template <int FMT>
__device__ __forceinline__ float slow_value(const RawBlock<FMT>& r, float cf) {
    static_assert(!blk16<FMT>, "16-element blocks: the element's half picks the scale (block_frags16_fixup)");
    if constexpr (FMT == FMT_Q8A)
        return keep_f32((cf - 128.0f) * r.d) + r.m;
    else if constexpr (FMT == FMT_Q8)
        return (cf - 128.0f) * r.d;
    else if constexpr (FMT == FMT_Q4)
        return (cf - 8.0f) * r.d;
    else
        return fmaf(cf - 8.0f, r.d, r.m);
}

__device__ __forceinline__ float byte_f32(uint32_t word, int i) { return (float)((word >> (8 * i)) & 0xFFu); }

// Elements 4q .. 4q+3 of a block as f32 (exact-mode staging), in the pages' order of operations for
// every scale: Q8 float(q) * d (their one rounding); Q4 (nibble - 8) d and Q4A (nibble - 8) d + m,
// computed from the signed byte 16 (nibble - 8) (the nibble moved to the byte's high half with its
// top bit flipped, converted by one instruction) times d / 16 -- exact, since d / 16 is a power-of-two
// rescaling of an f16 value (normal in f32) and the product has at most 15 significant bits -- and,
// for Q4A, one FMA with m (the product is exact, so the fused add rounds as the separate add does).
// The sign of a zero product is sign(d), as in (nibble - 8) * d.
template <int FMT>
__device__ __forceinline__ void block_quad_f32(const RawBlock<FMT>& r, int q, float (&v)[4]) {
    if constexpr (q8_layout<FMT>) {
        const uint32_t w[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
        const uint32_t x = w[q];
        float d = r.d, m = r.m;
        if constexpr (blk16<FMT>) {
            d = q < 4 ? r.d : r.d2;
            m = q < 4 ? r.m : r.m2;
        }
#pragma unroll
        for (int b = 0; b < 4; b++) {
            v[b] = (float)(int8_t)(x >> (8 * b)) * d;
            if constexpr (FMT == FMT_Q8A || FMT == FMT_Q8A16) v[b] = keep_f32(v[b]) + m;
        }
    } else {
        const uint32_t w[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
        const uint32_t x = keep_u32(q < 4 ? ((w[q & 3] << 4) & 0xF0F0F0F0u) ^ 0x80808080u
                                          : (w[q & 3] & 0xF0F0F0F0u) ^ 0x80808080u);
        const float d16 = 0.0625f * r.d;
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const float sv = (float)(int8_t)(x >> (8 * b));
            v[b] = FMT == FMT_Q4A ? fmaf(sv, d16, r.m) : sv * d16;
        }
    }
}

// Whole block to f32 (element order): exact-mode staging.
template <int FMT>
__device__ __forceinline__ void block_to_f32(const RawBlock<FMT>& r, float (&v)[32]) {
#pragma unroll
    for (int q = 0; q < 8; q++) {
        float t[4];
        block_quad_f32<FMT>(r, q, t);
#pragma unroll
        for (int b = 0; b < 4; b++) v[4 * q + b] = t[b];
    }
}

// Fast-mode fragments: element 8j + s of the block, rounded to the staged 16-bit type ST, is
// slot s of fragment j (j = 0..3); each fragment is one 8-wide operand of a 16-k MFMA step.
// Q4 into f16: packed f16 arithmetic.  The half with bits 0x6400 | c is 1024 + c, so
// (1024 + c) - 1032 = c - 8 exactly, and one f16 multiply by d rounds (c - 8) d -- exact in f32 --
// once to nearest-even: the same bits as narrowing the f32 value.  Other cases: the f32 value of
// (1), kept in a register, then narrowed (nearest-even).
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Value-byte word k (elements 4k .. 4k+3) of a block, as in value_bytes.
template <int FMT>
__device__ __forceinline__ uint32_t value_word(const RawBlock<FMT>& r, int k) {
    if constexpr (q8_layout<FMT>) {
        const uint32_t w[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
        return keep_u32(w[k] ^ 0x80808080u);
    } else {
        const uint32_t w[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
        return k < 4 ? keep_u32(w[k] & 0x0F0F0F0Fu) : keep_u32((w[k - 4] >> 4) & 0x0F0F0F0Fu);
    }
}

// Eight elements as (1) gives them from their two value-byte words c (elements 4k .. 4k+3 in word
// k), the block's scale d (dh its f16 bits, used by Q4 into f16) and c0 from block_c0; no fallback.
template <int FMT, int ST>
__device__ __forceinline__ short8_t frag16_words(const uint32_t (&c)[2], float d, uint32_t dh, float c0) {
    short8_t f;
    if constexpr (FMT == FMT_Q4 && ST == XT_F16) {
        const half2_t d2 = __builtin_bit_cast(half2_t, dh | (dh << 16));
        const half2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
        uint32_t o[4];
#pragma unroll
        for (int h = 0; h < 2; h++) {
            // halves (c0 | 0x6400, c1 | 0x6400) and (c2 | 0x6400, c3 | 0x6400)
            const half2_t lo = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, c[h], 0x04010400u));
            const half2_t hi = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, c[h], 0x04030402u));
            o[2 * h] = __builtin_bit_cast(uint32_t, (lo - off) * d2);
            o[2 * h + 1] = __builtin_bit_cast(uint32_t, (hi - off) * d2);
        }
        f = __builtin_bit_cast(short8_t, make_uint4(o[0], o[1], o[2], o[3]));
    } else {
#pragma unroll
        for (int s = 0; s < 8; s++)
            f[s] = (short)f32_to_16<ST>(keep_f32(fmaf(byte_f32(c[s >> 2], s & 3), d, c0)));
    }
    return f;
}

// Fragment jj (elements 8jj .. 8jj+7) of a block as (1) gives it, c0 from block_c0; no fallback.
template <int FMT, int ST>
__device__ __forceinline__ short8_t frag16_fast(const RawBlock<FMT>& r, float c0, int jj) {
    const uint32_t c[2] = {value_word<FMT>(r, 2 * jj), value_word<FMT>(r, 2 * jj + 1)};
    return frag16_words<FMT, ST>(c, r.d, r.dh, c0);
}

// The same eight elements in the pages' order of operations (the fallback of (1)): (c - 8) d,
// (c - 128) d or fma(c - 8, d, m) per element, then narrowed to ST.
template <int FMT, int ST>
__device__ __forceinline__ short8_t frag16_words_slow(const uint32_t (&c)[2], float d, float m) {
    short8_t f;
#pragma unroll
    for (int s = 0; s < 8; s++) {
        const float cf = byte_f32(c[s >> 2], s & 3);
        float v;
        if constexpr (FMT == FMT_Q8A || blk16<FMT>) v = keep_f32((cf - 128.0f) * d) + m;
        else if constexpr (FMT == FMT_Q8) v = (cf - 128.0f) * d;
        else if constexpr (FMT == FMT_Q4) v = (cf - 8.0f) * d;
        else v = fmaf(cf - 8.0f, d, m);
        f[s] = (short)f32_to_16<ST>(keep_f32(v));
    }
    return f;
}

// Fragment jj of a block in the pages' order, for the formats (1) never applies to (Q8A, Q8A16: two
// roundings); Q8A16 takes the (scale, offset) pair of the fragment's 16-element half.
template <int FMT, int ST>
__device__ __forceinline__ short8_t frag16_slow(const RawBlock<FMT>& r, int jj) {
    const uint32_t c[2] = {value_word<FMT>(r, 2 * jj), value_word<FMT>(r, 2 * jj + 1)};
    if constexpr (blk16<FMT>) return frag16_words_slow<FMT, ST>(c, jj < 2 ? r.d : r.d2, jj < 2 ? r.m : r.m2);
    else return frag16_words_slow<FMT, ST>(c, r.d, r.m);
}

// The fragments as (1) gives them, without the fallback for blocks where (1) does not apply.
template <int FMT, int ST>
__device__ __forceinline__ void block_to_frags16_fast(const RawBlock<FMT>& r, short8_t (&f)[4]) {
    bool fast;
    const float c0 = block_c0<FMT>(r, fast);
#pragma unroll
    for (int j = 0; j < 4; j++) f[j] = frag16_fast<FMT, ST>(r, c0, j);
}

// True when (1) is not exact for some lane's block of this wavefront (then every lane re-decodes
// its block with block_frags16_fixup, which gives the same bits where (1) was exact).
template <int FMT, int ST>
__device__ __forceinline__ bool frags16_need_fixup(const RawBlock<FMT>& r) {
    if constexpr (FMT == FMT_Q4 && ST == XT_F16) {
        return false;
    } else {
        bool fast;
        block_c0<FMT>(r, fast);
        return !__all(fast);
    }
}

// The pages' order of operations for every element of the block.
template <int FMT, int ST>
__device__ __forceinline__ void block_frags16_fixup(const RawBlock<FMT>& r, short8_t (&f)[4]) {
    uint32_t c[8];
    value_bytes<FMT>(r, c);
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
        for (int s = 0; s < 8; s++) {
            const int e = 8 * j + s;
            if constexpr (blk16<FMT>) {
                // elements 0..15 take (d, m), 16..31 (d2, m2): fl(fl(q d) + m), then the 16-bit rounding
                const float q = byte_f32(c[e >> 2], e & 3) - 128.0f;
                const float v = keep_f32(q * (j < 2 ? r.d : r.d2)) + (j < 2 ? r.m : r.m2);
                f[j][s] = (short)f32_to_16<ST>(keep_f32(v));
            } else {
                f[j][s] = (short)f32_to_16<ST>(keep_f32(slow_value<FMT>(r, byte_f32(c[e >> 2], e & 3))));
            }
        }
}

// Fast-mode fragments with the fallback: blocks where (1) does not apply are re-decoded in the
// pages' order.
template <int FMT, int ST>
__device__ __forceinline__ void block_to_frags16(const RawBlock<FMT>& r, short8_t (&f)[4]) {
    if constexpr (FMT == FMT_Q8A || blk16<FMT>) return block_frags16_fixup<FMT, ST>(r, f);  // no shortcut applies
    block_to_frags16_fast<FMT, ST>(r, f);
    if (frags16_need_fixup<FMT, ST>(r)) block_frags16_fixup<FMT, ST>(r, f);
}

// ---- direct copies into LDS ---------------------------------------------------------------------
// One buffer_load ... lds of 16 bytes per lane: lane l's bytes at byte offset voff of the buffer land
// at lds + 16 l (lds is wave-uniform); offsets at or past the buffer's size read as zero.
__device__ __forceinline__ void buffer_copy16_lds(__amdgpu_buffer_rsrc_t r, void* lds, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// ---- activations ---------------------------------------------------------------------------------
template <int XT>
__device__ __forceinline__ float x_load(const void* X, size_t i) {
    if constexpr (XT == XT_F32)
        return ((const float*)X)[i];
    else if constexpr (XT == XT_F16)
        return f16_to_f32(((const uint16_t*)X)[i]);
    else
        return bf16_to_f32(((const uint16_t*)X)[i]);
}

// 8 consecutive activations starting at element i (i % 8 == 0, 16-byte aligned rows), widened to f32.
template <int XT>
__device__ __forceinline__ void x_load8(const void* X, size_t i, float (&v)[8]) {
    if constexpr (XT == XT_F32) {
        const float4* p = (const float4*)((const float*)X + i);
        const float4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        const uint4 q = *(const uint4*)((const uint16_t*)X + i);
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            if constexpr (XT == XT_F16) {
                v[2 * j] = f16_to_f32((uint16_t)(w[j] & 0xFFFFu));
                v[2 * j + 1] = f16_to_f32((uint16_t)(w[j] >> 16));
            } else {
                v[2 * j] = __uint_as_float(w[j] << 16);
                v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
            }
        }
    }
}

// Eight codes of a fragment as exact f16 (the W-exact fast path): c holds 8 code bytes, Q4 a nibble
// per byte (0..15), Q8 q + 128 (the byte with its top bit flipped).  A byte b becomes the f16
// 1024 + b by a byte permutation into 0x64.., then 1024 + 8 (Q4) or 1024 + 128 (Q8) is subtracted
// in f16, exactly: nibble - 8 and q are small integers, exact in f16.
template <int FMT>
__device__ __forceinline__ short8_t frag16_codes(const uint32_t (&c)[2]) {
    typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
    const h2_t off = FMT == FMT_Q8 ? (h2_t){(_Float16)1152.0f, (_Float16)1152.0f}
                                   : (h2_t){(_Float16)1032.0f, (_Float16)1032.0f};
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const h2_t lo = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, c[j], 0x04010400u)) - off;
        const h2_t hi = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, c[j], 0x04030402u)) - off;
        w[2 * j] = __builtin_bit_cast(uint32_t, lo);
        w[2 * j + 1] = __builtin_bit_cast(uint32_t, hi);
    }
    short8_t r;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        r[2 * j] = (short)(w[j] & 0xFFFFu);
        r[2 * j + 1] = (short)(w[j] >> 16);
    }
    return r;
}

// ---- wavefront helpers ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Sums of each 16-lane row of the wavefront by DPP row shifts by 1, 2, 4, 8 (lanes without a source
// add 0): lane 15 of every row ends with its row's sum.
__device__ __forceinline__ float row16_sum_dpp(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xF, 0xF, false));
    return v;
}
// Full-wavefront sum: the row sums above, then the row-15 broadcast into rows 1 and 3 and the
// row-31 broadcast into rows 2 and 3 (lanes of other rows keep their value): lane 63 ends with the
// sum of all 64 lanes.
__device__ __forceinline__ float wave_sum_lane63(float v) {
    v = row16_sum_dpp(v);
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
    return v;
}
// Wavefront maximum of non-negative values by the same steps (identity 0), read back from lane 63
// into every lane.
__device__ __forceinline__ float wave_max_nonneg(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false)));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Power-of-two row scale (page "oxinfer 0.0.5 src/metal.rs", MMA_SHADER_SRC, row_scale): the
// largest magnitude lands in [2^13, 2^14); a zero or non-finite amax keeps scale 1.  The caller
// multiplies the row by 2^e before narrowing to f16 and the result by 2^-e.
__device__ __forceinline__ int row_scale_exp(float amax) {
    int e = 0;
    if (amax > 0.f && isfinite(amax)) {
        int fe;
        frexpf(amax, &fe);
        e = min(max(14 - fe, -100), 100);
    }
    return e;
}

// SwiGLU of one gate / up pair (page section silu_half): a = g / (1 + exp(-g)) * u in f32.
__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

}  // namespace qg
