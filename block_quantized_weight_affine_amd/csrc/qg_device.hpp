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

enum { FMT_Q4 = 0, FMT_Q4A = 1, FMT_Q8 = 2 };
enum { XT_F32 = 0, XT_F16 = 1, XT_BF16 = 2 };

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

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
    asm volatile("" : "+v"(v));
    return v;
}
template <int ST>
__device__ __forceinline__ uint16_t f32_to_16(float f) {
    return ST == XT_F16 ? f32_to_f16_bits(f) : f32_to_bf16_bits(f);
}

// ---- raw block of one row: the packed bytes and the block's scale (and offset) ------------------
// Q4 / Q4A: 16 code bytes; Q8: 32 code bytes.
template <int FMT>
struct RawBlock;
template <>
struct RawBlock<FMT_Q4> {
    uint4 q;
    float d;
    float m;
};
template <>
struct RawBlock<FMT_Q4A> {
    uint4 q;
    float d;
    float m;
};
template <>
struct RawBlock<FMT_Q8> {
    uint4 q0, q1;
    float d;
    float m;
};

// Loads block b of row n (all addresses in bounds: the caller clamps n and b).
template <int FMT>
__device__ __forceinline__ RawBlock<FMT> load_block(const void* codes, const void* scales, const uint16_t* offs,
                                                    int group, int K, int n, int b) {
    RawBlock<FMT> r;
    const size_t bi = (size_t)n * (size_t)(K >> 5) + (size_t)b;
    if constexpr (FMT == FMT_Q8) {
        const uint4* p = (const uint4*)((const int8_t*)codes + (size_t)n * (size_t)K + (size_t)b * 32);
        r.q0 = p[0];
        r.q1 = p[1];
        r.d = ((const float*)scales)[bi];
        r.m = 0.f;
    } else {
        const uint4* p = (const uint4*)((const uint8_t*)codes + (size_t)n * (size_t)(K >> 1) + (size_t)b * 16);
        r.q = *p;
        r.d = f16_to_f32(((const uint16_t*)scales)[bi]);
        if constexpr (FMT == FMT_Q4A)
            r.m = bf16_to_f32(offs[(size_t)n * (size_t)(K / group) + (size_t)((b * 32) / group)]);
        else
            r.m = 0.f;
    }
    return r;
}

// Code byte i (0..15) of a Q4 block.
__device__ __forceinline__ uint32_t q4_byte(const uint4& q, int i) {
    const uint32_t w = i < 4 ? q.x : i < 8 ? q.y : i < 12 ? q.z : q.w;
    return (w >> (8 * (i & 3))) & 0xFFu;
}

// The f32 value of element e (0..31) of a block: exactly what the pages' decoders compute.
template <int FMT>
__device__ __forceinline__ float block_value(const RawBlock<FMT>& r, int e) {
    if constexpr (FMT == FMT_Q8) {
        const uint4& q = e < 16 ? r.q0 : r.q1;
        const int i = e & 15;
        const uint32_t w = i < 4 ? q.x : i < 8 ? q.y : i < 12 ? q.z : q.w;
        const int c = (int)(int8_t)((w >> (8 * (i & 3))) & 0xFFu);
        return (float)c * r.d;
    } else {
        const uint32_t byte = q4_byte(r.q, e & 15);
        const uint32_t nib = e < 16 ? (byte & 15u) : (byte >> 4);
        const float v = ((float)nib - 8.0f) * r.d;
        if constexpr (FMT == FMT_Q4A)
            return v + r.m;
        else
            return v;
    }
}

// Whole block to f32, element order.
template <int FMT>
__device__ __forceinline__ void block_to_f32(const RawBlock<FMT>& r, float (&v)[32]) {
#pragma unroll
    for (int e = 0; e < 32; e++) v[e] = block_value<FMT>(r, e);
}

// Fast-mode fragments: element 8j + s of the block, rounded to the staged 16-bit type ST, is
// slot s of fragment j (j = 0..3).  Each fragment is one 8-wide operand of a 16-k MFMA step.
template <int FMT, int ST>
__device__ __forceinline__ void block_to_frags16(const RawBlock<FMT>& r, short8_t (&f)[4]) {
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
        for (int s = 0; s < 8; s++) f[j][s] = (short)f32_to_16<ST>(keep_f32(block_value<FMT>(r, 8 * j + s)));
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

// ---- wavefront helpers ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

}  // namespace qg
