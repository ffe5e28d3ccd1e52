// qg_misc.hip -- the dequant dump, the per-row f16 scaling, SwiGLU, the weighted combine, the
// device routing plan and the GGUF block repack.
#include <algorithm>
#include <mutex>

#include "qgemm.h"
#include "qg_device.hpp"
#include "qg_internal.hpp"

namespace qg {

// ---- fixed scratch of the no-allocation MoE chain ---------------------------------------------------
// QG_NOALLOC_SCRATCH_BYTES of device memory in every GPU the library runs on, held until the process
// ends.  In host code `scratch` is a host-side stand-in, not a device address: host code only ever
// uses the address hipGetSymbolAddress gives for the current device, kept per device below.
static __device__ __align__(256) unsigned char scratch[QG_NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

// ---- dequant dump ------------------------------------------------------------------------------
// One thread per (row, block) of the requested tile.  It runs the same block load and decode the
// MFMA kernels run (load_block + block_to_f32 for exact mode, load_block + block_to_frags16 for
// fast mode) and writes element e of the block to out[r][32*bb + e].
template <int FMT, int ST>
__global__ void dequant_dump_kernel(const void* codes, const void* scales, const uint16_t* offs, int group, int K,
                                    int n0, int k0, int rows, int cols, void* out) {
    const int nb = cols >> 5;
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= rows * nb) return;
    const int r = idx / nb, bb = idx % nb;
    const RawBlock<FMT> raw = load_block<FMT>(codes, scales, offs, group, K, n0 + r, (k0 >> 5) + bb);
    if constexpr (ST == XT_F32) {
        float v[32];
        block_to_f32<FMT>(raw, v);
        float* o = (float*)out + (size_t)r * cols + 32 * bb;
#pragma unroll
        for (int e = 0; e < 32; e++) o[e] = v[e];
    } else {
        short8_t f[4];
        block_to_frags16<FMT, ST>(raw, f);
        uint16_t* o = (uint16_t*)out + (size_t)r * cols + 32 * bb;
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int s = 0; s < 8; s++) o[8 * j + s] = (uint16_t)f[j][s];
    }
}

template <int FMT>
static void dump_st(int staged, const void* codes, const void* scales, const uint16_t* offs, int group, int K,
                    int n0, int k0, int rows, int cols, void* out, hipStream_t s) {
    const int total = rows * (cols >> 5);
    dim3 grid((total + 255) / 256);
    if (staged == XT_F32)
        hipLaunchKernelGGL((dequant_dump_kernel<FMT, XT_F32>), grid, dim3(256), 0, s, codes, scales, offs, group, K,
                           n0, k0, rows, cols, out);
    else if (staged == XT_F16)
        hipLaunchKernelGGL((dequant_dump_kernel<FMT, XT_F16>), grid, dim3(256), 0, s, codes, scales, offs, group, K,
                           n0, k0, rows, cols, out);
    else
        hipLaunchKernelGGL((dequant_dump_kernel<FMT, XT_BF16>), grid, dim3(256), 0, s, codes, scales, offs, group, K,
                           n0, k0, rows, cols, out);
}

hipError_t launch_dequant_dump(int fmt, const void* codes, const void* scales, const uint16_t* offs, int group,
                               int N, int K, int n0, int k0, int rows, int cols, int staged, void* out,
                               hipStream_t s) {
    (void)N;
    if (fmt == FMT_Q4) dump_st<FMT_Q4>(staged, codes, scales, offs, group, K, n0, k0, rows, cols, out, s);
    else if (fmt == FMT_Q4A) dump_st<FMT_Q4A>(staged, codes, scales, offs, group, K, n0, k0, rows, cols, out, s);
    else if (fmt == FMT_Q8A) dump_st<FMT_Q8A>(staged, codes, scales, offs, group, K, n0, k0, rows, cols, out, s);
    else if (fmt == FMT_Q8A16) dump_st<FMT_Q8A16>(staged, codes, scales, offs, group, K, n0, k0, rows, cols, out, s);
    else dump_st<FMT_Q8>(staged, codes, scales, offs, group, K, n0, k0, rows, cols, out, s);
    return hipGetLastError();
}

// ---- block-wide max / helpers ---------------------------------------------------------------------
__device__ __forceinline__ float block_max256(float m, float* red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = m;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}


// ---- x_half: gathered per-row scaling to f16 -----------------------------------------------------
// guard < 0: the row's own power-of-two scale (page "oxinfer 0.0.5 src/metal.rs", row_scale /
// x_half); guard = s >= 0: the fixed scale 2^-s of a guarded half site (page "cortiq-engine 0.8.3
// src/gpu_metal/qi21.rs", Guards), with no pass over the row for its maximum.
__global__ __launch_bounds__(256) void x_half_kernel(const float* X, int x_rows, const int32_t* row_src, int K,
                                                      int guard, uint16_t* Xh, float* rs) {
    __shared__ float red[4];
    const int r = blockIdx.x;
    int s = row_src ? row_src[r] : r;
    const bool valid = s >= 0 && s < x_rows;
    const float4* row = (const float4*)(X + (size_t)(valid ? s : 0) * K);
    const int n4 = K >> 2;
    int e = -guard;
    if (guard < 0) {  // uniform over the workgroup
        float m = 0.f;
        if (valid)
            for (int i = threadIdx.x; i < n4; i += 256) {
                const float4 v = row[i];
                m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
            }
        m = block_max256(m, red);
        e = row_scale_exp(m);
    }
    const float sc = ldexpf(1.0f, e);
    uint2* out = (uint2*)(Xh + (size_t)r * K);
    for (int i = threadIdx.x; i < n4; i += 256) {
        float4 v = valid ? row[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        // f32 product, then nearest-even narrowing (keep_f32 stops a fused multiply-add with a +0
        // addend, which would turn -0 into +0, and a one-rounding mixed-precision form)
        const uint32_t a = (uint32_t)f32_to_f16_bits(keep_f32(v.x * sc)) |
                           ((uint32_t)f32_to_f16_bits(keep_f32(v.y * sc)) << 16);
        const uint32_t b = (uint32_t)f32_to_f16_bits(keep_f32(v.z * sc)) |
                           ((uint32_t)f32_to_f16_bits(keep_f32(v.w * sc)) << 16);
        out[i] = make_uint2(a, b);
    }
    if (threadIdx.x == 0 && rs) rs[r] = ldexpf(1.0f, -e);
}

hipError_t launch_x_half(const float* X, int x_rows, const int32_t* row_src, int R, int K, int guard, uint16_t* Xh,
                         float* rs, hipStream_t s) {
    hipLaunchKernelGGL(x_half_kernel, dim3(R), dim3(256), 0, s, X, x_rows, row_src, K, guard, Xh, rs);
    return hipGetLastError();
}

// ---- SwiGLU (page section silu_half): a = g / (1 + exp(-g)) * u ------------------------------------

__global__ __launch_bounds__(256) void swiglu_f32_kernel(const float* GU, int I, float* A) {
    const int r = blockIdx.x;
    const float4* g = (const float4*)(GU + (size_t)r * 2 * I);
    const float4* u = g + (I >> 2);
    float4* a = (float4*)(A + (size_t)r * I);
    for (int i = threadIdx.x; i < (I >> 2); i += 256) {
        const float4 gv = g[i], uv = u[i];
        a[i] = make_float4(silu_mul(gv.x, uv.x), silu_mul(gv.y, uv.y), silu_mul(gv.z, uv.z), silu_mul(gv.w, uv.w));
    }
}

__global__ __launch_bounds__(256) void swiglu_f16_kernel(const float* GU, int I, uint16_t* A, float* rs) {
    __shared__ float red[4];
    const int r = blockIdx.x;
    const float4* g = (const float4*)(GU + (size_t)r * 2 * I);
    const float4* u = g + (I >> 2);
    float m = 0.f;
    for (int i = threadIdx.x; i < (I >> 2); i += 256) {
        const float4 gv = g[i], uv = u[i];
        m = fmaxf(m, fmaxf(fmaxf(fabsf(silu_mul(gv.x, uv.x)), fabsf(silu_mul(gv.y, uv.y))),
                           fmaxf(fabsf(silu_mul(gv.z, uv.z)), fabsf(silu_mul(gv.w, uv.w)))));
    }
    m = block_max256(m, red);
    const int e = row_scale_exp(m);
    const float sc = ldexpf(1.0f, e);
    uint2* out = (uint2*)(A + (size_t)r * I);
    for (int i = threadIdx.x; i < (I >> 2); i += 256) {
        const float4 gv = g[i], uv = u[i];
        const uint32_t a = (uint32_t)f32_to_f16_bits(keep_f32(silu_mul(gv.x, uv.x) * sc)) |
                           ((uint32_t)f32_to_f16_bits(keep_f32(silu_mul(gv.y, uv.y) * sc)) << 16);
        const uint32_t b = (uint32_t)f32_to_f16_bits(keep_f32(silu_mul(gv.z, uv.z) * sc)) |
                           ((uint32_t)f32_to_f16_bits(keep_f32(silu_mul(gv.w, uv.w) * sc)) << 16);
        out[i] = make_uint2(a, b);
    }
    if (threadIdx.x == 0) rs[r] = ldexpf(1.0f, -e);
}

hipError_t launch_swiglu(const float* GU, int R, int I, void* A, int at, float* rs, hipStream_t s) {
    if (R <= 0) return hipSuccess;
    if (at == XT_F32)
        hipLaunchKernelGGL(swiglu_f32_kernel, dim3(R), dim3(256), 0, s, GU, I, (float*)A);
    else
        hipLaunchKernelGGL(swiglu_f16_kernel, dim3(R), dim3(256), 0, s, GU, I, (uint16_t*)A, rs);
    return hipGetLastError();
}

// ---- weighted combine (page section moe_combine), f32 in slot order --------------------------------
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* O, int R, const int32_t* slot_row,
                                                           const float* slot_w, float* Y, int H, int k,
                                                           int accumulate) {
    const int t = blockIdx.y;
    const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (c >= H) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; j++) {
        const int row = slot_row[t * k + j];
        if (row < 0 || row >= R) continue;
        const float w = slot_w[t * k + j];
        const float4 o = *(const float4*)(O + (size_t)row * H + c);
        acc.x += w * o.x;
        acc.y += w * o.y;
        acc.z += w * o.z;
        acc.w += w * o.w;
    }
    float4* y = (float4*)(Y + (size_t)t * H + c);
    if (accumulate) {
        const float4 p = *y;
        acc.x += p.x;
        acc.y += p.y;
        acc.z += p.z;
        acc.w += p.w;
    }
    *y = acc;
}

hipError_t launch_moe_combine(const float* O, int R, const int32_t* slot_row, const float* slot_w, float* Y, int H,
                              int T, int k, int accumulate, hipStream_t s) {
    dim3 grid((H / 4 + 255) / 256, T);
    hipLaunchKernelGGL(moe_combine_kernel, grid, dim3(256), 0, s, O, R, slot_row, slot_w, Y, H, k, accumulate);
    return hipGetLastError();
}

}  // namespace qg

namespace qg {

// ---- routing plan on the device ----------------------------------------------------------------
// Pages: "cortiq-engine 0.8.44 src/gpu_metal/clover.rs", coreset_from_logits (top-k of a token's
// router logits, ties to the lower expert index) and the renormalised weights of its route step;
// "oxinfer 0.0.5 src/metal.rs", Backend::moe (rows grouped per expert, tokens ascending).  The
// pages build this on the host; here one workgroup builds it on the device, so a caller can chain
// it with the grouped matmuls without a round trip.  Same outputs as the host plan:
//  1. one wavefront per token: k rounds of a wavefront argmax under (larger logit, then lower
//     index) over the logits held in registers -- two DPP reductions, the largest order-preserving
//     key and then the lowest index holding it (a NaN logit ranks as -inf and sets the error
//     flag); lane j keeps the j-th pick; weight_j = exp(l_j - l_max) / sum_i exp(l_i - l_max)
//     in f64, summed in pick order, rounded to f32; the pick's expert is kept in LDS;
//  2. per-expert counts (LDS integer atomics) and their inclusive scan -> seg_off;
//  3. one wavefront per expert walks the slots in token order, 64 at a time: the ballot of slots
//     that picked it and their popcount ranks give each slot its gathered row, in ascending token
//     order; row_src[row] = token, slot_row[slot] = row.
// The kernel is instantiated for NPL = 1, 2, 4, 8, 16 logits per lane (E <= 64 NPL): each top-k
// round scans only the lane's NPL candidates (the rounds run on one CU's VALUs, so a fixed 16 cost
// E = 128 most of its time).  In step 3 a wavefront skips experts without slots and stops an
// expert's walk once its count is reached.
constexpr int kPlanThreads = 1024;
constexpr int kPlanNplMax = 16;      // logits per lane: E <= 1024
constexpr int kPlanSlots = 16384;    // T * k: the picks live in LDS (32 KiB)

// Order-preserving 32-bit image of a logit (larger value, larger key; -0 taken as +0 so that equal
// values compare equal); 0 lies below the key of every value, -inf included.
__device__ __forceinline__ uint32_t plan_key(float x) {
    const uint32_t u = __float_as_uint(x == 0.f ? 0.f : x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float plan_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
// Wavefront maximum / minimum, the same in every lane: DPP row shifts by 1, 2, 4 and 8 leave each
// row's extreme in its lane 15, the row-15 and row-31 broadcasts carry them to lane 63, which is read
// back.  Lanes without a source keep the identity (0 for the maximum, ~0 for the minimum).
__device__ __forceinline__ uint32_t wave_umax32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_umin32(uint32_t v) {
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x111, 0xF, 0xF, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x112, 0xF, 0xF, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x114, 0xF, 0xF, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x118, 0xF, 0xF, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x142, 0xA, 0xF, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x143, 0xC, 0xF, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

template <int NPL>
__global__ __launch_bounds__(kPlanThreads) void moe_plan_kernel(const float* logits, int T, int E, int k,
                                                                int32_t* seg_off, int32_t* row_src, int32_t* slot_row,
                                                                float* slot_w, int32_t* slot_expert, int32_t* status,
                                                                int32_t err_code) {
    __shared__ int cnt[NPL * 64 + 1];
    __shared__ uint16_t pick[kPlanSlots];
    __shared__ int bad;
    constexpr int W = kPlanThreads / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tk = T * k;
    for (int e = tid; e <= E; e += kPlanThreads) cnt[e] = 0;
    if (tid == 0) bad = 0;
    __syncthreads();

    for (int t = wave; t < T; t += W) {
        const float* row = logits + (size_t)t * E;
        float v[NPL];
        uint32_t taken = 0;  // bit i: candidate lane + 64 i is gone (picked, or past E)
        bool nan_seen = false;
#pragma unroll
        for (int i = 0; i < NPL; i++) {
            const int e = lane + 64 * i;
            v[i] = -INFINITY;
            if (e < E) {
                const float x = row[e];
                if (x != x)
                    nan_seen = true;
                else
                    v[i] = x;
            } else {
                taken |= 1u << i;
            }
        }
        if (__any(nan_seen) && lane == 0) bad = 1;
        int my_e = 0;
        float my_v = 0.f;
        for (int j = 0; j < k; j++) {
            // the lane's best untaken candidate (ascending index, so the lowest index among equal
            // keys), then the wavefront's largest key and the lowest index holding it
            uint32_t bk = 0;
            int bi = 0x7fffffff;
#pragma unroll
            for (int i = 0; i < NPL; i++) {
                const uint32_t key = ((taken >> i) & 1u) ? 0u : plan_key(v[i]);
                if (key > bk) {
                    bk = key;
                    bi = lane + 64 * i;
                }
            }
            const uint32_t kmax = wave_umax32(bk);
            // j < k <= E: an untaken real candidate remains, so kmax > 0 and the winner is < E
            const int win = (int)wave_umin32(bk == kmax ? (uint32_t)bi : 0xFFFFFFFFu);
            if ((win & 63) == lane) taken |= 1u << (win >> 6);
            if (lane == j) {
                my_e = win;
                my_v = plan_value(kmax);
            }
        }
        const double lmax = (double)__shfl(my_v, 0, 64);
        const double ex = lane < k ? exp((double)my_v - lmax) : 0.0;
        double sum = 0.0;
        for (int j = 0; j < k; j++) sum += __shfl(ex, j, 64);
        if (lane < k) {
            const size_t s = (size_t)t * k + lane;
            slot_w[s] = (float)(ex / sum);
            pick[s] = (uint16_t)my_e;
            if (slot_expert) slot_expert[s] = my_e;
            atomicAdd(&cnt[my_e + 1], 1);
        }
    }
    __syncthreads();

    if (wave == 0) {  // inclusive scan of the counts: cnt[e] = seg_off[e]
        int carry = 0;
        for (int c0 = 1; c0 <= E; c0 += 64) {
            const int e = c0 + lane;
            int x = e <= E ? cnt[e] : 0;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(x, o, 64);
                if (lane >= o) x += y;
            }
            x += carry;
            if (e <= E) cnt[e] = x;
            carry = __shfl(x, 63, 64);
        }
    }
    if (tid == 0 && status) status[0] = bad ? err_code : 0;
    __syncthreads();
    for (int e = tid; e <= E; e += kPlanThreads) seg_off[e] = cnt[e];

    for (int e = wave; e < E; e += W) {
        int base = cnt[e];
        const int end = cnt[e + 1];
        for (int c = 0; c < tk && base < end; c += 64) {
            const int i = c + lane;
            const bool match = i < tk && pick[i] == e;
            const uint64_t mask = __ballot(match);
            if (match) {
                const int pos = base + __popcll(mask & ((1ull << lane) - 1ull));
                row_src[pos] = i / k;
                slot_row[i] = pos;
            }
            base += __popcll(mask);
        }
    }
}

hipError_t launch_moe_plan(const float* logits, int T, int E, int k, int32_t* seg_off, int32_t* row_src,
                           int32_t* slot_row, float* slot_w, int32_t* slot_expert, int32_t* status, int err_code,
                           hipStream_t s) {
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(1), dim3(kPlanThreads), 0, s, logits, T, E, k, seg_off, row_src, slot_row,
                           slot_w, slot_expert, status, err_code);
    };
    if (E <= 64) go(moe_plan_kernel<1>);
    else if (E <= 128) go(moe_plan_kernel<2>);
    else if (E <= 256) go(moe_plan_kernel<4>);
    else if (E <= 512) go(moe_plan_kernel<8>);
    else go(moe_plan_kernel<kPlanNplMax>);
    return hipGetLastError();
}

}  // namespace qg

namespace qg {

// ---- GGUF blocks with in-block scales -> the split layout ------------------------------------------
// Page "oxinfer 0.0.5 src/metal.rs", SHADER_SRC, the GGUF dequantizers Q4_0W and Q8_0W: a row is
// K/32 blocks; Q4_0 = f16 scale then 16 nibble bytes (18 bytes), Q8_0 = f16 scale then 32 signed
// bytes (34 bytes); their values are those of Q4 and Q8 with the same codes and scale.  The repack
// is exact: code bytes are copied, the f16 scale is copied (Q4) or widened to f32 (Q8).  One thread
// per block, consecutive threads on consecutive blocks; blocks are 2-byte aligned, so they are read
// as 16-bit words.
template <int QB>  // code bytes per block: 16 (Q4_0) or 32 (Q8_0)
__global__ void repack_gguf_kernel(const uint16_t* src, size_t nblocks, uint8_t* codes, void* scales) {
    constexpr int W = 1 + QB / 2;  // 16-bit words per block
    for (size_t b = (size_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblocks; b += (size_t)gridDim.x * blockDim.x) {
        const uint16_t* B = src + b * W;
        uint32_t w[QB / 4];
#pragma unroll
        for (int i = 0; i < QB / 4; i++) w[i] = (uint32_t)B[1 + 2 * i] | ((uint32_t)B[2 + 2 * i] << 16);
        uint4* dst = (uint4*)(codes + b * QB);
#pragma unroll
        for (int i = 0; i < QB / 16; i++) dst[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
        if constexpr (QB == 16)
            ((uint16_t*)scales)[b] = B[0];
        else
            ((float*)scales)[b] = f16_to_f32(B[0]);
    }
}

// ---- normalisation statistics of the convolution input ---------------------------------------------
// Page "oxinfer 0.0.5 src/metal.rs", group_stats and row_stats: two passes, the mean first, then the
// mean squared deviation from it; rstd = 1 / sqrt(var + eps).  Group statistics: one workgroup of
// 1024 threads per group walks the group's npix x cpg values (consecutive threads on consecutive
// values: a pixel's cpg channels are contiguous), the (pixel, channel) position advanced by
// additions instead of a division per value; per-pixel statistics: one wavefront per pixel over its
// cin channels.  f32 sums: each thread strided, then the wavefront by xor shuffles, then the
// wavefronts through LDS in a fixed order.
constexpr int kStatsThreads = 1024;

__device__ __forceinline__ float block_sum_stats(float v, float* red) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kStatsThreads / 64; w++) t += red[w];
    return t;
}

template <bool DEV>
__device__ __forceinline__ float group_pass(const float* X, int npix, int cin, int cpg, int g, float mean) {
    const float* base = X + (size_t)g * cpg;
    if (kStatsThreads % cpg == 0) {
        // cpg divides the thread count: every thread keeps one channel and strides over the pixels,
        // so its loads are independent and go out eight at a time
        const int P = kStatsThreads / cpg, j = threadIdx.x % cpg;
        float s = 0.f;
#pragma unroll 8
        for (int q = threadIdx.x / cpg; q < npix; q += P) {
            const float x = base[(size_t)q * cin + j];
            if constexpr (DEV) {
                const float d = x - mean;
                s += d * d;
            } else {
                s += x;
            }
        }
        return s;
    }
    // thread t starts at value t of the group: pixel t / cpg, channel t % cpg, and steps by 1024
    const int dq = kStatsThreads / cpg, dj = kStatsThreads % cpg;
    int q = threadIdx.x / cpg, j = threadIdx.x % cpg;
    float s = 0.f;
    while (q < npix) {
        const float x = base[(size_t)q * cin + j];
        if constexpr (DEV) {
            const float d = x - mean;
            s += d * d;
        } else {
            s += x;
        }
        q += dq;
        j += dj;
        if (j >= cpg) {
            j -= cpg;
            q += 1;
        }
    }
    return s;
}

__global__ __launch_bounds__(kStatsThreads) void conv_group_stats_kernel(const float* X, int npix, int cin, int cpg,
                                                                         float eps, float* stats) {
    __shared__ float red[kStatsThreads / 64];
    const int g = blockIdx.x;
    const float total = (float)npix * (float)cpg;
    const float mean = block_sum_stats(group_pass<false>(X, npix, cin, cpg, g, 0.f), red) / total;
    const float var = block_sum_stats(group_pass<true>(X, npix, cin, cpg, g, mean), red) / total;
    if (threadIdx.x == 0) {
        stats[2 * g] = mean;
        stats[2 * g + 1] = 1.0f / sqrtf(var + eps);
    }
}

__global__ __launch_bounds__(256) void conv_pixel_stats_kernel(const float* X, int npix, int cin, float eps,
                                                               float* stats) {
    const int q = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (q >= npix) return;  // wave-uniform: the wavefront's pixel
    const float* row = X + (size_t)q * cin;
    float s = 0.f;
    for (int c = lane; c < cin; c += 64) s += row[c];
    const float mean = wave_sum(s) / (float)cin;
    float v = 0.f;
    for (int c = lane; c < cin; c += 64) {
        const float d = row[c] - mean;
        v += d * d;
    }
    const float var = wave_sum(v) / (float)cin;
    if (lane == 0) {
        stats[2 * q] = mean;
        stats[2 * q + 1] = 1.0f / sqrtf(var + eps);
    }
}

hipError_t launch_conv_stats(const float* X, int npix, int cin, int groups, float eps, float* stats, hipStream_t s) {
    if (groups > 0)
        hipLaunchKernelGGL(conv_group_stats_kernel, dim3(groups), dim3(kStatsThreads), 0, s, X, npix, cin,
                           cin / groups, eps, stats);
    else
        hipLaunchKernelGGL(conv_pixel_stats_kernel, dim3((npix + 3) / 4), dim3(256), 0, s, X, npix, cin, eps, stats);
    return hipGetLastError();
}

// ---- GGUF affine blocks -> Q8A ----------------------------------------------------------------------
// Page "oxinfer 0.0.5 src/metal.rs", GGUF_SHADER_SRC, the loaders of Q4_1, Q5_0, Q5_1 (load_q45) and
// Q4_K (with its 6-bit scale / min unpacking).  Each of these types gives element e of a 32-element
// block (a sub-block for Q4_K) as an integer code times an f32 scale plus an f32 offset, evaluated
// product first, then the add: Q4_1 nibble * d + m, Q5_0 (code5 - 16) * d (+ 0), Q5_1 code5 * d + m,
// Q4_K nibble * (d sc) - dmin mn.  Q8A holds exactly that: int8 codes, the scale and the offset in
// f32 (Q5_0: codes - 16 and offset +0; Q4_K: scale d sc and offset -(dmin mn), both rounded once as
// the loader rounds them).  Field layout, little-endian, f16 fields as h:
//   Q4_1 20 B: h d, h m, 16 bytes (byte j: element j low nibble, element j + 16 high nibble)
//   Q5_0 22 B: h d, 32-bit qh (bit e: 16s bit of element e), 16 nibble bytes as Q4_1
//   Q5_1 24 B: h d, h m, qh, 16 nibble bytes
//   Q4_K 144 B per 256 elements: h d, h dmin, 12 scale bytes, 128 code bytes; sub-block j's
//        elements are the low (j even) or high (j odd) nibbles of code bytes 32 (j / 2) .. + 31.
//   Q5_K 176 B per 256 elements (loader Q5_KW): h d, h dmin, the 12 scale bytes, 32 bytes qh, 128 code
//        bytes; as Q4_K with a fifth code bit, bit j of qh[e] for element e of sub-block j.
// One thread per output block, consecutive threads on consecutive blocks of a row-major [N][K/32]
// block grid (blocks are 2-byte aligned: read as 16-bit words).
template <int GT>
__global__ void repack_gguf_q8a_kernel(const uint16_t* src, size_t nblocks, uint8_t* codes, float* scales,
                                       float* offs) {
    for (size_t b = (size_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblocks; b += (size_t)gridDim.x * blockDim.x) {
        uint8_t nib[32];  // element e's code before any shift
        float d, m;
        if constexpr (GT == QG_GGUF_Q4_K || GT == QG_GGUF_Q5_K) {
            constexpr bool q5 = GT == QG_GGUF_Q5_K;
            const uint16_t* SB = src + (b >> 3) * (q5 ? 88 : 72);  // 176- / 144-byte super-block
            const int j = (int)(b & 7);
            uint8_t sb[12];
#pragma unroll
            for (int i = 0; i < 6; i++) {
                sb[2 * i] = (uint8_t)SB[2 + i];
                sb[2 * i + 1] = (uint8_t)(SB[2 + i] >> 8);
            }
            int sc, mn;
            if (j < 4) {
                sc = sb[j] & 63;
                mn = sb[j + 4] & 63;
            } else {
                sc = (sb[j + 4] & 15) | ((sb[j - 4] >> 6) << 4);
                mn = (sb[j + 4] >> 4) | ((sb[j] >> 6) << 4);
            }
            d = f16_to_f32(SB[0]) * (float)sc;
            m = -(f16_to_f32(SB[1]) * (float)mn);
            const uint16_t* q = SB + (q5 ? 24 : 8) + 16 * (j >> 1);
            const int sh = 4 * (j & 1);
#pragma unroll
            for (int i = 0; i < 16; i++) {
                nib[2 * i] = (uint8_t)((q[i] >> sh) & 15);
                nib[2 * i + 1] = (uint8_t)((q[i] >> (8 + sh)) & 15);
            }
            if constexpr (q5) {
                const uint16_t* qh = SB + 8;  // bytes 16 .. 47
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    nib[2 * i] = (uint8_t)(nib[2 * i] | (((qh[i] >> j) & 1) << 4));
                    nib[2 * i + 1] = (uint8_t)(nib[2 * i + 1] | (((qh[i] >> (8 + j)) & 1) << 4));
                }
            }
        } else {
            constexpr bool has_m = GT == QG_GGUF_Q4_1 || GT == QG_GGUF_Q5_1;
            constexpr bool has_h = GT == QG_GGUF_Q5_0 || GT == QG_GGUF_Q5_1;
            constexpr int W = (2 + (has_m ? 2 : 0) + (has_h ? 4 : 0) + 16) / 2;  // 16-bit words per block
            const uint16_t* B = src + b * W;
            d = f16_to_f32(B[0]);
            m = has_m ? f16_to_f32(B[1]) : 0.0f;
            constexpr int qo = 1 + (has_m ? 1 : 0) + (has_h ? 2 : 0);  // word of the first nibble byte
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const uint16_t w = B[qo + i];
                nib[2 * i] = (uint8_t)(w & 15);
                nib[2 * i + 1] = (uint8_t)((w >> 8) & 15);
                nib[16 + 2 * i] = (uint8_t)((w >> 4) & 15);
                nib[17 + 2 * i] = (uint8_t)(w >> 12);
            }
            if constexpr (has_h) {
                constexpr int ho = 1 + (has_m ? 1 : 0);
                const uint32_t qh = (uint32_t)B[ho] | ((uint32_t)B[ho + 1] << 16);
#pragma unroll
                for (int e = 0; e < 32; e++) nib[e] = (uint8_t)(nib[e] + 16 * ((qh >> e) & 1));
            }
            if constexpr (GT == QG_GGUF_Q5_0) {
#pragma unroll
                for (int e = 0; e < 32; e++) nib[e] = (uint8_t)(nib[e] - 16);  // int8 code - 16
            }
        }
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; i++)
            w[i] = (uint32_t)nib[4 * i] | ((uint32_t)nib[4 * i + 1] << 8) | ((uint32_t)nib[4 * i + 2] << 16) |
                   ((uint32_t)nib[4 * i + 3] << 24);
        uint4* dst = (uint4*)(codes + b * 32);
        dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
        dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
        scales[b] = d;
        offs[b] = m;
    }
}

hipError_t launch_repack_gguf_q8a(int type, const void* src, size_t nblocks, void* codes, float* scales,
                                  float* offs, hipStream_t s) {
    const unsigned grid = (unsigned)std::min<size_t>((nblocks + 255) / 256, 65535);
    const uint16_t* w = (const uint16_t*)src;
    uint8_t* c = (uint8_t*)codes;
    switch (type) {
        case QG_GGUF_Q4_1:
            hipLaunchKernelGGL(repack_gguf_q8a_kernel<QG_GGUF_Q4_1>, dim3(grid), dim3(256), 0, s, w, nblocks, c,
                               scales, offs);
            break;
        case QG_GGUF_Q5_0:
            hipLaunchKernelGGL(repack_gguf_q8a_kernel<QG_GGUF_Q5_0>, dim3(grid), dim3(256), 0, s, w, nblocks, c,
                               scales, offs);
            break;
        case QG_GGUF_Q5_1:
            hipLaunchKernelGGL(repack_gguf_q8a_kernel<QG_GGUF_Q5_1>, dim3(grid), dim3(256), 0, s, w, nblocks, c,
                               scales, offs);
            break;
        case QG_GGUF_Q4_K:
            hipLaunchKernelGGL(repack_gguf_q8a_kernel<QG_GGUF_Q4_K>, dim3(grid), dim3(256), 0, s, w, nblocks, c,
                               scales, offs);
            break;
        case QG_GGUF_Q5_K:
            hipLaunchKernelGGL(repack_gguf_q8a_kernel<QG_GGUF_Q5_K>, dim3(grid), dim3(256), 0, s, w, nblocks, c,
                               scales, offs);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---- GGUF K-quants with a scale per 16 elements -> Q8A16 ------------------------------------------
// Page "oxinfer 0.0.5 src/metal.rs", GGUF_SHADER_SRC (loaders Q6_KW, Q3_KW, Q2_KW).  256 elements per
// super-block; 32-element sub-block j has half n = j / 4 and position jj = j % 4; its element e lies
// in 16-element block s16 = 8 n + 2 jj + e / 16.  Field layout, little-endian, h = f16 as f32:
//   Q6_K 210 B: 128 B ql, 64 B qh, 16 int8 scales, h d.  Code = (nibble of ql[64 n + 32 (jj % 2) + e]
//        (high for jj >= 2) | bits 2 jj .. 2 jj + 1 of qh[32 n + e] << 4) - 32; scale d * sc[s16].
//   Q3_K 110 B: 32 B hmask, 64 B qs, 12 scale bytes, h d.  Code = bits 2 jj .. of qs[32 n + e], minus
//        4 when bit 4 n + jj of hmask[e] is clear; 6-bit scale of s16 = low four bits from byte s16
//        (s16 < 8, low nibble) or s16 - 8 (high nibble), top two bits from byte 8 + s16 % 4 at bit
//        2 (s16 / 4); scale d * (that - 32).
//   Q2_K 84 B: 16 scale bytes s, 64 B qs, h d, h dmin.  Code = bits 2 jj .. of qs[32 n + e]; scale
//        d * (s[s16] & 15), offset -(dmin * (s[s16] >> 4)).
// The pages evaluate code * scale (Q2_K: minus the min) in f32; every product here is exact, and
// Q8A16 computes fl(fl(code * scale) + offset) -- with offset -0 for Q6_K and Q3_K, which leaves
// every value, zeros' signs included, as the page computes it.  One thread per 16-element block:
// the block index in a row-major [N][K / 16] grid is (super-block) * 16 + s16.
template <int GT>
__global__ void repack_gguf_q8a16_kernel(const uint8_t* src, size_t nblk16, uint8_t* codes, float* scales,
                                         float* offs) {
    constexpr int SBB = GT == QG_GGUF_Q6_K ? 210 : GT == QG_GGUF_Q3_K ? 110 : 84;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nblk16; i += (size_t)gridDim.x * blockDim.x) {
        const uint8_t* SB = src + (i >> 4) * SBB;
        const int s16 = (int)(i & 15), half = s16 >> 3, pos = (s16 & 7) >> 1, e0 = 16 * (s16 & 1);
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        float d, m;
        if constexpr (GT == QG_GGUF_Q6_K) {
            d = f16_to_f32((uint16_t)(SB[208] | (SB[209] << 8))) * (float)(int8_t)SB[192 + s16];
            m = -0.0f;
            const uint8_t* ql = SB + 64 * half + 32 * (pos & 1) + e0;
            const uint8_t* qh = SB + 128 + 32 * half + e0;
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int low = pos >= 2 ? (ql[e] >> 4) : (ql[e] & 15);
                const int code = (low | (((qh[e] >> (2 * pos)) & 3) << 4)) - 32;
                w[e >> 2] |= (uint32_t)(uint8_t)(int8_t)code << (8 * (e & 3));
            }
        } else if constexpr (GT == QG_GGUF_Q3_K) {
            const int lo = s16 < 8 ? (SB[96 + s16] & 15) : (SB[96 + s16 - 8] >> 4);
            const int hi = (SB[104 + (s16 & 3)] >> (2 * (s16 >> 2))) & 3;
            d = f16_to_f32((uint16_t)(SB[108] | (SB[109] << 8))) * (float)((lo | (hi << 4)) - 32);
            m = -0.0f;
            const uint8_t* qs = SB + 32 + 32 * half + e0;
            const uint8_t* hm = SB + e0;
#pragma unroll
            for (int e = 0; e < 16; e++) {
                int code = (qs[e] >> (2 * pos)) & 3;
                if (!((hm[e] >> (4 * half + pos)) & 1)) code -= 4;
                w[e >> 2] |= (uint32_t)(uint8_t)(int8_t)code << (8 * (e & 3));
            }
        } else {
            const int sc = SB[s16];
            d = f16_to_f32((uint16_t)(SB[80] | (SB[81] << 8))) * (float)(sc & 15);
            m = -(f16_to_f32((uint16_t)(SB[82] | (SB[83] << 8))) * (float)(sc >> 4));
            const uint8_t* qs = SB + 16 + 32 * half + e0;
#pragma unroll
            for (int e = 0; e < 16; e++) w[e >> 2] |= (uint32_t)((qs[e] >> (2 * pos)) & 3) << (8 * (e & 3));
        }
        // the 16 codes of block i sit at byte 16 i of the row-major codes
        *(u32x4_t*)(codes + 16 * i) = u32x4_t{w[0], w[1], w[2], w[3]};
        scales[i] = d;
        if (offs) offs[i] = m;  // uniform: NULL for the offset-free layout (Q6_K, Q3_K)
    }
}

hipError_t launch_repack_gguf_q8a16(int type, const void* src, size_t nblk16, void* codes, float* scales,
                                    float* offs, hipStream_t s) {
    const unsigned grid = (unsigned)std::min<size_t>((nblk16 + 255) / 256, 65535);
    const uint8_t* b = (const uint8_t*)src;
    uint8_t* c = (uint8_t*)codes;
    switch (type) {
        case QG_GGUF_Q6_K:
            hipLaunchKernelGGL(repack_gguf_q8a16_kernel<QG_GGUF_Q6_K>, dim3(grid), dim3(256), 0, s, b, nblk16, c,
                               scales, offs);
            break;
        case QG_GGUF_Q3_K:
            hipLaunchKernelGGL(repack_gguf_q8a16_kernel<QG_GGUF_Q3_K>, dim3(grid), dim3(256), 0, s, b, nblk16, c,
                               scales, offs);
            break;
        case QG_GGUF_Q2_K:
            hipLaunchKernelGGL(repack_gguf_q8a16_kernel<QG_GGUF_Q2_K>, dim3(grid), dim3(256), 0, s, b, nblk16, c,
                               scales, offs);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---- q8_2f / q8_row: row scale into Q8 block scales; the column field applied to X ---------------
// Page "cortiq-engine 0.8.3 src/gpu_metal/qi21.rs" (the block loader's codec match: int8 codes
// [N][K], then f16 row scales [N], then, for q8_2f, the f16 column field [K]) and page
// "cortiq-engine 0.8.41 src/gpu_metal/clover.rs" (q8mm: the column field multiplies X as it is
// staged, the row scale multiplies the result).  The codes stay where they are (they already are the
// Q8 code layout); block scale (n, b) becomes the f32 row scale of row n, so the Q8 kernels apply
// it per block; the column field goes to f32 for qg_col_scale.
__global__ __launch_bounds__(256) void repack_q8f_kernel(const uint16_t* rs, const uint16_t* col, int N, int nb,
                                                         int K, float* scales, float* colf) {
    const size_t total = (size_t)N * nb;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total + (col ? (size_t)K : 0);
         i += (size_t)gridDim.x * 256) {
        if (i < total) scales[i] = f16_to_f32(rs[i / nb]);
        else colf[i - total] = f16_to_f32(col[i - total]);
    }
}

hipError_t launch_repack_q8f(const void* blob, int N, int K, bool has_col, float* scales, float* col, hipStream_t s) {
    const uint8_t* b = (const uint8_t*)blob;
    const uint16_t* rs = (const uint16_t*)(b + (size_t)N * K);
    const uint16_t* cf = has_col ? rs + N : nullptr;
    const size_t total = (size_t)N * (K / 32) + (has_col ? K : 0);
    const unsigned grid = (unsigned)std::min<size_t>((total + 255) / 256, 65535);
    hipLaunchKernelGGL(repack_q8f_kernel, dim3(grid), dim3(256), 0, s, rs, cf, N, K / 32, K, scales, col);
    return hipGetLastError();
}

// Xs[t][k] = x[t][k] col[k]: the f32 product, then (f16 / bf16 output) nearest-even narrowing.
// Eight values per thread and step (16-byte loads of f16 / bf16 X, two of f32).
template <int XT, int ST>
__global__ __launch_bounds__(256) void col_scale_kernel(const void* X, const float* col, int K, size_t n8,
                                                        void* Xs) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (size_t)gridDim.x * 256) {
        const int k0 = (int)((i * 8) % (size_t)K);
        float v[8];
        if constexpr (XT == XT_F32) {
            const float4 a = ((const float4*)X)[2 * i], b = ((const float4*)X)[2 * i + 1];
            v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
        } else {
            const uint4 q = ((const uint4*)X)[i];
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const uint16_t h = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
                v[j] = XT == XT_F16 ? f16_to_f32(h) : bf16_to_f32(h);
            }
        }
        const float4 c0 = *(const float4*)(col + k0), c1 = *(const float4*)(col + k0 + 4);
        const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
        for (int j = 0; j < 8; j++) v[j] = keep_f32(v[j] * c[j]);
        if constexpr (ST == XT_F32) {
            ((float4*)Xs)[2 * i] = make_float4(v[0], v[1], v[2], v[3]);
            ((float4*)Xs)[2 * i + 1] = make_float4(v[4], v[5], v[6], v[7]);
        } else {
            uint32_t o[4];
#pragma unroll
            for (int j = 0; j < 4; j++)
                o[j] = (uint32_t)f32_to_16<ST>(v[2 * j]) | ((uint32_t)f32_to_16<ST>(v[2 * j + 1]) << 16);
            ((uint4*)Xs)[i] = make_uint4(o[0], o[1], o[2], o[3]);
        }
    }
}

template <int XT>
static void col_scale_st(const void* X, const float* col, int K, size_t n8, void* Xs, int st, unsigned grid,
                         hipStream_t s) {
    if (st == XT_F32) hipLaunchKernelGGL((col_scale_kernel<XT, XT_F32>), dim3(grid), dim3(256), 0, s, X, col, K, n8, Xs);
    else if (st == XT_F16)
        hipLaunchKernelGGL((col_scale_kernel<XT, XT_F16>), dim3(grid), dim3(256), 0, s, X, col, K, n8, Xs);
    else hipLaunchKernelGGL((col_scale_kernel<XT, XT_BF16>), dim3(grid), dim3(256), 0, s, X, col, K, n8, Xs);
}

hipError_t launch_col_scale(const void* X, int xt, int T, int K, const float* col, void* Xs, int st, hipStream_t s) {
    const size_t n8 = (size_t)T * K / 8;
    const unsigned grid = (unsigned)std::min<size_t>((n8 + 255) / 256, 8192);
    if (xt == XT_F32) col_scale_st<XT_F32>(X, col, K, n8, Xs, st, grid, s);
    else if (xt == XT_F16) col_scale_st<XT_F16>(X, col, K, n8, Xs, st, grid, s);
    else col_scale_st<XT_BF16>(X, col, K, n8, Xs, st, grid, s);
    return hipGetLastError();
}

hipError_t launch_repack_gguf(int q8, const void* src, size_t nblocks, void* codes, void* scales, hipStream_t s) {
    const unsigned grid = (unsigned)std::min<size_t>((nblocks + 255) / 256, 65535);
    if (q8)
        hipLaunchKernelGGL(repack_gguf_kernel<32>, dim3(grid), dim3(256), 0, s, (const uint16_t*)src, nblocks,
                           (uint8_t*)codes, scales);
    else
        hipLaunchKernelGGL(repack_gguf_kernel<16>, dim3(grid), dim3(256), 0, s, (const uint16_t*)src, nblocks,
                           (uint8_t*)codes, scales);
    return hipGetLastError();
}

}  // namespace qg
