// qg_internal.hpp -- launch parameters shared by the host entry points and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qg {

struct ExpertPtr {
    const void* codes;
    const void* scales;
    const uint16_t* offsets;
};

// One matmul launch: either dense (one weight matrix, rows 0..R-1 of X) or grouped (an expert
// table and the row segments seg_off[e]..seg_off[e+1]-1 of each expert).
struct GemmParams {
    const void* codes;           // dense weights
    const void* scales;
    const uint16_t* offs;
    const ExpertPtr* experts;    // grouped: device table [E]
    const int32_t* seg_off;      // grouped: device [E+1]
    const int32_t* row_src;      // optional: X row of output row r
    const void* X;
    const float* rs;             // optional per-row output scale
    float* Y;                    // [R][N]
    int group;
    int N, K;
    int R;                       // output rows (dense: T)
    int E;                       // grouped: experts
    int x_rows;                  // rows of X (bounds for row_src)
};

// Convolution as an implicit GEMM (page "oxinfer 0.0.5 src/metal.rs", SHADER_SRC conv_body / CP):
// output row r of the GEMM is output pixel r = oy * ow + ox, K runs over (ky, kx, ci), and X is the
// image [H][W][cin] in f32.  norm 1: group norm with stats[c / cpg]; 2: layer norm with stats[input
// pixel]; stats are (mean, rstd) f32 pairs, gb gamma[cin] then beta[cin]; silu applies SiLU after.
struct ConvParams {
    int H, W, cin, ksz, stride, pad, ow;
    int norm, cpg, silu;
    const float* stats;
    const float* gb;
};

// Several weight matrices sharing one X row in one T = 1 launch: job j owns the global output rows
// [start[j], start[j+1]) and writes them to Y[j] (page "oxinfer 0.0.5 src/metal.rs",
// Backend::matmul, whose jobs share X).  Passed by value in the kernel arguments.
constexpr int kMaxBatchJobs = 8;
struct BatchJobs {
    int J;
    int start[kMaxBatchJobs + 1];
    const void* codes[kMaxBatchJobs];
    const void* scales[kMaxBatchJobs];
    const uint16_t* offs[kMaxBatchJobs];
    float* Y[kMaxBatchJobs];
};

// Kernel launchers; each returns a hipError_t from hipGetLastError after the launch.
hipError_t launch_gemm_fast(int fmt, int st, const GemmParams& p, bool grouped, hipStream_t s);
hipError_t launch_gemm_exact(int fmt, int xt, const GemmParams& p, bool grouped, hipStream_t s);
// The convolution through the exact kernel (f32 X gathered per tap; Q4 / Q8 weights); p.R = oh * ow
// output pixels, p.N output channels, p.K = ksz * ksz * cin.
hipError_t launch_conv_exact(int fmt, const GemmParams& p, const ConvParams& cv, hipStream_t s);
// (mean, rstd) pairs of the image [npix][cin]: groups > 0 per group (all pixels, cin / groups
// channels), groups == 0 per pixel.
hipError_t launch_conv_stats(const float* X, int npix, int cin, int groups, float eps, float* stats, hipStream_t s);
// Dense fast matmul with the weights kept exact (Q4 / Q8 codes as f16, f16 X, block scale on the f32
// block partial); hipErrorInvalidValue for another format.
hipError_t launch_gemm_fast_wexact(int fmt, const GemmParams& p, hipStream_t s);
hipError_t launch_gemv(int fmt, int xt, const GemmParams& p, bool grouped, hipStream_t s);
// T = 1, K <= 16384: every job of bj in one launch (p.N = bj.start[bj.J]); false if not applicable.
bool launch_gemv1_batch(int fmt, int xt, const GemmParams& p, const BatchJobs& bj, hipStream_t s, hipError_t& err);
// T = p.R = 2..8, K within the K-split kernel's limit: every job of bj in one launch; false if not
// applicable.
bool launch_gemv_batch(int fmt, int xt, const GemmParams& p, const BatchJobs& bj, hipStream_t s, hipError_t& err);
// Grouped matmul with short segments streamed per expert row (epi 0: Y = X W^T; epi 1: gate|up
// matrices of N = 2I rows, Y[r][j] = SiLU(g) * u with pitch I).  fast: f16 X through v_dot2, or f32
// X scaled to f16 per row in the kernel; otherwise f32 arithmetic.  grouped_rows_fits tells whether
// the shape is taken.
bool grouped_rows_fits(int fmt, int K, int N, int epi);
hipError_t launch_grouped_rows(int fmt, int xt, bool fast, int epi, const GemmParams& p, hipStream_t s);
hipError_t launch_dequant_dump(int fmt, const void* codes, const void* scales, const uint16_t* offs, int group,
                               int N, int K, int n0, int k0, int rows, int cols, int staged, void* out,
                               hipStream_t s);
hipError_t launch_x_half(const float* X, int x_rows, const int32_t* row_src, int R, int K, int guard, uint16_t* Xh,
                         float* rs, hipStream_t s);
hipError_t launch_swiglu(const float* GU, int R, int I, void* A, int at, float* rs, hipStream_t s);
hipError_t launch_moe_plan(const float* logits, int T, int E, int k, int32_t* seg_off, int32_t* row_src,
                           int32_t* slot_row, float* slot_w, int32_t* slot_expert, int32_t* status, int err_code,
                           hipStream_t s);
hipError_t launch_repack_gguf(int q8, const void* src, size_t nblocks, void* codes, void* scales, hipStream_t s);
hipError_t launch_repack_q8f(const void* blob, int N, int K, bool has_col, float* scales, float* col, hipStream_t s);
hipError_t launch_col_scale(const void* X, int xt, int T, int K, const float* col, void* Xs, int st, hipStream_t s);
hipError_t launch_repack_gguf_q8a(int type, const void* src, size_t nblocks, void* codes, float* scales,
                                  float* offs, hipStream_t s);
hipError_t launch_repack_gguf_q8a16(int type, const void* src, size_t nblk16, void* codes, float* scales,
                                    float* offs, hipStream_t s);
// Device address of this GPU's copy of the fixed scratch array (qg_moe_ffn_noalloc), looked up once
// per device with that device current.
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_moe_combine(const float* O, int R, const int32_t* slot_row, const float* slot_w, float* Y, int H,
                              int T, int k, int accumulate, hipStream_t s);

}  // namespace qg
