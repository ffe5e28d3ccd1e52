/*
 * qgemm.h -- C ABI of the block-quantized weight matrix multiply for MI355X (gfx950).
 *
 *     Y[T x N] = X[T x K] . dequant(W)[N x K]^T
 *
 * W is block-quantized along K and is dequantized while it is staged into on-chip tiles; it is
 * never written out to memory in dequantized form.  All pointers passed to the entry points below
 * are DEVICE pointers (memory the caller allocated on the GPU), except where an argument says
 * "host".  The caller owns every buffer; the library allocates nothing, keeps no state between
 * calls besides cached kernel attributes, never synchronizes, and enqueues its kernels on the
 * caller's stream.  Every entry point validates its arguments on the host before any HIP call and
 * returns a status code; nothing else is reported through the return value, and no C++ exception
 * crosses this boundary.
 *
 * Formats (page "oxinfer 0.0.5 src/metal.rs", SHADER_SRC, the dequantizers Q4W, Q4A and Q8W, and
 * Backend::upload for the offsets):
 *   Q4   codes  uint8 [N][K/2]: block b (32 consecutive k) of row n is the 16 bytes at
 *               n*K/2 + 16*b; byte j holds element 32b+j in its low nibble and element 32b+16+j
 *               in its high nibble.
 *        scales f16 bits [N][K/32]: one per block.
 *        value  w = (nibble - 8) * scale, computed in f32.
 *   Q4A  Q4 plus offsets bf16 bits [N][K/group]: w = (nibble - 8) * scale + offset, in f32, the
 *        offset of group floor(k/group) added to every element of the group (group a multiple
 *        of 32 that divides K).
 *   Q8   codes  int8 [N][K] (row-major), scales f32 [N][K/32]: w = float(q) * scale, in f32.
 * Activations X are row-major [T][K] in f32, f16 or bf16; results Y are row-major [T][N] f32.
 *
 * Modes (same page, module notes and MMA_SHADER_SRC):
 *   QG_EXACT  f32 operands, f32 accumulation (f32 MFMA or f32 FMA); 16-bit X is widened exactly.
 *   QG_FAST   the dequantized f32 weight is rounded to nearest-even into the 16-bit type of X
 *             (f16 or bf16) as it is staged; f16/bf16 MFMA with f32 accumulation.
 *
 * Shape and alignment rules shared by the matmul entry points (violations return the code named):
 *   N >= 1, T >= 0, K >= 32, K % 32 == 0                                 else QG_ESHAPE
 *   codes and X 16-byte aligned; Y 4-byte aligned (f32 elements); scales / offsets aligned to their
 *   element size; index arrays and row scales 4-byte aligned; expert tables 8-byte aligned
 *                                                                        else QG_EALIGN
 *   null pointers (with T > 0), or an enum value out of range            QG_EINVAL
 *   T == 0 returns QG_OK without launching anything.
 * Rows of Y at or beyond T, and columns at or beyond N, are never written.
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QG_ABI_VERSION 1

typedef enum {
    QG_OK = 0,
    QG_EINVAL = 1,       /* null pointer, unknown enum value, or inconsistent sizes */
    QG_EALIGN = 2,       /* a pointer is not aligned as required */
    QG_ESHAPE = 3,       /* N, K, T, group, E or k outside what the kernels support */
    QG_EUNSUPPORTED = 4, /* a mode / activation type combination the library does not provide */
    QG_ELAUNCH = 5,      /* the HIP launch reported an error (hipGetLastError) */
    QG_EPLAN = 6,        /* a routing plan input is invalid (expert id, non-finite logit) */
    QG_EWORKSPACE = 7,   /* the workspace is smaller than the call needs */
    QG_ESCRATCH = 8      /* the call needs more than the library's fixed scratch memory */
} qg_status;

typedef enum { QG_X_F32 = 0, QG_X_F16 = 1, QG_X_BF16 = 2 } qg_xtype;
/* QG_FAST_WEXACT (dense matmuls only): the fast mode with the weights kept exact -- see below. */
typedef enum { QG_EXACT = 0, QG_FAST = 1, QG_FAST_WEXACT = 2 } qg_mode;
/* QG_FMT_Q8A: the target layout of the affine GGUF types (see qg_repack_gguf_q8a); dense entry
 * points, the GEMV, the batched call and the dump only.  QG_FMT_Q8A16: Q8A with a scale and an
 * offset per 16-element block, the target layout of QG_GGUF_Q6_K / Q3_K / Q2_K (see
 * qg_repack_gguf_q8a16); dense entry points and the dump only. */
typedef enum { QG_FMT_Q4 = 0, QG_FMT_Q4A = 1, QG_FMT_Q8 = 2, QG_FMT_Q8A = 3, QG_FMT_Q8A16 = 4 } qg_format;
/* GGUF block types with the scale inside each block (the values are GGML's type ids). */
typedef enum {
    QG_GGUF_Q4_0 = 2,
    QG_GGUF_Q4_1 = 3,
    QG_GGUF_Q5_0 = 6,
    QG_GGUF_Q5_1 = 7,
    QG_GGUF_Q8_0 = 8,
    QG_GGUF_Q2_K = 10,
    QG_GGUF_Q3_K = 11,
    QG_GGUF_Q4_K = 12,
    QG_GGUF_Q5_K = 13,
    QG_GGUF_Q6_K = 14
} qg_gguf_type;

/* Text for a status code (static storage; never NULL). */
const char* qg_strerror(qg_status s);
/* QG_ABI_VERSION of the library that was loaded. */
int qg_abi_version(void);

/* ---------------------------------------------------------------------------------------------
 * Dense matmuls.  Y[t][n] = sum_k X[t][k] * w(n, k) for t < T, n < N; Y is overwritten.
 * T <= 8 runs the wavefront-reduction GEMV (exact f32 arithmetic whatever the mode); larger T
 * runs the MFMA tile kernel of the mode.  QG_FAST needs X in f16 or bf16 (the MFMA operand
 * type); an f32 X in QG_FAST with T > 8 returns QG_EUNSUPPORTED (convert it with qg_x_half and
 * use qgemm_moe_grouped with one expert, or use QG_EXACT).  QG_FAST stages each decoded weight
 * rounded to the X type.  QG_FAST_WEXACT (Q4 and Q8, f16 X; else QG_EUNSUPPORTED) keeps the
 * weights exact instead: the codes (Q4 nibble - 8, Q8 q) enter the f16 MFMA as exact f16 values,
 * each 32-k block's products are summed into an f32 block partial, and the block scale multiplies
 * that partial into the f32 result (page "cortiq-engine 0.8.41 src/gpu_metal/clover.rs", Pipes,
 * the q8 pipelines: W exact in half, the scale on the f32 result -- a per-row scale there, constant
 * over k; here the scale varies per 32-k block, so it is applied per block).  Only the rounding of
 * X to f16 and the f32 sums remain.
 * Sources: oxinfer src/metal.rs, Backend::matmul (f32 GEMM) and matmul_mma (matrix-unit GEMM).
 */
qg_status qgemm_q4(const uint8_t* codes, const uint16_t* scales_f16, const void* X, qg_xtype xt,
                   float* Y, int N, int K, int T, qg_mode mode, hipStream_t stream);
qg_status qgemm_q4a(const uint8_t* codes, const uint16_t* scales_f16, const uint16_t* offsets_bf16,
                    int group, const void* X, qg_xtype xt, float* Y, int N, int K, int T,
                    qg_mode mode, hipStream_t stream);
qg_status qgemm_q8(const int8_t* codes, const float* scales_f32, const void* X, qg_xtype xt,
                   float* Y, int N, int K, int T, qg_mode mode, hipStream_t stream);
/* Q8A: int8 codes q [N][K] (16-byte aligned), f32 scales d and f32 offsets m [N][K/32] (4-byte
 * aligned; offsets NULL gives QG_EINVAL); w(n, k) = fl(fl(q d) + m), the product rounded to f32,
 * then the add (page "oxinfer 0.0.5 src/metal.rs", GGUF_SHADER_SRC, the loaders load_q45 and Q4_KW,
 * which evaluate the affine GGUF types in that order).  Exact mode stages that value; QG_FAST
 * stages it rounded to the X type; QG_FAST_WEXACT gives QG_EUNSUPPORTED.  Every other rule as
 * qgemm_q8. */
qg_status qgemm_q8a(const int8_t* codes, const float* scales_f32, const float* offsets_f32,
                    const void* X, qg_xtype xt, float* Y, int N, int K, int T, qg_mode mode,
                    hipStream_t stream);
/* Q8A16: as qgemm_q8a with f32 scales and offsets [N][K/16], one pair per 16-element block
 * (entry n K/16 + floor(k/16)); w(n, k) = fl(fl(q d) + m).  offsets_f32 may be NULL: no offset
 * term, w(n, k) = fl(q d) (the Q6_K and Q3_K layout, 4 bytes per 16 weights fewer to read).  This holds the GGUF K-quants whose
 * scale changes every 16 elements exactly (page "oxinfer 0.0.5 src/metal.rs", GGUF_SHADER_SRC,
 * the loaders Q6_KW, Q3_KW, Q2_KW; see qg_repack_gguf_q8a16).  T <= 8 runs the GEMV; larger T runs
 * the exact f32 MFMA kernel in QG_EXACT, and in QG_FAST the decoded-tile f16 / bf16 kernel, which
 * stages each value rounded to the X type (an f32 X in QG_FAST runs the exact kernel, whose result
 * lies well inside the fast tolerance); QG_FAST_WEXACT gives QG_EUNSUPPORTED.  Not accepted by qgemm_batch
 * (QG_EUNSUPPORTED) nor by the grouped and convolution calls. */
qg_status qgemm_q8a16(const int8_t* codes, const float* scales_f32, const float* offsets_f32,
                      const void* X, qg_xtype xt, float* Y, int N, int K, int T, qg_mode mode,
                      hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * T <= 8 GEMV: one weight row per wavefront group, coalesced 16-byte loads of the packed blocks,
 * decode in registers, f32 FMA, wavefront reduction.  T > 8 returns QG_ESHAPE.
 * Source: page "cortiq-engine 0.8.41 src/gpu_metal/clover.rs", q4rows (the narrow <= 8-row
 * kernel) and oxinfer src/metal.rs module notes on memory-bound decode.
 */
qg_status qgemv_q4(const uint8_t* codes, const uint16_t* scales_f16, const void* X, qg_xtype xt,
                   float* Y, int N, int K, int T, hipStream_t stream);
qg_status qgemv_q4a(const uint8_t* codes, const uint16_t* scales_f16, const uint16_t* offsets_bf16,
                    int group, const void* X, qg_xtype xt, float* Y, int N, int K, int T,
                    hipStream_t stream);
qg_status qgemv_q8(const int8_t* codes, const float* scales_f32, const void* X, qg_xtype xt,
                   float* Y, int N, int K, int T, hipStream_t stream);
qg_status qgemv_q8a(const int8_t* codes, const float* scales_f32, const float* offsets_f32,
                    const void* X, qg_xtype xt, float* Y, int N, int K, int T, hipStream_t stream);
/* Q8A16 (see qgemm_q8a16): each lane's 16-byte unit of codes is exactly one 16-element block. */
qg_status qgemv_q8a16(const int8_t* codes, const float* scales_f32, const float* offsets_f32,
                      const void* X, qg_xtype xt, float* Y, int N, int K, int T, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Debug dump of a staged weight tile: out[r][c] = the value the GEMM kernels stage for element
 * (n0 + r, k0 + c), produced on the device by the block load and decode functions the GEMM kernels
 * call (the f32 decode of exact mode; the nearest-even 16-bit rounding of that value in fast mode).
 * staged = QG_X_F32: f32 values (exact mode); QG_X_F16 / QG_X_BF16: 16-bit patterns (fast mode).
 * Needs k0 % 32 == 0, cols % 32 == 0, 0 <= n0, n0 + rows <= N, k0 + cols <= K, rows >= 1;
 * out is [rows][cols] of 4 or 2 bytes, 16-byte aligned.  fmt QG_FMT_Q4 / Q4A take uint16 f16
 * scales, QG_FMT_Q8 / Q8A / Q8A16 f32 scales; offsets are read for QG_FMT_Q4A (bf16 bits) and
 * QG_FMT_Q8A / Q8A16 (f32 values passed through this pointer, 4-byte aligned; NULL allowed for
 * QG_FMT_Q8A16, meaning no offset term) only.
 */
qg_status qg_dequant_dump(qg_format fmt, const void* codes, const void* scales,
                          const uint16_t* offsets_bf16, int group, int N, int K, int n0, int k0,
                          int rows, int cols, qg_xtype staged, void* out, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * MoE pieces.  Sources: oxinfer src/metal.rs, Backend::upload_moe (per-expert address tables),
 * Backend::moe (the plan: rows grouped by expert, experts ascending, tokens ascending within an
 * expert; the chain x_half -> grouped gate|up -> silu_half -> grouped down -> combine), the
 * kernels x_half, silu_half and moe_combine of MMA_SHADER_SRC; page "cortiq-engine 0.8.44
 * src/clover.rs" for the top-k rule and the renormalised weights.
 */

/* One expert's weights (device pointers).  scales point to f16 bits (Q4, Q4A) or f32 (Q8);
 * offsets are used by Q4A only (may be NULL otherwise). */
typedef struct {
    const void* codes;
    const void* scales;
    const uint16_t* offsets;
} qg_expert;

/* One weight matrix of a batched call: device pointers as in qgemm_q4 / qgemm_q4a / qgemm_q8 /
 * qgemm_q8a (offsets used by QG_FMT_Q4A and, as f32, QG_FMT_Q8A only), Y f32 [T][N]. */
typedef struct {
    const void* codes;
    const void* scales;
    const uint16_t* offsets;
    float* Y;
    int N;
} qg_job;

/* Several weight matrices that share one X (page "oxinfer 0.0.5 src/metal.rs", Backend::matmul,
 * whose jobs share X): for every job j < J, jobs[j].Y = X . dequant(W_j)^T with the same rules as
 * the single-matrix entry points (format fmt and group for all jobs, X [T][K] of type xt, mode).
 * jobs is a HOST array (read during the call, not kept); its pointers are device memory.  T = 1
 * with K <= 16384 runs every 8 jobs in one launch of the streaming GEMV (the jobs' rows walked as one
 * matrix); T = 2..8 with K <= 16384 (8192 for T > 4) every 8 jobs in one launch of the K-split GEMV
 * (one column of workgroups per job), which saves a launch per job in decode; other shapes (T > 8,
 * where each job's tile launch fills the chip on its own, or longer K) run one call per job.  Every job is
 * validated before anything is launched (the first failing job's status is returned, with the
 * codes of qgemm_q4 / qgemm_q8); 1 <= J <= 64 else QG_ESHAPE; jobs NULL gives QG_EINVAL. */
qg_status qgemm_batch(qg_format fmt, int group, const qg_job* jobs, int J, const void* X, qg_xtype xt,
                      int K, int T, qg_mode mode, hipStream_t stream);

/* GGUF blocks to the split layout, on the device (page "oxinfer 0.0.5 src/metal.rs", SHADER_SRC,
 * the GGUF dequantizers Q4_0W and Q8_0W).  src: N rows of K/32 blocks each, row after row;
 * QG_GGUF_Q4_0 block = f16 scale d (little-endian) then 16 bytes, byte j holding element j in its low
 * nibble and element j + 16 in its high nibble, value (nibble - 8) * d; QG_GGUF_Q8_0 block = f16 d
 * then 32 signed bytes q, value q * d.  Writes the same weights in this library's layout, exactly:
 * Q4_0 -> Q4 codes uint8 [N][K/2] and f16 scales [N][K/32] (bytes copied); Q8_0 -> Q8 codes int8
 * [N][K] and f32 scales [N][K/32] (each f16 scale widened, which is exact), so every qgemm_q4 /
 * qgemm_q8 / qgemv_* entry point then computes with them.  Device pointers owned by the caller;
 * src 2-byte aligned, codes 16-byte aligned, scales 2- (Q4_0) or 4-byte (Q8_0) aligned, else
 * QG_EALIGN; N >= 1, K >= 32, K % 32 == 0, else QG_ESHAPE; an unknown type or a null pointer gives
 * QG_EINVAL.  Asynchronous on `stream`; nothing is allocated. */
qg_status qg_repack_gguf(qg_gguf_type type, const void* src, int N, int K, void* codes, void* scales,
                         hipStream_t stream);

/* Affine GGUF blocks to the Q8A layout, on the device (page "oxinfer 0.0.5 src/metal.rs",
 * GGUF_SHADER_SRC, the loaders load_q45 for Q4_1 / Q5_0 / Q5_1, and Q4_KW / Q5_KW with their 6-bit
 * scale and min unpacking).  src: N rows of K/32 blocks (K/256 super-blocks for QG_GGUF_Q4_K), row after row,
 * little-endian, f16 fields as h:
 *   QG_GGUF_Q4_1 (20 bytes): h d, h m, 16 nibble bytes (byte j: element j in its low nibble,
 *                element j + 16 in its high nibble); value nibble * d + m.
 *   QG_GGUF_Q5_0 (22 bytes): h d, a 32-bit qh, 16 nibble bytes; code = nibble + 16 * bit e of qh;
 *                value (code - 16) * d.
 *   QG_GGUF_Q5_1 (24 bytes): h d, h m, qh, 16 nibble bytes; value code * d + m.
 *   QG_GGUF_Q4_K (144 bytes per 256 elements): h d, h dmin, 12 bytes of 6-bit scales sc and mins
 *                mn of the eight 32-element sub-blocks, 128 code bytes; value nibble * (d sc) -
 *                dmin mn.
 *   QG_GGUF_Q5_K (176 bytes per 256 elements, loader Q5_KW): h d, h dmin, the 12 scale bytes, 32
 *                bytes qh, 128 code bytes; code = nibble | (bit j of qh[e]) << 4 for element e of
 *                sub-block j; value code * (d sc) - dmin mn.
 * Each value is a product rounded to f32 and then an add, so the Q8A layout holds it exactly: codes
 * int8 [N][K] (the code; Q5_0 code - 16), scales f32 [N][K/32] (d; Q4_K d sc rounded once) and
 * offsets f32 [N][K/32] (m; Q5_0 +0; Q4_K / Q5_K -(dmin mn) rounded once), and qgemm_q8a / qgemv_q8a then
 * compute with the GGUF values.  Device pointers owned by the caller; src 2-byte aligned, codes
 * 16-byte aligned, scales and offsets 4-byte aligned, else QG_EALIGN; N >= 1, K >= 32, K % 32 == 0
 * (K % 256 == 0 for Q4_K and Q5_K), else QG_ESHAPE; a type not listed here or a null pointer gives
 * QG_EINVAL.  Asynchronous on `stream`; nothing is allocated. */
qg_status qg_repack_gguf_q8a(qg_gguf_type type, const void* src, int N, int K, int8_t* codes,
                             float* scales_f32, float* offsets_f32, hipStream_t stream);

/* GGUF K-quants with a scale per 16 elements to the Q8A16 layout, on the device (page "oxinfer
 * 0.0.5 src/metal.rs", GGUF_SHADER_SRC, the loaders Q6_KW, Q3_KW, Q2_KW).  src: N rows of K/256
 * super-blocks, row after row, little-endian, f16 fields as h.  Sub-block j (elements 32 j ..
 * 32 j + 31 of a super-block) has half n = j / 4 and position jj = j % 4; its element e belongs to
 * the 16-element block s = 8 n + 2 jj + e / 16.
 *   QG_GGUF_Q6_K (210 bytes): 128 bytes ql, 64 bytes qh, 16 int8 scales sc, h d.  q = (nibble of
 *                ql[64 n + 32 (jj % 2) + e], the high one for jj >= 2) | (bits 2 jj, 2 jj + 1 of
 *                qh[32 n + e]) << 4; value (q - 32) * (d sc[s]).
 *   QG_GGUF_Q3_K (110 bytes): 32 bytes hmask, 64 bytes qs, 12 scale bytes, h d.  code = bits 2 jj,
 *                2 jj + 1 of qs[32 n + e], minus 4 when bit 4 n + jj of hmask[e] is clear; the
 *                6-bit scale of s takes its low four bits from scale byte s (s < 8, low nibble) or
 *                s - 8 (high nibble) and its top two from byte 8 + s % 4 at bit 2 (s / 4); value
 *                code * (d (scale - 32)).
 *   QG_GGUF_Q2_K (84 bytes): 16 scale bytes b, 64 bytes qs, h d, h dmin.  code = bits 2 jj,
 *                2 jj + 1 of qs[32 n + e]; value code * (d (b[s] & 15)) - dmin (b[s] >> 4).
 * Every product is exact in f32, so the layout holds the values exactly: codes int8 [N][K] (Q6_K
 * q - 32), scales f32 [N][K/16] and offsets f32 [N][K/16] (-0 for Q6_K and Q3_K, which keeps a
 * zero's sign; Q2_K -(dmin (b >> 4))); qgemm_q8a16 / qgemv_q8a16 then compute with the GGUF values.
 * For Q6_K and Q3_K offsets_f32 may be NULL (nothing written): the offset-free layout, which the
 * matmuls take with NULL offsets; Q2_K needs it (else QG_EINVAL).
 * Device pointers owned by the caller; src 2-byte aligned, codes 16-byte aligned, scales and
 * offsets 4-byte aligned, else QG_EALIGN; N >= 1, K >= 256, K % 256 == 0, else QG_ESHAPE; a type
 * not listed here or a null pointer gives QG_EINVAL.  Asynchronous on `stream`; nothing is
 * allocated. */
qg_status qg_repack_gguf_q8a16(qg_gguf_type type, const void* src, int N, int K, int8_t* codes,
                               float* scales_f32, float* offsets_f32, hipStream_t stream);

/* q8_2f and q8_row tensors (page "cortiq-engine 0.8.3 src/gpu_metal/qi21.rs", the block loader's
 * codec match; page "cortiq-engine 0.8.41 src/gpu_metal/clover.rs", q8mm): blob is N*K int8 codes
 * (row-major [N][K]), then N f16 row scales rs, then, for q8_2f (has_col != 0), K f16 column-field
 * values col; q8_row has no column field (col = 1).  The weight is w[n][k] = q[n][k] col[k] rs[n].
 * The codes are used in place: blob itself is the codes argument of the Q8 calls (qgemm_q8,
 * qgemv_q8, qgemm_batch).  This call writes scales f32 [N][K/32], every block of row n holding
 * f32(rs[n]) (exact), and for q8_2f col f32 [K] (exact); the column field is then applied to X by
 * qg_col_scale.  The matmul of the pages is thus qg_col_scale (q8_2f only) followed by a Q8 call:
 * QG_EXACT with f32 Xs (tau_exact), or, as the pages' half path (W exact in f16, the row scale on
 * the f32 result), QG_FAST_WEXACT with f16 Xs.  K % 32 == 0, else QG_ESHAPE; blob 16-byte aligned
 * (its codes feed the Q8 kernels), scales 4, col 16, else QG_EALIGN.  Asynchronous; nothing is
 * allocated. */
qg_status qg_repack_q8f(const void* blob, int N, int K, int has_col, float* scales, float* col,
                        hipStream_t stream);

/* The column field on X: Xs[t][k] = x[t][k] col[k], the f32 product, rounded to nearest-even when
 * st is f16 or bf16 (X of any qg_xtype, col f32 [K], Xs [T][K] of type st).  K % 8 == 0, else
 * QG_ESHAPE; X, col and Xs 16-byte aligned, else QG_EALIGN.  Asynchronous; nothing is allocated. */
qg_status qg_col_scale(const void* X, qg_xtype xt, int T, int K, const float* col, void* Xs, qg_xtype st,
                       hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Convolution as an implicit GEMM over the same quantized weights (page "oxinfer 0.0.5
 * src/metal.rs": SHADER_SRC conv_body / CONV / norm4, group_stats and row_stats, and
 * Backend::conv2d).
 *
 * qg_conv2d: X is one image [H][W][cin] f32 (channels innermost, 16-byte aligned); the weights are
 * a Q4 (uint16 f16 scales) or Q8 (f32 scales) matrix [n_out][K] in this library's layout with
 * K = ksize * ksize * cin in the order (ky, kx, ci).  pad = ksize / 2; oh = (H + 2 pad - ksize) /
 * stride + 1, likewise ow; Y f32 [oh * ow][n_out] (output pixel oy * ow + ox, then channel):
 *     Y[p][o] = sum_{ky, kx, ci} w(o, (ky * ksize + kx) * cin + ci) * x'(oy*stride + ky - pad,
 *                                                                       ox*stride + kx - pad, ci),
 * where x' is 0 outside the image and otherwise the input value, normalised when norm != 0:
 * y = (x - mean) * rstd * gamma[ci] + beta[ci] with (mean, rstd) = stats[ci / (cin / groups)]
 * (norm 1, group norm) or stats[iy * W + ix] (norm 2, per-pixel layer norm), then SiLU
 * y / (1 + exp(-y)) when silu = 1 (silu needs norm != 0, as on the page).  stats f32 pairs
 * (mean, rstd) [groups or H*W][2] (qg_conv_stats), gamma_beta f32 [2 * cin] (gamma then beta);
 * both read only when norm != 0.  Exact mode only (f32 MFMA, the exact GEMM kernel with the tap
 * gather in its X staging; QG_FAST / QG_FAST_WEXACT give QG_EUNSUPPORTED), Q4 / Q8 only (affine
 * formats give QG_EUNSUPPORTED, as the page has no affine convolution kernel).  Tolerance as the
 * dense matmul in exact mode.  Checks, before any HIP call: cin % 32 == 0, cin >= 32, ksize 1..64,
 * stride >= 1, H * W <= 2^26, H * W * cin < 2^31, K <= 2^20, oh * ow <= 2^21 (else QG_ESHAPE);
 * norm 1 needs groups >= 1 dividing cin (QG_ESHAPE); a null pointer, an unknown norm or silu
 * without norm give QG_EINVAL; codes and X 16-byte, scales 2 / 4-byte, Y, stats and gamma_beta
 * 4-byte aligned (QG_EALIGN).  Asynchronous on `stream`; nothing is allocated.
 *
 * qg_conv_stats: the page's two-pass statistics of X [npix][cin] in f32: mean = sum x / n, then
 * var = sum (x - mean)^2 / n and rstd = 1 / sqrt(var + eps), written as (mean, rstd) to
 * stats[j][2]: groups > 0 -> one pair per group j of cin / groups channels over all npix pixels
 * (groups must divide cin); groups == 0 -> one pair per pixel over its cin channels.  Each sum is an
 * f32 sum in a fixed order (error at most (n / 1024 + 24) 2^-24 of sum |x| for the group
 * statistics, (n / 64 + 8) 2^-24 per pixel).  npix >= 1, cin >= 1, npix * cin < 2^31 (QG_ESHAPE);
 * eps finite and >= 0, X and stats non-null (QG_EINVAL); 4-byte aligned (QG_EALIGN). */
qg_status qg_conv_stats(const float* X, int npix, int cin, int groups, float eps, float* stats,
                        hipStream_t stream);
qg_status qg_conv2d(qg_format fmt, const void* codes, const void* scales, const float* X, int H, int W,
                    int cin, int ksize, int stride, int n_out, int norm, int groups,
                    const float* stats, const float* gamma_beta, int silu, float* Y, qg_mode mode,
                    hipStream_t stream);

/* Routing plan, on the HOST (all pointers host memory).  logits f32 [T][E].  For each token:
 * the k largest logits, equal logits in ascending expert index; weight_j = exp(l_j - l_max) /
 * sum over the k kept of exp(l_i - l_max).  Outputs: seg_off [E+1] (expert e's gathered rows are
 * seg_off[e] .. seg_off[e+1]-1), row_src [T*k] (token of each gathered row; tokens ascending
 * within an expert), slot_row [T*k] (gathered row of token t's j-th choice at t*k + j, j in
 * descending-logit order), slot_w [T*k] (its weight, f32), slot_expert [T*k] (its expert id; may
 * be NULL).  Needs 1 <= k <= E <= 4096, T >= 1; QG_EPLAN if a logit is NaN. */
qg_status qg_moe_plan_host(const float* logits, int T, int E, int k, int32_t* seg_off,
                           int32_t* row_src, int32_t* slot_row, float* slot_w, int32_t* slot_expert);

/* Routing plan on the DEVICE (pages: "cortiq-engine 0.8.44 src/gpu_metal/clover.rs",
 * coreset_from_logits and its route step's renormalised weights; "oxinfer 0.0.5 src/metal.rs",
 * Backend::moe, which builds the same grouping on the host).  The outputs of qg_moe_plan_host, for
 * logits already in device memory, computed by one workgroup on `stream` without a host round trip:
 * logits f32 [T][E]; seg_off [E+1], row_src [T*k], slot_row [T*k], slot_w [T*k] and slot_expert
 * [T*k] (may be NULL) as described there; all pointers device memory owned by the caller, 4-byte
 * aligned.  The index outputs equal the host plan's; the weights are the same f64 expression
 * rounded to f32 (the device exp may differ from the host's in the last f64 bit, so a weight may
 * differ by one f32 unit in the last place).  status (device int32, may be NULL) receives 0, or
 * QG_EPLAN if some logit is NaN (NaN logits rank below all others; the plan is then still well
 * formed but meaningless).  Needs T >= 1, 1 <= E <= 1024, 1 <= k <= min(E, 32), T*k <= 16384,
 * else QG_ESHAPE.  Asynchronous; nothing is allocated. */
qg_status qg_moe_plan(const float* logits, int T, int E, int k, int32_t* seg_off, int32_t* row_src,
                      int32_t* slot_row, float* slot_w, int32_t* slot_expert, int32_t* status,
                      hipStream_t stream);

/* Gathered per-row power-of-two scaling of f32 rows to f16 (page section x_half / row_scale):
 * for r < R, source row s = row_src ? row_src[r] : r (rows with s outside [0, x_rows) read as
 * zeros); amax over the row; e from frexp(amax) -> scale 2^(14 - e) clamped to 2^[-100, 100]
 * (scale 1 for a zero or non-finite amax); Xh[r][:] = f16(X[s][:] * scale) (nearest-even),
 * rs[r] = 1 / scale.  X f32 [x_rows][K], Xh f16 bits [R][K], rs f32 [R].  K % 8 == 0. */
qg_status qg_x_half(const float* X, int x_rows, const int32_t* row_src, int R, int K, uint16_t* Xh,
                    float* rs, hipStream_t stream);

/* Power-of-two range guard of a half site (page "cortiq-engine 0.8.3 src/gpu_metal/qi21.rs",
 * Guards and p2: the site stores x 2^-s, the matmul reading it multiplies by 2^s): as qg_x_half
 * with the fixed scale 2^-shift for every row, Xh[r][:] = f16(X[s][:] * 2^-shift) (nearest-even;
 * magnitudes past the f16 range become infinities), rs[r] = 2^shift when rs is not NULL.  Passing
 * rs to qgemm_moe_grouped with Xh as its f16 X undoes the guard in the matmul's epilogue.
 * 0 <= shift <= 14 (the pages' range), else QG_EINVAL; shapes and alignment as qg_x_half.
 * Asynchronous; nothing is allocated. */
qg_status qg_x_half_guard(const float* X, int x_rows, const int32_t* row_src, int R, int K, int shift,
                          uint16_t* Xh, float* rs, hipStream_t stream);

/* Ragged grouped matmul over experts: for every expert e < E and every gathered row r in
 * [seg_off[e], seg_off[e+1]), Y[r][n] = (rs ? rs[r] : 1) * sum_k x_r[k] * w_e(n, k), n < N, where
 * x_r = X[row_src[r]] if row_src is given (row ids outside [0, x_rows) read as zeros) else X[r].
 * experts is a DEVICE array of E qg_expert (all of format fmt, each [N][K]); seg_off is a DEVICE
 * int32 [E+1], non-decreasing, seg_off[0] >= 0, seg_off[E] <= R (rows outside every segment are
 * not written).  Kernels: short segments (R <= 8 E) stream each expert's weight rows once through
 * the expert-row kernel when K <= 2048 (Q4, Q4A) or 1024 (Q8), else through the K-split GEMV
 * (exact mode) or the MFMA tile kernel (fast mode); R > 8 E takes the MFMA tile kernel of the mode.
 * QG_EXACT: X f32 / f16 / bf16, f32 arithmetic throughout.  QG_FAST: X f16 or bf16 -- the tile
 * kernel rounds the decoded weights to that type for f16 / bf16 MFMA; the expert-row kernel keeps
 * them exact (f16 X: the codes as exact f16 pairs through v_dot2 into an f32 partial per block,
 * scaled by the block scale; bf16 X: f32 arithmetic).  QG_FAST with f32 X (any R, K within the
 * expert-row kernel's limit, else QG_EUNSUPPORTED): each gathered row is scaled to f16 inside that
 * kernel exactly as qg_x_half does and the inverse scale multiplies the outputs (times rs when
 * given); for R <= 8 E, where the f16 call takes the same kernel, the result equals qg_x_half
 * followed by the f16 call bit for bit.  Y f32 [R][N].
 * QG_ESHAPE also when a tile-kernel launch (QG_FAST, or QG_EXACT with R > 8 E) would need more than
 * 65535 row tiles ((R + 31) / 32 + min(E, R)).  fmt QG_FMT_Q8A gives QG_EUNSUPPORTED here and in
 * qg_moe_ffn. */
qg_status qgemm_moe_grouped(qg_format fmt, const qg_expert* experts, int group,
                            const int32_t* seg_off, const int32_t* row_src, int x_rows,
                            const void* X, qg_xtype xt, const float* rs, float* Y, int N, int K,
                            int R, int E, qg_mode mode, hipStream_t stream);

/* SwiGLU of fused [gate | up] rows (page section silu_half): GU f32 [R][2I] (gate in columns
 * 0..I-1, up in I..2I-1); a = gate / (1 + exp(-gate)) * up.  at = QG_X_F32: A f32 [R][I], rs
 * unused (may be NULL).  at = QG_X_F16: A f16 bits [R][I] scaled per row by a power of two as
 * qg_x_half does, rs f32 [R] the inverse scales.  I % 8 == 0. */
qg_status qg_swiglu(const float* GU, int R, int I, void* A, qg_xtype at, float* rs,
                    hipStream_t stream);

/* Weighted combine (page section moe_combine): for t < T, c < H:
 * Y[t][c] (+)= sum_{j<k} slot_w[t*k+j] * O[slot_row[t*k+j]][c], summed in f32 in j order;
 * accumulate = 0 overwrites Y, 1 adds to it (the page's y += out).  O f32 [R][H], slot_row int32
 * and slot_w f32 [T*k] (device); slot rows outside [0, R) contribute nothing.  H % 4 == 0. */
qg_status qg_moe_combine(const float* O, int R, const int32_t* slot_row, const float* slot_w,
                         float* Y, int H, int T, int k, int accumulate, hipStream_t stream);

/* Workspace bytes qg_moe_ffn needs for R = T*k routed rows. */
size_t qg_moe_ffn_workspace(int H, int I, int T, int k, qg_mode mode);

/* The whole expert block on the stream (page section Backend::moe): [fast: qg_x_half gather] ->
 * grouped gate|up ([2I][H] per expert) -> qg_swiglu -> grouped down ([H][I] per expert) ->
 * qg_moe_combine into Y f32 [T][H] (accumulate as above).  With short segments (T k <= 8 E) and
 * H, I within the expert-row kernel's K limit (qgemm_moe_grouped) this runs as three launches: the
 * gate|up matmul with SwiGLU in its epilogue (A f32; fast mode scales X rows to f16 inside it),
 * the down matmul (fast mode scales the rows of A to f16 inside it, as qg_swiglu's f16 output
 * would be), and the combine -- the same results as the separate calls (qgemm_moe_grouped from f32
 * rows, qg_swiglu to f32, qgemm_moe_grouped, qg_moe_combine) bit for bit.  gate_up / down are DEVICE arrays of E
 * experts of format fmt; seg_off, row_src, slot_row, slot_w are the device copies of a plan
 * (qg_moe_plan_host) for these T tokens and k slots; X f32 [T][H].  The workspace (device,
 * 256-byte aligned) holds the intermediates; QG_EWORKSPACE if ws_bytes is too small. */
qg_status qg_moe_ffn(qg_format fmt, const qg_expert* gate_up, const qg_expert* down, int group,
                     int E, int H, int I, const float* X, int T, int k, const int32_t* seg_off,
                     const int32_t* row_src, const int32_t* slot_row, const float* slot_w,
                     float* Y, int accumulate, qg_mode mode, void* workspace, size_t ws_bytes,
                     hipStream_t stream);

/* Bytes of the fixed device scratch that qg_moe_ffn_noalloc uses (one copy per GPU). */
#define QG_NOALLOC_SCRATCH_BYTES (16u << 20)

/* qg_moe_ffn without a workspace argument, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * semantics, checks and kernels as qg_moe_ffn; the intermediates live in a fixed scratch array of
 * QG_NOALLOC_SCRATCH_BYTES that the library holds in each GPU's memory from its first call on that
 * GPU (the stream's GPU must be the current device) until the process ends.  Calls on one GPU share
 * that array: calls that overlap in time on one GPU (two streams, two host threads) race and give
 * wrong results; calls ordered on one stream are safe.  Nothing in the array has to start at zero
 * (every intermediate the chain reads it has written first in the same call).  A call whose
 * qg_moe_ffn_workspace(H, I, T, k, mode) exceeds QG_NOALLOC_SCRATCH_BYTES returns QG_ESCRATCH before
 * any HIP call (exact mode at H 2048, I 1536 needs 26 624 bytes per routed row: up to 630 rows, 78
 * tokens at top 8); a failure to find the array's device address returns QG_ELAUNCH.  Allocates
 * nothing: no hipMalloc / hipFree. */
qg_status qg_moe_ffn_noalloc(qg_format fmt, const qg_expert* gate_up, const qg_expert* down,
                             int group, int E, int H, int I, const float* X, int T, int k,
                             const int32_t* seg_off, const int32_t* row_src,
                             const int32_t* slot_row, const float* slot_w, float* Y,
                             int accumulate, qg_mode mode, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
