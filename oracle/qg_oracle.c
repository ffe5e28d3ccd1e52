/*
 * qg_oracle.c -- plain, slow, obviously correct CPU oracle for the block-quantized
 * weight matrix multiply Y[T x N] = X[T x K] . dequant(W)[N x K]^T and its MoE chain.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU
 * baseline load this library.  It shares no code, header, table or helper with the HIP
 * library: it has its own bit decoding, its own f16 / bf16 conversions and its own
 * rounding routines, written from the definitions of the formats.
 *
 * Sources (all on the page "oxinfer 0.0.5 src/metal.rs" unless another page is named):
 *   - Q4 block layout and value, SHADER_SRC, "Dequantizers" (struct Q4W, nib_lo, nib_hi,
 *     load(Q4W)): block b of row n is 16 bytes at n*K/2 + 16 b; byte j carries element j in
 *     its low nibble and element j + 16 in its high nibble; the f16 scale of the block is
 *     entry n*K/32 + b of the scale array; value = (nibble - 8) * scale, evaluated in f32.
 *   - Affine Q4, SHADER_SRC (struct Q4A, load(Q4A)) and Backend::upload (offsets row
 *     stride K/group, group/32 blocks per offset): a bf16 offset m, entry
 *     n*(K/group) + floor(k/group), is added (in f32) to every element of the group.
 *   - Q8, SHADER_SRC (struct Q8W, load(Q8W)): int8 code at n*K + k, f32 scale of the
 *     32-element block at n*K/32 + floor(k/32); value = float(q) * scale in f32.
 *   - Q8A (the split layout the affine GGUF blocks below are repacked into): Q8 plus an f32
 *     offset m of the block at n*K/32 + floor(k/32); value = (float(q) * scale) + m in f32, two
 *     roundings as written (the GGUF sources make the product exact, so their single rounding
 *     at the add is the same).
 *   - Q8A16 (the split layout Q6_K, Q3_K and Q2_K below are repacked into): Q8A with one scale
 *     and one offset per 16-element block, entry n*K/16 + floor(k/16); the same two roundings.
 *     Without offsets (a NULL array) the value is float(q) * scale alone, as the Q6_K and Q3_K
 *     loaders compute it.
 *   - Fast-mode staging, MMA_SHADER_SRC (mma_tile): the f32 value is converted to a 16-bit
 *     float as it is written to the tile (round to nearest, ties to even).
 *   - Row scaling to f16, MMA_SHADER_SRC (row_scale, x_half): per row, amax; frexp exponent
 *     e; scale 2^(14 - e) clamped to 2^[-100, 100]; scale 1 for a zero or non-finite amax;
 *     the inverse scale is kept for the epilogue.
 *   - SiLU(gate) * up, MMA_SHADER_SRC (silu_half) and the tests' MoE reference.
 *   - Weighted combine, MMA_SHADER_SRC (moe_combine): out[t] = sum over the token's slots
 *     of weight * o[row], in slot order.
 *   - Routing: page "cortiq-engine 0.8.44 src/clover.rs", coreset_from_logits (top-k set:
 *     descending logit, lower index first on ties) and the route closure of
 *     clover_metal_pass (weight = p[e] / sum of the kept p); segment order: Backend::moe
 *     (experts ascending; rows of one expert in token order).
 *
 * Arithmetic: the dequantized weight is the f32 value the pages' decoders compute (v32);
 * every sum is taken in f64 in ascending index order.  Build with -ffp-contract=off so the
 * f32 decode is two separately rounded operations, as written.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_Q4 = 0, ORC_Q4A = 1, ORC_Q8 = 2, ORC_Q8A = 3, ORC_Q8A16 = 4 };
enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2, ORC_F64 = 3 };

/* ---------------------------------------------------------------------------------------
 * 16-bit float definitions, decoded field by field.
 * f16: 1 sign, 5 exponent (bias 15), 10 fraction bits.  bf16: 1 sign, 8 exponent (bias 127),
 * 7 fraction bits.  Subnormals have exponent field 0 and no implicit bit.
 */
double orc_f16_value(uint16_t h) {
    int sign = h >> 15, ex = (h >> 10) & 0x1F, fr = h & 0x3FF;
    double v;
    if (ex == 0)
        v = ldexp((double)fr, -24);
    else if (ex == 0x1F)
        v = fr ? NAN : INFINITY;
    else
        v = ldexp((double)(fr + 1024), ex - 25);
    return sign ? -v : v;
}

double orc_bf16_value(uint16_t b) {
    int sign = b >> 15, ex = (b >> 7) & 0xFF, fr = b & 0x7F;
    double v;
    if (ex == 0)
        v = ldexp((double)fr, -133);
    else if (ex == 0xFF)
        v = fr ? NAN : INFINITY;
    else
        v = ldexp((double)(fr + 128), ex - 134);
    return sign ? -v : v;
}

/* Round a finite magnitude a >= 0 to the grid of a binary float with `p` significand bits,
 * smallest normal exponent emin (value 2^emin) and ties to even.  Returns the rounded
 * magnitude (may be 2^(emax+1), which the caller turns into infinity). */
static double round_to_grid(double a, int p, int emin) {
    if (a == 0.0) return 0.0;
    int e2;
    frexp(a, &e2);               /* a = f * 2^e2, f in [0.5, 1): floor(log2 a) = e2 - 1 */
    int lsb = e2 - 1 - (p - 1);  /* exponent of the last significand bit */
    if (lsb < emin - (p - 1)) lsb = emin - (p - 1);
    double q = ldexp(1.0, lsb);
    double r = a / q;            /* exact: division by a power of two */
    double fl = floor(r);
    double frac = r - fl;
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    return fl * q;
}

/* Encode an already representable magnitude into the fields of a 16-bit float. */
static uint16_t encode16(double a, int fbits, int bias, int emax_field) {
    if (a == 0.0) return 0;
    int e2;
    double f = frexp(a, &e2);    /* a = f 2^e2 */
    int ex = e2 - 1 + bias;      /* biased exponent if normal */
    if (ex >= emax_field) return (uint16_t)(emax_field << fbits);  /* infinity */
    if (ex <= 0) {               /* subnormal: a = fr * 2^(1 - bias - fbits) */
        double fr = ldexp(a, bias - 1 + fbits);
        return (uint16_t)fr;
    }
    double fr = (2.0 * f - 1.0) * (double)(1 << fbits);
    return (uint16_t)((ex << fbits) | (int)fr);
}

uint16_t orc_f32_to_f16(float x) {
    if (isnan(x)) return 0x7E00;
    uint16_t s = signbit(x) ? 0x8000 : 0;
    double a = fabs((double)x);
    if (isinf(x) || a >= 65520.0) return s | 0x7C00;
    double r = round_to_grid(a, 11, -14);
    return s | encode16(r, 10, 15, 31);
}

uint16_t orc_f32_to_bf16(float x) {
    if (isnan(x)) return 0x7FC0;
    uint16_t s = signbit(x) ? 0x8000 : 0;
    double a = fabs((double)x);
    if (isinf(x)) return s | 0x7F80;
    double r = round_to_grid(a, 8, -126);
    return s | encode16(r, 7, 127, 255);
}

/* ---------------------------------------------------------------------------------------
 * Dequantization of one element (n, k).
 */
static int q4_nibble(const uint8_t* codes, int K, int n, int k) {
    int b = k / 32, j = k % 32;
    uint8_t byte = codes[(size_t)n * (K / 2) + 16 * b + (j % 16)];
    return j < 16 ? (byte & 0xF) : (byte >> 4);
}

/* Exact real value of the weight (all three formats are exact in f64). */
double orc_weight_exact(int fmt, const void* codes, const void* scales, const uint16_t* offs, int group,
                        int N, int K, int n, int k) {
    (void)N;
    size_t bi = fmt == ORC_Q8A16 ? (size_t)n * (K / 16) + k / 16 : (size_t)n * (K / 32) + k / 32;
    if (fmt == ORC_Q8 || fmt == ORC_Q8A || fmt == ORC_Q8A16) {
        int q = ((const int8_t*)codes)[(size_t)n * K + k];
        double v = (double)q * (double)((const float*)scales)[bi];
        if (fmt != ORC_Q8 && offs) v += (double)((const float*)(const void*)offs)[bi];
        return v;
    }
    int nib = q4_nibble((const uint8_t*)codes, K, n, k);
    double v = (double)(nib - 8) * orc_f16_value(((const uint16_t*)scales)[bi]);
    if (fmt == ORC_Q4A) v += orc_bf16_value(offs[(size_t)n * (K / group) + k / group]);
    return v;
}

/* The f32 value the decoders compute (v32). */
float orc_weight_f32(int fmt, const void* codes, const void* scales, const uint16_t* offs, int group,
                     int N, int K, int n, int k) {
    (void)N;
    size_t bi = fmt == ORC_Q8A16 ? (size_t)n * (K / 16) + k / 16 : (size_t)n * (K / 32) + k / 32;
    if (fmt == ORC_Q8 || fmt == ORC_Q8A || fmt == ORC_Q8A16) {
        int q = ((const int8_t*)codes)[(size_t)n * K + k];
        float d = ((const float*)scales)[bi];
        float v = (float)q * d;
        if (fmt != ORC_Q8 && offs) {
            float m = ((const float*)(const void*)offs)[bi];
            v = v + m;
        }
        return v;
    }
    int nib = q4_nibble((const uint8_t*)codes, K, n, k);
    float d = (float)orc_f16_value(((const uint16_t*)scales)[bi]);
    float v = (float)(nib - 8) * d;
    if (fmt == ORC_Q4A) {
        float m = (float)orc_bf16_value(offs[(size_t)n * (K / group) + k / group]);
        v = v + m;
    }
    return v;
}

/* The tile a GEMM stages: out[r][c] for element (n0 + r, k0 + c), as f32 (exact mode) or as
 * the f16 / bf16 bits of the nearest-even rounding of the f32 value (fast mode). */
void orc_dequant_tile(int fmt, const void* codes, const void* scales, const uint16_t* offs, int group,
                      int N, int K, int n0, int k0, int rows, int cols, int staged, void* out) {
    for (int r = 0; r < rows; r++)
        for (int c = 0; c < cols; c++) {
            float v = orc_weight_f32(fmt, codes, scales, offs, group, N, K, n0 + r, k0 + c);
            size_t o = (size_t)r * cols + c;
            if (staged == ORC_F32)
                ((float*)out)[o] = v;
            else if (staged == ORC_F16)
                ((uint16_t*)out)[o] = orc_f32_to_f16(v);
            else
                ((uint16_t*)out)[o] = orc_f32_to_bf16(v);
        }
}

/* Activation element as stored, widened exactly to f64. */
double orc_x_value(const void* X, int xtype, size_t i) {
    switch (xtype) {
    case ORC_F32: return (double)((const float*)X)[i];
    case ORC_F16: return orc_f16_value(((const uint16_t*)X)[i]);
    case ORC_BF16: return orc_bf16_value(((const uint16_t*)X)[i]);
    default: return ((const double*)X)[i];
    }
}

/* ---------------------------------------------------------------------------------------
 * GEMM: Y[t][n] = sum_k x[t][k] * v32[n][k] and S[t][n] = sum_k |x[t][k] * v32[n][k]|, in
 * f64, k ascending.  Optional index lists select a sample of rows n (ns, nn) and tokens
 * (ts, nt); outputs are [nt][nn].  Threads split the selected n.
 */
typedef struct {
    int fmt; const void* codes; const void* scales; const uint16_t* offs; int group;
    int N, K; const void* X; int xtype; const int* ns; int nn; const int* ts; int nt;
    double* Y; double* S; int i0, i1;
} gemm_job;

static void* gemm_worker(void* arg) {
    gemm_job* j = (gemm_job*)arg;
    double* w = (double*)malloc(sizeof(double) * (size_t)j->K);
    for (int i = j->i0; i < j->i1; i++) {
        int n = j->ns ? j->ns[i] : i;
        for (int k = 0; k < j->K; k++)
            w[k] = (double)orc_weight_f32(j->fmt, j->codes, j->scales, j->offs, j->group, j->N, j->K, n, k);
        for (int a = 0; a < j->nt; a++) {
            int t = j->ts ? j->ts[a] : a;
            double y = 0.0, s = 0.0;
            for (int k = 0; k < j->K; k++) {
                double p = orc_x_value(j->X, j->xtype, (size_t)t * j->K + k) * w[k];
                y += p;
                s += fabs(p);
            }
            j->Y[(size_t)a * j->nn + i] = y;
            if (j->S) j->S[(size_t)a * j->nn + i] = s;
        }
    }
    free(w);
    return NULL;
}

int orc_gemm(int fmt, const void* codes, const void* scales, const uint16_t* offs, int group, int N, int K,
             const void* X, int xtype, int T, const int* ns, int nn, const int* ts, int nt,
             double* Y, double* S, int nthreads) {
    if (!ns) nn = N;
    if (!ts) nt = T;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > nn) nthreads = nn > 0 ? nn : 1;
    gemm_job jobs[256];
    pthread_t th[256];
    if (nthreads > 256) nthreads = 256;
    for (int i = 0; i < nthreads; i++) {
        gemm_job j = {fmt, codes, scales, offs, group, N, K, X, xtype, ns, nn, ts, nt, Y, S,
                      (int)((long)nn * i / nthreads), (int)((long)nn * (i + 1) / nthreads)};
        jobs[i] = j;
    }
    for (int i = 1; i < nthreads; i++) pthread_create(&th[i], NULL, gemm_worker, &jobs[i]);
    gemm_worker(&jobs[0]);
    for (int i = 1; i < nthreads; i++) pthread_join(th[i], NULL);
    return nthreads;
}

/* ---------------------------------------------------------------------------------------
 * Per-row power-of-two scaling to f16.  Row r of the output is source row src[r] (or r).
 * xh gets the f16 bits of x * 2^e (product in f32, then nearest-even), rs the inverse 2^-e.
 */
void orc_x_half(const float* X, int K, const int* src, int R, uint16_t* xh, float* rs) {
    for (int r = 0; r < R; r++) {
        const float* row = X + (size_t)(src ? src[r] : r) * K;
        float amax = 0.0f;
        for (int k = 0; k < K; k++) {
            float a = fabsf(row[k]);
            if (a > amax) amax = a;
        }
        int e = 0;
        if (amax > 0.0f && isfinite(amax)) {
            int fe;
            frexpf(amax, &fe);
            e = 14 - fe;
            if (e < -100) e = -100;
            if (e > 100) e = 100;
        }
        float s = ldexpf(1.0f, e);
        for (int k = 0; k < K; k++) {
            float v = row[k] * s;
            xh[(size_t)r * K + k] = orc_f32_to_f16(v);
        }
        rs[r] = ldexpf(1.0f, -e);
    }
}

/* ---------------------------------------------------------------------------------------
 * q8_2f and q8_row (page "cortiq-engine 0.8.3 src/gpu_metal/qi21.rs", the block loader's codec
 * match: a q8_2f tensor of N rows and K columns is N*K int8 codes, row-major, then N f16 row
 * scales, then K f16 column-field values; a q8_row tensor stops after the row scales and its
 * column field is 1.  Page "cortiq-engine 0.8.41 src/gpu_metal/clover.rs", q8mm: the column field
 * multiplies X, the row scale the result.)  The weight is w[n][k] = q[n][k] col[k] rs[n], exact in
 * f64 (30 significant bits at most).  The 16-bit fields are read byte by byte, little-endian.
 */
static uint16_t orc_le16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

void orc_q8f_fields(const void* blob, int has_col, int N, int K, double* rs, double* col) {
    const uint8_t* b = (const uint8_t*)blob;
    for (int n = 0; n < N; n++) rs[n] = orc_f16_value(orc_le16(b + (size_t)N * K + 2 * (size_t)n));
    for (int k = 0; k < K; k++)
        col[k] = has_col ? orc_f16_value(orc_le16(b + (size_t)N * K + 2 * (size_t)N + 2 * (size_t)k)) : 1.0;
}

/* Y[t][n] = sum_k x[t][k] w[n][k] and S[t][n] = sum_k |x[t][k] w[n][k]|, f64, ascending k. */
void orc_q8f_gemm(const void* blob, int has_col, int N, int K, const void* X, int xtype, int T, double* Y,
                  double* S) {
    const int8_t* q = (const int8_t*)blob;
    double* rs = (double*)malloc(sizeof(double) * (size_t)N);
    double* col = (double*)malloc(sizeof(double) * (size_t)K);
    orc_q8f_fields(blob, has_col, N, K, rs, col);
    for (int t = 0; t < T; t++)
        for (int n = 0; n < N; n++) {
            double y = 0.0, a = 0.0;
            for (int k = 0; k < K; k++) {
                const double w = (double)q[(size_t)n * K + k] * col[k] * rs[n];
                const double p = orc_x_value(X, xtype, (size_t)t * K + k) * w;
                y += p;
                a += fabs(p);
            }
            Y[(size_t)t * N + n] = y;
            S[(size_t)t * N + n] = a;
        }
    free(rs);
    free(col);
}

/* The column field on X (page "cortiq-engine 0.8.41 src/gpu_metal/clover.rs", q8mm: applied to X
 * as it is staged): out[t][k] = x[t][k] * col[k], the product in f32 (round to nearest), then for
 * a 16-bit output type nearest-even narrowing; out is f32 or 16-bit bits by out_type. */
void orc_col_scale(const void* X, int xtype, int T, int K, const float* col, int out_type, void* out) {
    for (size_t i = 0; i < (size_t)T * K; i++) {
        const float v = (float)orc_x_value(X, xtype, i) * col[i % (size_t)K];
        if (out_type == ORC_F32) ((float*)out)[i] = v;
        else if (out_type == ORC_F16) ((uint16_t*)out)[i] = orc_f32_to_f16(v);
        else ((uint16_t*)out)[i] = orc_f32_to_bf16(v);
    }
}

/* ---------------------------------------------------------------------------------------
 * Power-of-two range guard (page "cortiq-engine 0.8.3 src/gpu_metal/qi21.rs", Guards and p2):
 * a half site stores x * 2^-s for a fixed shift s of the site, 0 <= s <= 14, and the matmul
 * that reads it multiplies its result by 2^s.  Row r of the output is source row src[r] (or r);
 * a source outside [0, x_rows) reads as zeros.  xh gets the f16 bits of x * 2^-s (product in
 * f32, then nearest-even, overflow to infinity), rs the factor 2^s.
 */
void orc_x_half_guard(const float* X, int x_rows, int K, const int* src, int R, int shift, uint16_t* xh,
                      float* rs) {
    const float s = ldexpf(1.0f, -shift);
    for (int r = 0; r < R; r++) {
        const int sr = src ? src[r] : r;
        const int ok = sr >= 0 && sr < x_rows;
        for (int k = 0; k < K; k++) {
            float v = ok ? X[(size_t)sr * K + k] * s : 0.0f;
            xh[(size_t)r * K + k] = orc_f32_to_f16(v);
        }
        rs[r] = ldexpf(1.0f, shift);
    }
}

/* a = SiLU(g) * u = g / (1 + exp(-g)) * u, f64, elementwise. */
void orc_swiglu(const double* G, const double* U, size_t n, double* A) {
    for (size_t i = 0; i < n; i++) A[i] = G[i] / (1.0 + exp(-G[i])) * U[i];
}

/* ---------------------------------------------------------------------------------------
 * Routing plan for T rows of E router logits, k experts per row.
 * Top-k: logits sorted descending, equal logits in ascending expert index; the first k.
 * Weights: exp(l_j - l_max) / sum over the kept of exp(l_i - l_max)  (= p_j / sum kept p).
 * Segments: experts ascending; seg_off[e] .. seg_off[e+1] are expert e's gathered rows,
 * holding its tokens in ascending order.  row_src[r] = token of gathered row r.
 * slot_row[t*k + j] = gathered row of token t's j-th expert (j in top-k order),
 * slot_w[t*k + j] its weight.  Returns R = T*k.
 */
static const float* sort_row;
static int cmp_desc(const void* a, const void* b) {
    int x = *(const int*)a, y = *(const int*)b;
    if (sort_row[x] > sort_row[y]) return -1;
    if (sort_row[x] < sort_row[y]) return 1;
    return x < y ? -1 : (x > y);
}

int orc_moe_plan(const float* logits, int T, int E, int k, int* seg_off, int* row_src, int* slot_row,
                 double* slot_w, int* slot_expert) {
    int* idx = (int*)malloc(sizeof(int) * (size_t)E);
    int* topk = (int*)malloc(sizeof(int) * (size_t)T * k);
    for (int t = 0; t < T; t++) {
        const float* row = logits + (size_t)t * E;
        for (int e = 0; e < E; e++) idx[e] = e;
        sort_row = row;
        qsort(idx, (size_t)E, sizeof(int), cmp_desc);
        double lmax = (double)row[idx[0]], sum = 0.0;
        for (int j = 0; j < k; j++) sum += exp((double)row[idx[j]] - lmax);
        for (int j = 0; j < k; j++) {
            topk[t * k + j] = idx[j];
            slot_w[t * k + j] = exp((double)row[idx[j]] - lmax) / sum;
            if (slot_expert) slot_expert[t * k + j] = idx[j];
        }
    }
    for (int e = 0; e <= E; e++) seg_off[e] = 0;
    for (int i = 0; i < T * k; i++) seg_off[topk[i] + 1]++;
    for (int e = 0; e < E; e++) seg_off[e + 1] += seg_off[e];
    int* fill = (int*)malloc(sizeof(int) * (size_t)E);
    for (int e = 0; e < E; e++) fill[e] = seg_off[e];
    for (int t = 0; t < T; t++)
        for (int j = 0; j < k; j++) {
            int e = topk[t * k + j];
            int r = fill[e]++;
            row_src[r] = t;
            slot_row[t * k + j] = r;
        }
    free(fill);
    free(topk);
    free(idx);
    return T * k;
}

/* y[t][c] = sum_j slot_w[t*k+j] * O[slot_row[t*k+j]][c] (f64, j ascending);
 * b[t][c] = sum_j |slot_w * O| (the tolerance denominator). */
void orc_moe_combine(const double* O, int H, const int* slot_row, const double* slot_w, int T, int k,
                     double* y, double* b) {
    for (int t = 0; t < T; t++)
        for (int c = 0; c < H; c++) {
            double acc = 0.0, s = 0.0;
            for (int j = 0; j < k; j++) {
                double p = slot_w[t * k + j] * O[(size_t)slot_row[t * k + j] * H + c];
                acc += p;
                s += fabs(p);
            }
            y[(size_t)t * H + c] = acc;
            if (b) b[(size_t)t * H + c] = s;
        }
}

/* ---------------------------------------------------------------------------------------
 * Array forms of the conversions (used by the tests to sweep whole encodings). */
void orc_f16_values(const uint16_t* h, size_t n, double* out) {
    for (size_t i = 0; i < n; i++) out[i] = orc_f16_value(h[i]);
}
void orc_bf16_values(const uint16_t* h, size_t n, double* out) {
    for (size_t i = 0; i < n; i++) out[i] = orc_bf16_value(h[i]);
}
void orc_f32_to_f16_array(const float* x, size_t n, uint16_t* out) {
    for (size_t i = 0; i < n; i++) out[i] = orc_f32_to_f16(x[i]);
}
void orc_f32_to_bf16_array(const float* x, size_t n, uint16_t* out) {
    for (size_t i = 0; i < n; i++) out[i] = orc_f32_to_bf16(x[i]);
}
/* Whole dequantized matrix, exact (f64) or as the f32 decode. */
void orc_dequant_exact(int fmt, const void* codes, const void* scales, const uint16_t* offs, int group,
                       int N, int K, double* out) {
    for (int n = 0; n < N; n++)
        for (int k = 0; k < K; k++)
            out[(size_t)n * K + k] = orc_weight_exact(fmt, codes, scales, offs, group, N, K, n, k);
}

/* ---------------------------------------------------------------------------------------
 * GGUF blocks with the scale inside the block (page "oxinfer 0.0.5 src/metal.rs",
 * GGUF_SHADER_SRC: the loaders Q4_0W, Q8_0W, Q4_1W / Q5_0W / Q5_1W (load_q45) and Q4_KW with
 * scale_min_k4).  Multi-byte fields are little-endian; h = an f16 field as f32.
 *   Q4_0 (type 2): 18 bytes per 32 elements = h d, then 16 bytes; byte j holds element j in its
 *         low nibble and element j + 16 in its high nibble; value = (nibble - 8) * d.
 *   Q8_0 (type 8): 34 bytes = h d, then 32 signed bytes q; value = float(q) * d.
 *   Q4_1 (type 3): 20 bytes = h d, h m, 16 nibble bytes as Q4_0; value = nibble * d + m.
 *   Q5_0 (type 6): 22 bytes = h d, a 32-bit word qh, 16 nibble bytes; element j's code is its
 *         nibble + 16 * bit j of qh; value = (code - 16) * d + 0.
 *   Q5_1 (type 7): 24 bytes = h d, h m, qh, 16 nibble bytes; value = code * d + m.
 *   Q4_K (type 12): 144 bytes per 256 elements = h d, h dmin, 12 scale bytes s, 128 code bytes.
 *         Sub-block j (elements 32 j .. 32 j + 31) has a 6-bit scale sc and min mn:
 *         j < 4: sc = s[j] & 63, mn = s[j + 4] & 63; j >= 4: sc = (s[j + 4] & 15) | ((s[j - 4] >> 6)
 *         << 4), mn = (s[j + 4] >> 4) | ((s[j] >> 6) << 4).  d1 = d * sc, m1 = dmin * mn (f32);
 *         element e of sub-block j is nibble (j % 2 ? high : low) of code byte 32 (j / 2) + e;
 *         value = nibble * d1 - m1.
 *   Q5_K (type 13, loader Q5_KW): 176 bytes per 256 elements = h d, h dmin, the 12 scale bytes of
 *         Q4_K, 32 bytes qh, 128 code bytes; sub-block j as Q4_K (code bytes 48 + 32 (j / 2) + e,
 *         the same scale / min unpacking) with a fifth bit: code = nibble | (bit j of qh[e]) << 4;
 *         value = code * d1 - m1.
 * The K-quants with a scale per 16 elements (loaders Q6_KW, Q3_KW, Q2_KW): 256 elements per
 * super-block; sub-block j = (k % 256) / 32 of it has half n = j / 4 and position jj = j % 4;
 * element e = k % 32 of the sub-block has 16-element index s16 = 8 n + 2 jj + e / 16.
 *   Q6_K (type 14): 210 bytes = 128 bytes ql, 64 bytes qh, 16 signed scale bytes sc, h d.
 *         Low four bits: nibble (jj >= 2 ? high : low) of ql[64 n + 32 (jj % 2) + e]; high two
 *         bits: bits 2 jj, 2 jj + 1 of qh[32 n + e]; q = low | high << 4 (0..63).
 *         dl = d * sc[s16] (f32); value = (q - 32) * dl.
 *   Q3_K (type 11): 110 bytes = 32 bytes hmask, 64 bytes qs, 12 scale bytes, h d.  q = bits
 *         2 jj, 2 jj + 1 of qs[32 n + e]; it is lowered by 4 unless bit 4 n + jj of hmask[e] is
 *         set.  The 6-bit scale of s16: low four bits = (s16 < 8 ? scales[s16] & 15 :
 *         scales[s16 - 8] >> 4), high two bits = bits 2 (s16 / 4), +1 of scales[8 + s16 % 4];
 *         dl = d * (that - 32) (f32); value = code * dl.
 *   Q2_K (type 10): 84 bytes = 16 scale bytes s, 64 bytes qs, h d, h dmin.  q = bits 2 jj,
 *         2 jj + 1 of qs[32 n + e]; dl = d * (s[s16] & 15), ml = dmin * (s[s16] >> 4) (f32);
 *         value = q * dl - ml.
 * Every value is evaluated in f32 in the order written.  A row holds K / 32 blocks (K / 256
 * super-blocks for the K-quants).
 */
#define ORC_GGUF_Q4_0 2
#define ORC_GGUF_Q4_1 3
#define ORC_GGUF_Q5_0 6
#define ORC_GGUF_Q5_1 7
#define ORC_GGUF_Q8_0 8
#define ORC_GGUF_Q4_K 12
#define ORC_GGUF_Q5_K 13
#define ORC_GGUF_Q2_K 10
#define ORC_GGUF_Q3_K 11
#define ORC_GGUF_Q6_K 14

/* Bytes of one row of K elements. */
static size_t gguf_row_bytes(int type, int K) {
    switch (type) {
    case ORC_GGUF_Q4_0: return (size_t)(K / 32) * 18;
    case ORC_GGUF_Q4_1: return (size_t)(K / 32) * 20;
    case ORC_GGUF_Q5_0: return (size_t)(K / 32) * 22;
    case ORC_GGUF_Q5_1: return (size_t)(K / 32) * 24;
    case ORC_GGUF_Q8_0: return (size_t)(K / 32) * 34;
    case ORC_GGUF_Q5_K: return (size_t)(K / 256) * 176;
    case ORC_GGUF_Q6_K: return (size_t)(K / 256) * 210;
    case ORC_GGUF_Q3_K: return (size_t)(K / 256) * 110;
    case ORC_GGUF_Q2_K: return (size_t)(K / 256) * 84;
    default: return (size_t)(K / 256) * 144;
    }
}

static float gguf_h(const uint8_t* p) { return (float)orc_f16_value((uint16_t)(p[0] | (p[1] << 8))); }

/* Q4_K: the 6-bit scale and min of sub-block j from the 12 scale bytes. */
static void gguf_k4_scale_min(int j, const uint8_t* s, int* sc, int* mn) {
    if (j < 4) {
        *sc = s[j] & 63;
        *mn = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        *mn = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/* The integer code, f32 scale and f32 offset of element (n, k): value = code * scale + offset
 * in the types' own evaluation order (see gguf_value). */
static void gguf_element(int type, const uint8_t* src, int K, int n, int k, int* code, float* d, float* m) {
    const uint8_t* row = src + (size_t)n * gguf_row_bytes(type, K);
    int j = k % 32;
    if (type == ORC_GGUF_Q6_K || type == ORC_GGUF_Q3_K || type == ORC_GGUF_Q2_K) {
        int sub = (k % 256) / 32, half = sub / 4, pos = sub % 4, s16 = 8 * half + 2 * pos + j / 16;
        if (type == ORC_GGUF_Q6_K) {
            const uint8_t* SB = row + (size_t)(k / 256) * 210;
            uint8_t lb = SB[64 * half + 32 * (pos % 2) + j];
            int low = pos >= 2 ? (lb >> 4) : (lb & 15);
            int high = (SB[128 + 32 * half + j] >> (2 * pos)) & 3;
            *code = (low | (high << 4)) - 32;
            *d = gguf_h(SB + 208) * (float)(int8_t)SB[192 + s16];
            *m = 0.0f;
        } else if (type == ORC_GGUF_Q3_K) {
            const uint8_t* SB = row + (size_t)(k / 256) * 110;
            int q = (SB[32 + 32 * half + j] >> (2 * pos)) & 3;
            if (!((SB[j] >> (4 * half + pos)) & 1)) q -= 4;
            int lo = s16 < 8 ? (SB[96 + s16] & 15) : (SB[96 + s16 - 8] >> 4);
            int hi = (SB[104 + s16 % 4] >> (2 * (s16 / 4))) & 3;
            *code = q;
            *d = gguf_h(SB + 108) * (float)((lo | (hi << 4)) - 32);
            *m = 0.0f;
        } else {
            const uint8_t* SB = row + (size_t)(k / 256) * 84;
            uint8_t sc = SB[s16];
            *code = (SB[16 + 32 * half + j] >> (2 * pos)) & 3;
            *d = gguf_h(SB + 80) * (float)(sc & 15);
            *m = gguf_h(SB + 82) * (float)(sc >> 4);
        }
        return;
    }
    if (type == ORC_GGUF_Q5_K) {
        const uint8_t* SB = row + (size_t)(k / 256) * 176;
        int sub = (k % 256) / 32, sc, mn;
        gguf_k4_scale_min(sub, SB + 4, &sc, &mn);
        float d1 = gguf_h(SB) * (float)sc;
        float m1 = gguf_h(SB + 2) * (float)mn;
        uint8_t byte = SB[48 + 32 * (sub / 2) + j];
        int nib = (sub % 2) ? (byte >> 4) : (byte & 15);
        *code = nib | (((SB[16 + j] >> sub) & 1) << 4);
        *d = d1;
        *m = m1;
        return;
    }
    if (type == ORC_GGUF_Q4_K) {
        const uint8_t* SB = row + (size_t)(k / 256) * 144;
        int sub = (k % 256) / 32, sc, mn;
        gguf_k4_scale_min(sub, SB + 4, &sc, &mn);
        float d1 = gguf_h(SB) * (float)sc;
        float m1 = gguf_h(SB + 2) * (float)mn;
        uint8_t byte = SB[16 + 32 * (sub / 2) + j];
        *code = (sub % 2) ? (byte >> 4) : (byte & 15);
        *d = d1;
        *m = m1;
        return;
    }
    int minb = type == ORC_GGUF_Q4_1 || type == ORC_GGUF_Q5_1;
    int hib = type == ORC_GGUF_Q5_0 || type == ORC_GGUF_Q5_1;
    size_t bb = gguf_row_bytes(type, 32);
    const uint8_t* B = row + (size_t)(k / 32) * bb;
    if (type == ORC_GGUF_Q8_0) {
        *code = (int8_t)B[2 + j];
        *d = gguf_h(B);
        *m = 0.0f;
        return;
    }
    *d = gguf_h(B);
    *m = minb ? gguf_h(B + 2) : 0.0f;
    const uint8_t* qs = B + 2 + (minb ? 2 : 0) + (hib ? 4 : 0);
    uint8_t byte = qs[j % 16];
    int nib = j < 16 ? (byte & 15) : (byte >> 4);
    if (hib) {
        const uint8_t* h = B + 2 + (minb ? 2 : 0);
        uint32_t qh = (uint32_t)h[0] | ((uint32_t)h[1] << 8) | ((uint32_t)h[2] << 16) | ((uint32_t)h[3] << 24);
        nib += 16 * (int)((qh >> j) & 1);
    }
    *code = nib;
}

/* The f32 value of element (n, k), as the type's loader evaluates it. */
float orc_gguf_weight_f32(int type, const uint8_t* src, int K, int n, int k) {
    int code;
    float d, m;
    gguf_element(type, src, K, n, k, &code, &d, &m);
    switch (type) {
    case ORC_GGUF_Q4_0: {
        float v = (float)(code - 8) * d;
        return v;
    }
    case ORC_GGUF_Q8_0: {
        float v = (float)code * d;
        return v;
    }
    case ORC_GGUF_Q5_0: {
        float p = (float)(code - 16) * d;
        float v = p + m;
        return v;
    }
    case ORC_GGUF_Q4_K:
    case ORC_GGUF_Q5_K:
    case ORC_GGUF_Q2_K: {
        float p = (float)code * d;
        float v = p - m;
        return v;
    }
    case ORC_GGUF_Q6_K:
    case ORC_GGUF_Q3_K: {
        float v = (float)code * d;
        return v;
    }
    default: { /* Q4_1, Q5_1 */
        float p = (float)code * d;
        float v = p + m;
        return v;
    }
    }
}

void orc_gguf_dequant(int type, const uint8_t* src, int N, int K, float* out) {
    for (int n = 0; n < N; n++)
        for (int k = 0; k < K; k++) out[(size_t)n * K + k] = orc_gguf_weight_f32(type, src, K, n, k);
}

/* The split layout of the same weights: Q4_0 -> Q4 codes [N][K/2] (the 16 code bytes of each
 * block, unchanged) and f16 scales [N][K/32] (the block's 2 scale bytes); Q8_0 -> Q8 codes
 * [N][K] and f32 scales [N][K/32] (the f16 scale widened, exactly). */
void orc_gguf_repack(int type, const uint8_t* src, int N, int K, uint8_t* codes, void* scales) {
    size_t bb = gguf_row_bytes(type, 32), nb = (size_t)K / 32;
    for (int n = 0; n < N; n++)
        for (size_t b = 0; b < nb; b++) {
            const uint8_t* B = src + ((size_t)n * nb + b) * bb;
            uint16_t dh = (uint16_t)(B[0] | (B[1] << 8));
            if (type == ORC_GGUF_Q4_0) {
                for (int j = 0; j < 16; j++) codes[(size_t)n * (K / 2) + 16 * b + j] = B[2 + j];
                ((uint16_t*)scales)[(size_t)n * nb + b] = dh;
            } else {
                for (int j = 0; j < 32; j++) codes[(size_t)n * K + 32 * b + j] = B[2 + j];
                ((float*)scales)[(size_t)n * nb + b] = (float)orc_f16_value(dh);
            }
        }
}

/* Q4_1, Q5_0, Q5_1, Q4_K, Q5_K -> the Q8A layout: int8 codes [N][K], f32 scales and f32 offsets
 * [N][K/32], with q * scale + offset equal to the type's value: Q4_1 / Q5_1 (code, d, m);
 * Q5_0 (code - 16, d, +0); Q4_K / Q5_K (code, d1, -m1) per 32-element sub-block. */
void orc_gguf_repack_q8a(int type, const uint8_t* src, int N, int K, int8_t* codes, float* scales, float* offs) {
    for (int n = 0; n < N; n++)
        for (int k = 0; k < K; k++) {
            int code;
            float d, m;
            gguf_element(type, src, K, n, k, &code, &d, &m);
            size_t bi = (size_t)n * (K / 32) + k / 32;
            if (type == ORC_GGUF_Q5_0) code -= 16;
            codes[(size_t)n * K + k] = (int8_t)code;
            scales[bi] = d;
            offs[bi] = (type == ORC_GGUF_Q4_K || type == ORC_GGUF_Q5_K) ? -m : m;
        }
}

/* ---------------------------------------------------------------------------------------
 * The MoE expert block (page "oxinfer 0.0.5 src/metal.rs", Backend::upload_moe for the fused
 * gate|up matrix [2I][H] -- gate rows 0..I-1, up rows I..2I-1 -- and the down matrix [H][I],
 * Backend::moe for the chain, and the reference loop of its test mma_moe_matches_cpu):
 * for every gathered row r of expert e (seg_off[e] <= r < seg_off[e+1]) and its token
 * t = row_src[r]:
 *     g = W_gate[e] x_t,  u = W_up[e] x_t                       (each an f64 GEMM row)
 *     a_i = g_i / (1 + exp(-g_i)) * u_i                         (SiLU(gate) * up, f64)
 *     o_r = W_down[e] a                                         (f64)
 * and y[t] = sum_j slot_w[t*k+j] * o[slot_row[t*k+j]], j ascending.  Weights are the f32 values
 * of the format (v32), as in orc_gemm.
 *
 * Error-bound components for a chain that evaluates these steps with per-step errors: for
 * output (t, c),
 *     b_dn = sum_j |w_j| sum_i |a_i wd[c][i]|                     (the down GEMM's own S)
 *     b_gu = sum_j |w_j| sum_i |wd[c][i]| (1.1 |u_i| Sg_i + |silu(g_i)| Su_i)
 * where Sg_i, Su_i are the S sums (sum_k |x_k w_k|) of gate / up row i.  A gate or up value off
 * by at most tau*S moves a_i by at most 1.1 |u_i| tau Sg_i + |silu(g_i)| tau Su_i to first order
 * (|d silu / dg| <= 1.1 for every g), and the down GEMM carries that through |wd|; a relative
 * error rho in a itself and a down GEMM error of tau*S add (rho + tau) b_dn.
 * Optional outputs: GU [R][2I], A [R][I], O [R][H].  X f32 [T][H].  Per-expert pointer arrays
 * (offsets used by Q4A only).  Returns R = seg_off[E], or -1 if a row's token is out of range.
 */
static double silu_f64(double g) { return g / (1.0 + exp(-g)); }

int orc_moe_ffn(int fmt, const void* const* gu_codes, const void* const* gu_scales, const uint16_t* const* gu_offs,
                const void* const* dn_codes, const void* const* dn_scales, const uint16_t* const* dn_offs,
                int group, int E, int H, int I, const float* X, int T, int k, const int* seg_off,
                const int* row_src, const int* slot_row, const double* slot_w, double* y, double* b_dn,
                double* b_gu, double* GU, double* A, double* O, int nthreads) {
    const int R = seg_off[E];
    for (int r = 0; r < R; r++)
        if (row_src[r] < 0 || row_src[r] >= T) return -1;
    double* o_all = (double*)calloc((size_t)R * H, sizeof(double));
    double* so_all = (double*)calloc((size_t)R * H, sizeof(double));
    double* sd_all = (double*)calloc((size_t)R * H, sizeof(double));
    for (int e = 0; e < E; e++) {
        const int r0 = seg_off[e], n = seg_off[e + 1] - r0;
        if (n <= 0) continue;
        float* xg = (float*)malloc(sizeof(float) * (size_t)n * H);
        for (int i = 0; i < n; i++)
            memcpy(xg + (size_t)i * H, X + (size_t)row_src[r0 + i] * H, sizeof(float) * (size_t)H);
        double* gu = (double*)malloc(sizeof(double) * (size_t)n * 2 * I);
        double* sgu = (double*)malloc(sizeof(double) * (size_t)n * 2 * I);
        orc_gemm(fmt, gu_codes[e], gu_scales[e], gu_offs ? gu_offs[e] : NULL, group, 2 * I, H, xg, ORC_F32, n,
                 NULL, 0, NULL, 0, gu, sgu, nthreads);
        double* a = (double*)malloc(sizeof(double) * (size_t)n * I);
        double* da = (double*)malloc(sizeof(double) * (size_t)n * I);
        for (int i = 0; i < n; i++)
            for (int c = 0; c < I; c++) {
                const double g = gu[(size_t)i * 2 * I + c], u = gu[(size_t)i * 2 * I + I + c];
                const double sg = sgu[(size_t)i * 2 * I + c], su = sgu[(size_t)i * 2 * I + I + c];
                a[(size_t)i * I + c] = silu_f64(g) * u;
                da[(size_t)i * I + c] = 1.1 * fabs(u) * sg + fabs(silu_f64(g)) * su;
            }
        /* o = W_down a, so = sum_i |a_i wd_i|; sd = sum_i |da_i wd_i| = sum_i da_i |wd_i| (da >= 0) */
        orc_gemm(fmt, dn_codes[e], dn_scales[e], dn_offs ? dn_offs[e] : NULL, group, H, I, a, ORC_F64, n, NULL, 0,
                 NULL, 0, o_all + (size_t)r0 * H, so_all + (size_t)r0 * H, nthreads);
        double* junk = (double*)malloc(sizeof(double) * (size_t)n * H);
        orc_gemm(fmt, dn_codes[e], dn_scales[e], dn_offs ? dn_offs[e] : NULL, group, H, I, da, ORC_F64, n, NULL, 0,
                 NULL, 0, junk, sd_all + (size_t)r0 * H, nthreads);
        if (GU) memcpy(GU + (size_t)r0 * 2 * I, gu, sizeof(double) * (size_t)n * 2 * I);
        if (A) memcpy(A + (size_t)r0 * I, a, sizeof(double) * (size_t)n * I);
        free(junk);
        free(da);
        free(a);
        free(sgu);
        free(gu);
        free(xg);
    }
    if (O) memcpy(O, o_all, sizeof(double) * (size_t)R * H);
    double* aw = (double*)malloc(sizeof(double) * (size_t)T * k);
    for (int i = 0; i < T * k; i++) aw[i] = fabs(slot_w[i]);
    orc_moe_combine(o_all, H, slot_row, slot_w, T, k, y, NULL);
    if (b_dn) orc_moe_combine(so_all, H, slot_row, aw, T, k, b_dn, NULL);
    if (b_gu) orc_moe_combine(sd_all, H, slot_row, aw, T, k, b_gu, NULL);
    free(aw);
    free(sd_all);
    free(so_all);
    free(o_all);
    return R;
}

/* ---------------------------------------------------------------------------------------
 * Convolution as an implicit GEMM over the same quantized weights (page "oxinfer 0.0.5
 * src/metal.rs": SHADER_SRC conv_body / CONV / norm4, group_stats and row_stats, and
 * Backend::conv2d).
 *   - X is one image [H][W][cin] (f32, channels innermost); the output has one row per output
 *     pixel p = oy * ow + ox and one column per output channel o: Y[p][o].
 *   - The weight row o has K = ksz * ksz * cin elements in the order (ky, kx, ci): element
 *     k = (ky * ksz + kx) * cin + ci, decoded exactly as for the GEMM (v32).
 *   - pad = ksz / 2; the input pixel of tap (ky, kx) is (oy * stride + ky - pad,
 *     ox * stride + kx - pad); taps outside the image contribute 0 (they are not normalised).
 *     Output size: oh = (H + 2 pad - ksz) / stride + 1, likewise ow (the page takes oh / ow
 *     from its geometry record; this is the usual definition with that padding).
 *   - Optional normalisation of each gathered input value v of channel c at input pixel q:
 *     y = (v - mean) * rstd * gamma[c] + beta[c], with (mean, rstd) = stats[c / cpg] (group
 *     norm, cpg channels per group) or stats[q] (layer norm over the cin channels of pixel q);
 *     then optionally SiLU: y / (1 + exp(-y)).
 *   - Statistics (group_stats / row_stats): two passes, mean = sum x / n, then
 *     var = sum (x - mean)^2 / n, rstd = 1 / sqrt(var + eps), over the n values of the group
 *     (all pixels, its cpg channels) or of the pixel (its cin channels).
 * Arithmetic here: f64 throughout; the statistics the convolution uses are passed in as f32
 * (the precision the device computes them in), widened exactly.
 */

/* (mean, rstd) pairs: groups > 0 -> one per group; groups == 0 -> one per pixel. */
void orc_conv_stats(const float* X, int npix, int cin, int groups, double eps, double* out) {
    if (groups > 0) {
        const int cpg = cin / groups;
        const double n = (double)npix * cpg;
        for (int g = 0; g < groups; g++) {
            double s = 0.0, v = 0.0;
            for (int q = 0; q < npix; q++)
                for (int c = g * cpg; c < (g + 1) * cpg; c++) s += (double)X[(size_t)q * cin + c];
            const double mean = s / n;
            for (int q = 0; q < npix; q++)
                for (int c = g * cpg; c < (g + 1) * cpg; c++) {
                    const double d = (double)X[(size_t)q * cin + c] - mean;
                    v += d * d;
                }
            out[2 * g] = mean;
            out[2 * g + 1] = 1.0 / sqrt(v / n + eps);
        }
    } else {
        for (int q = 0; q < npix; q++) {
            double s = 0.0, v = 0.0;
            for (int c = 0; c < cin; c++) s += (double)X[(size_t)q * cin + c];
            const double mean = s / cin;
            for (int c = 0; c < cin; c++) {
                const double d = (double)X[(size_t)q * cin + c] - mean;
                v += d * d;
            }
            out[2 * q] = mean;
            out[2 * q + 1] = 1.0 / sqrt(v / cin + eps);
        }
    }
}

/* The gathered input rows of the implicit GEMM for the output pixels ps[0..np-1]:
 * A[i][k] = the (normalised, activated) input value of tap k for pixel ps[i], and
 * M[i][k] = a magnitude that bounds the error of evaluating it in f32: |A| plus, when
 * normalising, |v - mean| |rstd| |gamma| + |beta| + |y| (every term an f32 rounding touches). */
void orc_conv_gather(const float* X, int H, int W, int cin, int ksz, int stride, int norm, int cpg,
                     const float* stats, const float* gb, int silu, const int* ps, int np, double* A, double* M) {
    const int pad = ksz / 2, ow = (W + 2 * pad - ksz) / stride + 1, K = ksz * ksz * cin;
    for (int i = 0; i < np; i++) {
        const int p = ps[i], oy = p / ow, ox = p % ow;
        for (int ky = 0; ky < ksz; ky++)
            for (int kx = 0; kx < ksz; kx++) {
                const int iy = oy * stride + ky - pad, ix = ox * stride + kx - pad;
                const int inside = iy >= 0 && iy < H && ix >= 0 && ix < W;
                for (int c = 0; c < cin; c++) {
                    const size_t k = (size_t)(ky * ksz + kx) * cin + c;
                    double a = 0.0, m = 0.0;
                    if (inside) {
                        const double v = (double)X[((size_t)iy * W + ix) * cin + c];
                        a = v;
                        if (norm) {
                            const int si = norm == 1 ? c / cpg : iy * W + ix;
                            const double mean = (double)stats[2 * si], rstd = (double)stats[2 * si + 1];
                            const double g = (double)gb[c], b = (double)gb[cin + c];
                            const double y = (v - mean) * rstd * g + b;
                            a = silu ? y / (1.0 + exp(-y)) : y;
                            m = fabs(v - mean) * fabs(rstd) * fabs(g) + fabs(b) + fabs(y);
                        }
                        m += fabs(a);
                    }
                    A[(size_t)i * K + k] = a;
                    M[(size_t)i * K + k] = m;
                }
            }
    }
}

/* Y[i][j] = sum_k A[i][k] v32[os[j]][k] and S[i][j] = sum_k M[i][k] |v32[os[j]][k]| for the
 * output pixels ps and output channels os (all of them when a list is NULL). */
int orc_conv2d(int fmt, const void* codes, const void* scales, const uint16_t* offs, int group, int n_out,
               const float* X, int H, int W, int cin, int ksz, int stride, int norm, int cpg,
               const float* stats, const float* gb, int silu, const int* ps, int np, const int* os, int nos,
               double* Y, double* S, int nthreads) {
    const int pad = ksz / 2;
    const int oh = (H + 2 * pad - ksz) / stride + 1, ow = (W + 2 * pad - ksz) / stride + 1;
    const int K = ksz * ksz * cin;
    int* all = NULL;
    if (!ps) {
        np = oh * ow;
        all = (int*)malloc(sizeof(int) * (size_t)np);
        for (int i = 0; i < np; i++) all[i] = i;
        ps = all;
    }
    double* A = (double*)malloc(sizeof(double) * (size_t)np * K);
    double* M = (double*)malloc(sizeof(double) * (size_t)np * K);
    orc_conv_gather(X, H, W, cin, ksz, stride, norm, cpg, stats, gb, silu, ps, np, A, M);
    const int nn = os ? nos : n_out;
    double* junk = (double*)malloc(sizeof(double) * (size_t)np * nn);
    int used = orc_gemm(fmt, codes, scales, offs, group, n_out, K, A, ORC_F64, np, os, nos, NULL, 0, Y, NULL,
                        nthreads);
    orc_gemm(fmt, codes, scales, offs, group, n_out, K, M, ORC_F64, np, os, nos, NULL, 0, junk, S, nthreads);
    free(junk);
    free(M);
    free(A);
    free(all);
    return used;
}

/* Q6_K, Q3_K, Q2_K -> the Q8A16 layout: int8 codes [N][K], f32 scales and f32 offsets [N][K/16],
 * with fl(fl(code * scale) + offset) equal to the type's value: Q6_K and Q3_K (code, dl, -0)
 * (adding -0 leaves every value, a zero's sign included, unchanged); Q2_K (code, dl, -ml).
 * offs may be NULL (Q6_K, Q3_K: the offset-free layout). */
void orc_gguf_repack_q8a16(int type, const uint8_t* src, int N, int K, int8_t* codes, float* scales, float* offs) {
    for (int n = 0; n < N; n++)
        for (int k = 0; k < K; k++) {
            int code;
            float d, m;
            gguf_element(type, src, K, n, k, &code, &d, &m);
            size_t bi = (size_t)n * (K / 16) + k / 16;
            codes[(size_t)n * K + k] = (int8_t)code;
            scales[bi] = d;
            if (offs) offs[bi] = -m;
        }
}
