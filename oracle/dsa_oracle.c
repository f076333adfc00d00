/*
 * dsa_oracle.c -- plain, slow, fp64 CPU oracle for the DSA stage
 * (Lightning Indexer scoring -> Top-K -> Sparse Flash Attention).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or helper with
 * the HIP library: every format decoder below is written from the format's
 * definition, and every loop follows the pages' description of the method.
 *
 * Pages cited (Baidu AI Cloud articles), tagged for brevity:
 *  [A] "Day0 Inference Adaptation and Performance Optimization for a New
 *       Architecture Domestic Large Language Model on Ascend"
 *  [B] "Day0 Inference Optimization for New Architecture LLMs Based on CANN"
 *  [C] "Optimizing LLM Inference for New Architectures: Day-0 Adaptation,
 *       Sparse Attention, and Long-Sequence Parallelism"
 *  [D] "Day0 Inference Adaptation and Performance Optimization for
 *       New-Architecture LLMs"
 *  [E] "Inference Optimization for a Novel LLM Architecture: From Operator
 *       Fusion to Multi-Dimensional Parallelism"
 *
 * What is computed (the pages give prose, no formulas; where they are silent
 * the plainest reading is taken):
 *  1. dequantize every input to fp64 (value(code) * scale) -- exact;
 *  2. indexer: I[r,s] = sum_j w[r,j] * max(0, sum_c qI[r,j,c] * kI[s,c])
 *     for every causal history position s < L_r  ([A] §2 "Sparse Attention
 *     (DSA)", [D] §4.1 "Indexer Fusion": relevance scoring then per-head
 *     weighted aggregation; the ReLU is the stated nonlinearity);
 *  3. Top-K: the k_r = min(top_k, L_r) positions with the largest I, ties to
 *     the lowest position, emitted in ascending order, padded with -1
 *     ([D] §4.1, its top-k step; only the set matters, [D] §5.1);
 *  4. sparse attention over the selected positions of the MLA latent cache:
 *     z_s = sm_scale * q[r,h,:].kv[s,:], two-pass softmax, out = sum p_s *
 *     kv[s, :d_v], lse = m + log sum exp(z - m)  ([A] §2, [D] §2.2: the
 *     sparse core reads only the selected KV entries);
 *  5. dense causal attention over all s < L_r (used only by invariants);
 *  6. cache append: this step's index keys and latent rows written into the
 *     paged pools, copied when the pool has the input's format, quantized in
 *     fp32 when the pool is e4m3 (the quantizer's decisions are integer
 *     codes, so they are taken in the kernel's fp32);
 *  7. indexer prolog: the index query and head weights projected from the
 *     hidden state and the new index key RMS-normalized, exactly in fp64
 *     ([D] §4.2 "Three-Stream Coordination for Indexer Preprocessing").
 *
 * Paging ([A] §4 "Sparse attention read"; [D] §8 "Paged KV cache"): logical
 * position s of sequence b lives at pool row
 *     block_table[b*max_blocks + s/block_size]*block_size + s%block_size.
 * Positions whose physical block is outside [0, num_blocks) are absent:
 * the indexer gives them score -inf and attention skips them.
 *
 * Row r = b*n_q + i sees L_r = seq_lens[b] - n_q + i + 1 positions (the
 * query sees itself; decode with n_q > 1 is causal between its queries).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* dtype codes understood by the oracle (its own numbering) */
#define ORC_F32  0
#define ORC_BF16 1
#define ORC_E4M3 2

/* scale kinds */
#define ORC_SCALE_NONE 0
#define ORC_SCALE_F32  1   /* one fp32 factor per group of `group` elements   */
#define ORC_SCALE_E8M0 2   /* one power-of-two factor 2^(byte-127) per group  */

/* ---------------------------------------------------------------- formats */

/* bfloat16: the upper 16 bits of an IEEE-754 binary32. */
double oracle_bf16_to_f64(uint16_t h) {
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits.
 * Exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN; there is no
 * infinity, so the largest finite magnitude is 1.75 * 2^8 = 448. */
double oracle_e4m3_to_f64(uint8_t c) {
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 0xF;
    int m = c & 0x7;
    double v;
    if (e == 0xF && m == 0x7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* OCP MX E8M0 shared scale: 2^(byte - 127); byte 0xFF is NaN. */
double oracle_e8m0_to_f64(uint8_t b) {
    if (b == 0xFF) return NAN;
    return ldexp(1.0, (int)b - 127);
}

static double load_elem(const void* base, int dtype, int64_t idx) {
    switch (dtype) {
    case ORC_F32:  return (double)((const float*)base)[idx];
    case ORC_BF16: return oracle_bf16_to_f64(((const uint16_t*)base)[idx]);
    case ORC_E4M3: return oracle_e4m3_to_f64(((const uint8_t*)base)[idx]);
    default: return NAN;
    }
}

static double load_scale(const void* scales, int kind, int64_t idx) {
    if (kind == ORC_SCALE_F32) return (double)((const float*)scales)[idx];
    if (kind == ORC_SCALE_E8M0) return oracle_e8m0_to_f64(((const uint8_t*)scales)[idx]);
    return 1.0;
}

/* Dequantize one vector of `width` elements that starts at element `row*width`
 * of `data`; element c belongs to group c/group, and the row's groups share
 * scales number row*ngroups + c/group, ngroups = ceil(width/group) (a last,
 * shorter group when group does not divide width, as for the 576-wide
 * latent row in groups of 128). */
static void dequant_row(const void* data, int dtype, const void* scales, int scale_kind,
                        int group, int width, int64_t row, double* out) {
    int ngroups = (scale_kind == ORC_SCALE_NONE || group <= 0) ? 0 : (width + group - 1) / group;
    for (int c = 0; c < width; ++c) {
        double v = load_elem(data, dtype, row * (int64_t)width + c);
        if (ngroups > 0) v *= load_scale(scales, scale_kind, row * (int64_t)ngroups + c / group);
        out[c] = v;
    }
}

/* Exported for the tests: dequantize n vectors of `width` elements. */
int oracle_dequant(const void* data, int dtype, const void* scales, int scale_kind,
                   int group, int width, int64_t n, double* out) {
    for (int64_t r = 0; r < n; ++r)
        dequant_row(data, dtype, scales, scale_kind, group, width, r, out + r * width);
    return 0;
}

/* ----------------------------------------------------------- batch layout */

typedef struct {
    int batch, n_q;
    const int32_t* seq_lens;     /* [batch], includes this step's n_q tokens */
    const int32_t* block_table;  /* [batch][max_blocks] physical block ids    */
    int max_blocks, block_size;
    int64_t num_blocks;          /* blocks in the pool                        */
} orc_batch;

static int history_len(const orc_batch* B, int r) {
    int b = r / B->n_q, i = r % B->n_q;
    int L = B->seq_lens[b] - B->n_q + i + 1;
    return L < 0 ? 0 : L;
}

/* pool row of logical position s of sequence b, or -1 when absent */
static int64_t pool_row(const orc_batch* B, int b, int s) {
    int j = s / B->block_size;
    if (j >= B->max_blocks) return -1;
    int64_t phys = B->block_table[(int64_t)b * B->max_blocks + j];
    if (phys < 0 || phys >= B->num_blocks) return -1;
    return phys * B->block_size + s % B->block_size;
}

/* ---------------------------------------------------------------- indexer */

/* Indexer scores for the `n_rows` query rows listed in `rows` (all rows when
 * rows == NULL).  Output row i of `scores` (leading dimension ld) holds
 * I[rows[i], s] for s < L_r and NaN beyond.
 *  q_idx   [rows_total, H_I, d_I] in q_dtype; q_scale [rows_total, H_I, d_I/q_group]
 *          of kind q_kind (fp32 factors or E8M0 bytes)
 *  head_w  [rows_total, H_I] fp32
 *  k_pool  [num_blocks*block_size, d_I] in k_dtype; k_scale [.., d_I/k_group] of kind k_kind */
int oracle_indexer_scores(int batch, int n_q, const int32_t* seq_lens, const int32_t* block_table,
                          int max_blocks, int block_size, int64_t num_blocks,
                          const void* q_idx, int q_dtype, const void* q_scale, int q_kind, int q_group,
                          int n_idx_heads, int d_idx, const float* head_w,
                          const void* k_pool, int k_dtype, const void* k_scale, int k_kind, int k_group,
                          const int32_t* rows, int n_rows, double* scores, int64_t ld) {
    orc_batch B = {batch, n_q, seq_lens, block_table, max_blocks, block_size, num_blocks};
    if (q_scale == NULL) q_kind = ORC_SCALE_NONE;
    if (k_scale == NULL) k_kind = ORC_SCALE_NONE;
    if (rows == NULL) n_rows = batch * n_q;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < n_rows; ++i) {
        int r = rows ? rows[i] : i;
        int b = r / n_q;
        int L = history_len(&B, r);
        double* q = (double*)malloc(sizeof(double) * (size_t)n_idx_heads * d_idx);
        double* k = (double*)malloc(sizeof(double) * (size_t)d_idx);
        for (int j = 0; j < n_idx_heads; ++j)
            dequant_row(q_idx, q_dtype, q_scale, q_kind, q_group, d_idx,
                        (int64_t)r * n_idx_heads + j, q + (size_t)j * d_idx);
        double* out = scores + (int64_t)i * ld;
        for (int64_t s = 0; s < ld; ++s) out[s] = NAN;
        for (int s = 0; s < L; ++s) {
            int64_t pr = pool_row(&B, b, s);
            if (pr < 0) { out[s] = -INFINITY; continue; }
            dequant_row(k_pool, k_dtype, k_scale, k_kind, k_group, d_idx, pr, k);
            double I = 0.0;
            for (int j = 0; j < n_idx_heads; ++j) {
                double d = 0.0;
                for (int c = 0; c < d_idx; ++c) d += q[(size_t)j * d_idx + c] * k[c];
                double relu = d > 0.0 ? d : 0.0;
                I += (double)head_w[(int64_t)r * n_idx_heads + j] * relu;
            }
            out[s] = I;
        }
        free(q);
        free(k);
    }
    return 0;
}

/* ------------------------------------------------------------------ top-k */

typedef struct { double v; int32_t pos; } scored_pos;

/* order: larger score first; equal scores (+0 and -0 are equal) keep the
 * lower position first -- the result of a stable descending sort */
static int cmp_desc_then_pos(const void* a, const void* b) {
    const scored_pos* x = (const scored_pos*)a;
    const scored_pos* y = (const scored_pos*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->pos > y->pos) - (x->pos < y->pos);
}

static int cmp_int32(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/* Per row i: select from scores[i, 0:row_len[i]] the min(top_k, row_len[i])
 * largest, ties to the lowest position; write them ascending into
 * indices[i, 0:top_k] and -1 into the unused slots. */
int oracle_topk(int n_rows, const int32_t* row_len, const double* scores, int64_t ld,
                int top_k, int32_t* indices) {
    #pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < n_rows; ++i) {
        int L = row_len[i];
        int k = L < top_k ? L : top_k;
        scored_pos* a = (scored_pos*)malloc(sizeof(scored_pos) * (size_t)(L > 0 ? L : 1));
        for (int s = 0; s < L; ++s) { a[s].v = scores[(int64_t)i * ld + s]; a[s].pos = s; }
        qsort(a, (size_t)L, sizeof(scored_pos), cmp_desc_then_pos);
        int32_t* out = indices + (int64_t)i * top_k;
        for (int t = 0; t < k; ++t) out[t] = a[t].pos;
        qsort(out, (size_t)k, sizeof(int32_t), cmp_int32);
        for (int t = k; t < top_k; ++t) out[t] = -1;
        free(a);
    }
    return 0;
}

/* -------------------------------------------------------- sparse attention */

/* Attention of one row over a list of positions (already validated and
 * dequantized into kvrows[n][d_qk]).  Two-pass softmax in fp64. */
static void attend_row(const double* q, int n_heads, int d_qk, int d_v,
                       const double* kvrows, int n, double sm_scale,
                       double* out, double* lse, double* z) {
    for (int h = 0; h < n_heads; ++h) {
        const double* qh = q + (size_t)h * d_qk;
        double* oh = out + (size_t)h * d_v;
        for (int c = 0; c < d_v; ++c) oh[c] = 0.0;
        if (n == 0) { lse[h] = -INFINITY; continue; }
        double m = -INFINITY;
        for (int t = 0; t < n; ++t) {
            double acc = 0.0;
            for (int c = 0; c < d_qk; ++c) acc += qh[c] * kvrows[(size_t)t * d_qk + c];
            z[t] = sm_scale * acc;
            if (z[t] > m) m = z[t];
        }
        double sum = 0.0;
        for (int t = 0; t < n; ++t) sum += exp(z[t] - m);
        for (int t = 0; t < n; ++t) {
            double p = exp(z[t] - m) / sum;
            for (int c = 0; c < d_v; ++c) oh[c] += p * kvrows[(size_t)t * d_qk + c];
        }
        lse[h] = m + log(sum);
    }
}

/* Shared driver: when `indices` is NULL every position s < L_r is used
 * (dense causal attention); otherwise the row's index list, where entries
 * outside [0, L_r) -- including the -1 padding -- are skipped.
 *  q       [rows_total, H, d_qk] in q_dtype
 *  kv_pool [num_blocks*block_size, d_qk] in kv_dtype, scales per group
 *  out     [n_rows, H, d_v] fp64 ; lse [n_rows, H] fp64 */
static int attention_impl(int batch, int n_q, const int32_t* seq_lens, const int32_t* block_table,
                          int max_blocks, int block_size, int64_t num_blocks,
                          const void* q, int q_dtype, int n_heads, int d_qk, int d_v,
                          const void* kv_pool, int kv_dtype, const void* kv_scale, int kv_scale_kind,
                          int kv_group, const int32_t* indices, int top_k, double sm_scale,
                          const int32_t* rows, int n_rows, double* out, double* lse) {
    orc_batch B = {batch, n_q, seq_lens, block_table, max_blocks, block_size, num_blocks};
    if (rows == NULL) n_rows = batch * n_q;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < n_rows; ++i) {
        int r = rows ? rows[i] : i;
        int b = r / n_q;
        int L = history_len(&B, r);
        int cap = indices ? top_k : L;
        double* qd = (double*)malloc(sizeof(double) * (size_t)n_heads * d_qk);
        double* kvr = (double*)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1) * d_qk);
        double* z = (double*)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1));
        for (int h = 0; h < n_heads; ++h)
            dequant_row(q, q_dtype, NULL, ORC_SCALE_NONE, 0, d_qk, (int64_t)r * n_heads + h,
                        qd + (size_t)h * d_qk);
        int n = 0;
        for (int t = 0; t < cap; ++t) {
            int s = indices ? indices[(int64_t)r * top_k + t] : t;
            if (s < 0 || s >= L) continue;
            int64_t pr = pool_row(&B, b, s);
            if (pr < 0) continue;
            dequant_row(kv_pool, kv_dtype, kv_scale, kv_scale_kind, kv_group, d_qk, pr,
                        kvr + (size_t)n * d_qk);
            ++n;
        }
        attend_row(qd, n_heads, d_qk, d_v, kvr, n, sm_scale,
                   out + (int64_t)i * n_heads * d_v, lse + (int64_t)i * n_heads, z);
        free(qd);
        free(kvr);
        free(z);
    }
    return 0;
}

/* Sparse attention over the index lists `indices[rows_total, top_k]`. */
int oracle_sparse_attn(int batch, int n_q, const int32_t* seq_lens, const int32_t* block_table,
                       int max_blocks, int block_size, int64_t num_blocks,
                       const void* q, int q_dtype, int n_heads, int d_qk, int d_v,
                       const void* kv_pool, int kv_dtype, const void* kv_scale, int kv_scale_kind,
                       int kv_group, const int32_t* indices, int top_k, double sm_scale,
                       const int32_t* rows, int n_rows, double* out, double* lse) {
    if (!indices) return -1;
    return attention_impl(batch, n_q, seq_lens, block_table, max_blocks, block_size, num_blocks,
                          q, q_dtype, n_heads, d_qk, d_v, kv_pool, kv_dtype, kv_scale,
                          kv_scale_kind, kv_group, indices, top_k, sm_scale, rows, n_rows,
                          out, lse);
}

/* Dense causal attention over every position s < L_r. */
int oracle_dense_attn(int batch, int n_q, const int32_t* seq_lens, const int32_t* block_table,
                      int max_blocks, int block_size, int64_t num_blocks,
                      const void* q, int q_dtype, int n_heads, int d_qk, int d_v,
                      const void* kv_pool, int kv_dtype, const void* kv_scale, int kv_scale_kind,
                      int kv_group, double sm_scale,
                      const int32_t* rows, int n_rows, double* out, double* lse) {
    return attention_impl(batch, n_q, seq_lens, block_table, max_blocks, block_size, num_blocks,
                          q, q_dtype, n_heads, d_qk, d_v, kv_pool, kv_dtype, kv_scale,
                          kv_scale_kind, kv_group, NULL, 0, sm_scale, rows, n_rows, out, lse);
}

/* ------------------------------------------------------------ cache append */

/* Nearest-even rounding of a non-negative double to an integer. */
static double round_half_even(double q) {
    double f = floor(q), d = q - f;
    if (d > 0.5) return f + 1.0;
    if (d < 0.5) return f;
    return fmod(f, 2.0) == 0.0 ? f : f + 1.0;
}

/* OCP FP8 E4M3 code of a float, from the format's definition: magnitudes
 * below 2^-6 on the subnormal grid m * 2^-9, the others as (1 + m/8) * 2^E,
 * E in [-6, 8], both rounded to the nearest code (ties to the even mantissa);
 * magnitudes above 448 saturate to 448; NaN gives 0x7F. */
uint8_t oracle_f32_to_e4m3(float x) {
    if (isnan(x)) return 0x7F;
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs((double)x);
    if (a > 448.0) a = 448.0;
    if (a < ldexp(1.0, -6)) return (uint8_t)(sign | (uint8_t)round_half_even(a / ldexp(1.0, -9)));
    int e2;
    frexp(a, &e2);              /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;             /* floor(log2 a) */
    double m = round_half_even((a / ldexp(1.0, E) - 1.0) * 8.0);
    if (m == 8.0) { m = 0.0; E += 1; }
    return (uint8_t)(sign | ((E + 7) << 3) | (int)m);
}

/* Quantize one vector of `width` values (fp32) into `codes` with one scale per
 * `group` elements (a shorter last group when group does not divide width),
 * in fp32 as the dynamic quantization of the pages' layered quantization
 * ([A] §5 "Layered Quantization"; [D] §4.2: scales computed in the adjacent
 * operator):
 *   ORC_SCALE_F32:  scale = amax/448 (1 when amax = 0), code = e4m3(x/scale)
 *   ORC_SCALE_E8M0: e = floor(log2 amax) - 8 (-127 when amax = 0), clamped to
 *                   [-127, 127]; code = e4m3(x * 2^-e); the byte is e + 127
 * The quotient is clamped to +-448 before the rounding. */
static void quantize_vector(const float* x, int width, int kind, int group, uint8_t* codes, void* scales) {
    int ng = (width + group - 1) / group;
    for (int g = 0; g < ng; ++g) {
        int c0 = g * group, c1 = c0 + group < width ? c0 + group : width;
        float amax = 0.0f;
        for (int c = c0; c < c1; ++c) amax = fabsf(x[c]) > amax ? fabsf(x[c]) : amax;
        if (kind == ORC_SCALE_F32) {
            volatile float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
            ((float*)scales)[g] = scale;
            for (int c = c0; c < c1; ++c) {
                volatile float v = x[c] / scale;
                float w = v > 448.0f ? 448.0f : (v < -448.0f ? -448.0f : v);
                codes[c] = oracle_f32_to_e4m3(w);
            }
        } else {
            int e2 = 0;
            frexpf(amax, &e2);
            int e = amax > 0.0f ? e2 - 1 - 8 : -127;
            e = e < -127 ? -127 : (e > 127 ? 127 : e);
            ((uint8_t*)scales)[g] = (uint8_t)(e + 127);
            for (int c = c0; c < c1; ++c) {
                volatile float v = ldexpf(x[c], -e);   /* exact: a power-of-two scaling */
                float w = v > 448.0f ? 448.0f : (v < -448.0f ? -448.0f : v);
                codes[c] = oracle_f32_to_e4m3(w);
            }
        }
    }
}

/* Cache append: row r = b*n_q + i is this step's token at position
 * s = L_b - n_q + i of sequence b; its `width` values x_new[r] are written to
 * the pool row of s (skipped when s < 0 or its block is absent).  The pool
 * formats and the input each one takes:
 *   ORC_F32 pool,  fp32 input (x_dtype ORC_F32): the values, copied;
 *   ORC_BF16 pool, bf16 input (x_dtype ORC_BF16): the 16-bit codes, copied
 *                  bit for bit (NaN payloads included);
 *   ORC_E4M3 pool, bf16 input: each code decoded to fp32 (exact), then e4m3
 *                  codes plus scales (scale kind and group as above).
 * Any other pairing returns -1 and writes nothing.  x_new: [rows][width] of
 * x_dtype; scales: [pool rows][ceil(width/group)]. */
int oracle_cache_append(int batch, int n_q, const int32_t* seq_lens, const int32_t* block_table,
                        int max_blocks, int block_size, int64_t num_blocks, const void* x_new, int x_dtype,
                        int width, int dtype, int scale_kind, int group, void* pool, void* scales) {
    if (!((dtype == ORC_F32 && x_dtype == ORC_F32) || (dtype == ORC_BF16 && x_dtype == ORC_BF16) ||
          (dtype == ORC_E4M3 && x_dtype == ORC_BF16)))
        return -1;
    orc_batch B = {batch, n_q, seq_lens, block_table, max_blocks, block_size, num_blocks};
    int ng = scale_kind == ORC_SCALE_NONE ? 0 : (width + group - 1) / group;
    float* row = (float*)malloc(sizeof(float) * (size_t)width);
    if (row == NULL) return -1;
    for (int r = 0; r < batch * n_q; ++r) {
        int b = r / n_q;
        int s = history_len(&B, r) - 1;
        if (s < 0) continue;
        int64_t pr = pool_row(&B, b, s);
        if (pr < 0) continue;
        if (dtype == ORC_F32) {
            memcpy((float*)pool + pr * width, (const float*)x_new + (int64_t)r * width,
                   sizeof(float) * (size_t)width);
        } else if (dtype == ORC_BF16) {
            memcpy((uint16_t*)pool + pr * width, (const uint16_t*)x_new + (int64_t)r * width,
                   sizeof(uint16_t) * (size_t)width);
        } else {
            const uint16_t* xb = (const uint16_t*)x_new + (int64_t)r * width;
            for (int c = 0; c < width; ++c) row[c] = (float)oracle_bf16_to_f64(xb[c]);  /* exact */
            uint8_t* codes = (uint8_t*)pool + pr * width;
            void* sc = scale_kind == ORC_SCALE_F32 ? (void*)((float*)scales + pr * ng)
                                                   : (void*)((uint8_t*)scales + pr * ng);
            quantize_vector(row, width, scale_kind, group, codes, sc);
        }
    }
    free(row);
    return 0;
}

/* Exported for the tests: e4m3 codes of n floats (the encoder above). */
int oracle_e4m3_encode(const float* x, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_e4m3(x[i]);
    return 0;
}

/* ---------------------------------------------------------- indexer prolog */

/* Indexer prolog ([D] §4.2 "Three-Stream Coordination for Indexer
 * Preprocessing"; [A] §4 "Three-stream coordination in input preparation"):
 * the inputs of the indexer made from each query token's hidden state x,
 *   q[r][n]      = sum_c W_q[n][c] * x[r][c]     for n < n_heads*head_dim
 *                  (the query projection, n = head*head_dim + channel)
 *   head_w[r][j] = sum_c W_h[j][c] * x[r][c]     for j < n_heads
 *                  (the head-weight projection)
 *   k_norm[r][c] = k[r][c] * gain[c] / sqrt(mean_c' k[r][c']^2 + eps)
 *                  (the RMS normalization of the new index key)
 * in fp64 on the decoded bf16 inputs (x [rows][d_x], W_q [n_heads*head_dim]
 * [d_x], W_h [n_heads][d_x], k [rows][head_dim]; gain fp32 [head_dim]).  The
 * projections use bf16 operands as the pages keep them ([A] §5: projections
 * stay BF16); quantizing q for the index path ([A] §5: MXFP8, one scale per
 * 32) and rounding outputs to bf16 are decisions taken from these values. */
int oracle_indexer_prolog(int rows, int d_x, const uint16_t* x, const uint16_t* w_q,
                          const uint16_t* w_h, const uint16_t* k, const float* gain, double eps,
                          int n_heads, int head_dim, double* q, double* head_w, double* k_norm) {
    const int nq = n_heads * head_dim, ncols = nq + n_heads;
    double* xd = (double*)malloc(sizeof(double) * (size_t)rows * (size_t)d_x);
    if (!xd) return -1;
    for (int64_t i = 0; i < (int64_t)rows * d_x; ++i) xd[i] = oracle_bf16_to_f64(x[i]);
    #pragma omp parallel
    {
        double* wrow = (double*)malloc(sizeof(double) * (size_t)d_x);
        #pragma omp for schedule(dynamic, 16)
        for (int n = 0; n < ncols; ++n) {
            const uint16_t* src = n < nq ? w_q + (int64_t)n * d_x : w_h + (int64_t)(n - nq) * d_x;
            for (int c = 0; c < d_x; ++c) wrow[c] = oracle_bf16_to_f64(src[c]);
            for (int r = 0; r < rows; ++r) {
                double acc = 0.0;
                for (int c = 0; c < d_x; ++c) acc += wrow[c] * xd[(int64_t)r * d_x + c];
                if (n < nq) q[(int64_t)r * nq + n] = acc;
                else head_w[(int64_t)r * n_heads + (n - nq)] = acc;
            }
        }
        free(wrow);
    }
    free(xd);
    for (int r = 0; r < rows; ++r) {
        double ss = 0.0;
        for (int c = 0; c < head_dim; ++c) {
            double v = oracle_bf16_to_f64(k[(int64_t)r * head_dim + c]);
            ss += v * v;
        }
        double inv = 1.0 / sqrt(ss / head_dim + eps);
        for (int c = 0; c < head_dim; ++c)
            k_norm[(int64_t)r * head_dim + c] =
                oracle_bf16_to_f64(k[(int64_t)r * head_dim + c]) * (double)gain[c] * inv;
    }
    return 0;
}

/* Number of OpenMP threads a parallel region of the oracle will use. */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
