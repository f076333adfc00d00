/*
 * dsa.h -- C ABI of the MI355X (gfx950) DSA stage library, libdsa.so.
 *
 * The DSA stage of a hybrid KDA+DSA model, as the pages describe it: a
 * lightweight indexer scores every causal history position of each query,
 * weights the per-head scores, keeps the Top-K positions, and a sparse
 * attention core reads only those positions of the MLA latent KV cache.
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
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers documented "device" must be HIP device (or managed) memory;
 *    structs and scalars are read on the host during the call only.
 *  - Ownership: the caller owns every buffer, workspaces included.  The
 *    library allocates no memory and keeps no state between calls; calls on
 *    different streams are independent when each has its own workspace.
 *    The one exception is dsa_forward_noalloc, which works in a fixed
 *    per-GPU scratch array of the library (see there).
 *  - Asynchrony: all device work is enqueued on `stream` (a hipStream_t, or
 *    NULL for the null stream); nothing synchronizes the device.
 *  - Layout: row-major, innermost dimension contiguous.  A query row is a
 *    query token r = b*n_q + i (sequence b, query i of that sequence).
 *    Positions are logical per sequence; both paged pools share the one
 *    block table ([A] §4 "Sparse attention read": the paged layout follows
 *    the indexer's addressing).  Row r sees the causal history
 *        L_r = L_b - n_q + i + 1,  L_b = min(seq_lens[b], max_seq_len)
 *    positions (a query sees itself; queries of one step are causal among
 *    themselves, as in speculative verification).
 *  - Errors: every check that needs only host data happens before anything
 *    is launched and returns a status.  Data that lives on the device is
 *    handled by rule, never by a fault: a block-table entry outside
 *    [0, num_blocks) makes that position absent (indexer score -inf,
 *    skipped by attention); an index outside [0, L_r), such as the -1
 *    padding, is skipped; a row with nothing to attend outputs zeros and
 *    lse = -inf.  A failed launch returns DSA_ERR_HIP.  Nothing prints.
 *  - Supported shapes (anything else returns DSA_ERR_UNSUPPORTED):
 *      indexer  BF16, E4M3 + fp32 scale per 128, or MXFP8 (E4M3 + E8M0 per
 *               32): n_heads 64, head_dim 128
 *               F32: n_heads <= 16, head_dim <= 128
 *      attention BF16 q, and BF16, MXFP8 (E4M3 + E8M0 per 32) or E4M3 with
 *               an fp32 scale per 128 (groups 0..4 of a 576 row; the
 *               last covers the 64 rope channels) KV:
 *               n_heads 128, d_qk 576, d_v 512
 *               F32 q and KV: n_heads <= 16, d_qk <= 128, d_v <= d_qk
 *      block_size 64, 1 <= top_k <= 4096, any n_q >= 1 (decode, speculative
 *      verification, chunked prefill and whole-sequence prefill alike),
 *      batch <= 65535 and batch * n_q <= 2^24 (else DSA_ERR_SHAPE).
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSA_OK = 0,
    DSA_ERR_NULL = 1,         /* a required pointer is NULL                        */
    DSA_ERR_SHAPE = 2,        /* sizes inconsistent or out of range                */
    DSA_ERR_UNSUPPORTED = 3,  /* valid, but no kernel for this shape/dtype         */
    DSA_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than the size query     */
    DSA_ERR_HIP = 5           /* a HIP runtime call or kernel launch failed        */
} dsa_status;

typedef enum {
    DSA_F32 = 0,
    DSA_BF16 = 1,
    DSA_E4M3 = 2              /* OCP FP8 E4M3 ("e4m3fn": bias 7, max 448, no inf)  */
} dsa_dtype;

typedef enum {
    DSA_SCALE_NONE = 0,
    DSA_SCALE_F32 = 1,        /* one fp32 factor per `group` elements              */
    DSA_SCALE_E8M0 = 2        /* one OCP MX E8M0 byte, 2^(b-127), per `group`      */
} dsa_scale_kind;

/* A paged cache pool of num_blocks blocks of block_size (64) positions, each
 * position a row of `width` elements of `dtype`.  Index-K pool ([B] §2.1: the
 * indexer reads the paged K cache directly) and MLA latent KV pool ([D] §2.2:
 * KV compressed into a low-rank latent row per position, shared by all
 * heads).  Element c of row o of block p is at
 *     data + p*block_stride + o*row_stride + c        (in elements of dtype)
 * and, for quantized pools ([A] §5 "Layered Quantization"), its factor at
 *     scales + p*scale_block_stride + o*scale_row_stride + c/group
 * (in scale elements: fp32 or E8M0 bytes); the element value is value(code) *
 * factor, with a last, shorter group when group does not divide width.  A
 * stride of 0 means the dense layout: row_stride = width, block_stride =
 * 64*row_stride, scale_row_stride = ceil(width/group), scale_block_stride =
 * 64*scale_row_stride.  Strides are >= 0 and row_stride >= width; for BF16
 * and E4M3 pools the data pointer and both data strides (in bytes) must be
 * multiples of 16 (rows are read in 16-byte pieces), for F32 pools of 4; an
 * E8M0 index-K scale row (its four bytes) must be 4-byte aligned.  Distinct
 * positions must not overlap (the caller's layout; it is not checked). */
typedef struct {
    const void* data;           /* device, see above                               */
    const void* scales;         /* device, fp32 or E8M0 bytes; NULL when NONE      */
    dsa_dtype dtype;
    dsa_scale_kind scale_kind;
    int32_t group;              /* elements per scale: 128 (F32 kind), 32 (E8M0)   */
    int32_t width;              /* elements per position: d_I or d_qk              */
    int64_t num_blocks;         /* blocks in the pool                              */
    int64_t block_stride;       /* elements between blocks, 0: dense               */
    int64_t row_stride;         /* elements between positions of a block, 0: dense */
    int64_t scale_block_stride; /* scale elements between blocks, 0: dense         */
    int64_t scale_row_stride;   /* scale elements between positions, 0: dense      */
} dsa_cache;

/* The batch: sequences, their lengths and the shared block table ([D] §8:
 * paged KV cache). */
typedef struct {
    int32_t batch;              /* sequences                                       */
    int32_t n_q;                /* query tokens per sequence (rows = batch*n_q)    */
    const int32_t* seq_lens;    /* device [batch]: L_b, counting this step's n_q   */
    const int32_t* block_table; /* device [batch][max_blocks]: physical block ids  */
    int32_t max_blocks;         /* table row length                                */
    int32_t block_size;         /* tokens per block; must be 64                    */
    int32_t max_seq_len;        /* host bound >= every L_b; <= max_blocks*64       */
} dsa_batch;

/* Indexer inputs ([D] §4.1 "Indexer Fusion": q_idx, paged K cache, head
 * weights; [D] §4.2: the head weights come from the head-weight projection). */
typedef struct {
    const void* q;              /* device [rows][n_heads][head_dim] in dtype;      */
                                /*   BF16 and E4M3: 16-byte aligned                */
    dsa_dtype dtype;            /* F32, BF16 or E4M3; k.dtype must match           */
    const void* q_scale;        /* device, E4M3 only, same kind and group as k:    */
                                /*   [rows][n_heads][head_dim/group] fp32 or E8M0, */
                                /*   4-byte aligned                                */
    int32_t n_heads;            /* H_I                                             */
    int32_t head_dim;           /* d_I                                             */
    const float* head_w;        /* device [rows][n_heads] fp32                     */
    dsa_cache k;                /* index-K pool, width == head_dim                 */
} dsa_indexer_args;

/* Sparse attention inputs and outputs ([A] §4 "Sparse attention read";
 * [D] §2.2: the sparse core reads only the selected cache entries, in chunks).
 * K is the whole latent row [latent | rope]; V is its first d_v channels. */
typedef struct {
    const void* q;              /* device [rows][n_heads][d_qk] in dtype           */
    dsa_dtype dtype;            /* F32 or BF16; the output has the same dtype      */
    int32_t n_heads;            /* H                                               */
    int32_t d_v;                /* value channels                                  */
    float sm_scale;             /* logit scale, finite and > 0, e.g. 1/sqrt(d_qk)  */
    dsa_cache kv;               /* latent pool, width == d_qk                      */
    void* out;                  /* device [rows][n_heads][d_v] in dtype            */
    float* lse;                 /* device [rows][n_heads] natural-log LSE, or NULL */
} dsa_attn_args;

/* Human-readable name of a status code (static storage). */
const char* dsa_status_string(dsa_status s);

/* Library version as major*10000 + minor*100 + patch. */
int32_t dsa_version(void);

/*
 * dsa_indexer_scores -- relevance scoring and head-weighted sum
 * ([D] §4.1 "Indexer Fusion": per-head scoring, then the weighted sum;
 *  [A] §2 "Sparse Attention (DSA)": the indexer scores historical positions).
 *
 *   scores[r][s] = sum_j head_w[r][j] * max(0, sum_c q[r][j][c] * k[s][c])
 *
 * for s < L_r, with k[s] read through the block table and dequantized
 * (E4M3 code * fp32 scale).  Accumulation is fp32.  Only [0, L_r) of each
 * row is written.  scores: device fp32 [rows][ld_scores], ld_scores >=
 * max_seq_len.  Errors: NULL, SHAPE, UNSUPPORTED, HIP.
 */
dsa_status dsa_indexer_scores(const dsa_batch* batch, const dsa_indexer_args* idx,
                              float* scores, int64_t ld_scores, void* stream);

/* Workspace bytes dsa_topk needs for this batch and top_k (may be 0). */
size_t dsa_topk_workspace_bytes(const dsa_batch* batch, int32_t top_k);

/*
 * dsa_topk -- Top-K selection per row ([D] §4.1, its top-k step;
 * [C] §3: the fused indexer outputs only the final Top-K indices).
 *
 * For each row, the k_r = min(top_k, L_r) positions of scores[r][0:L_r]
 * with the largest values.  Ties go to the lowest position; -0.0 equals
 * +0.0.  indices: device int32 [rows][top_k], positions ascending, the
 * slots from k_r on set to -1.  Reads only scores[r][0:L_r].  Scores must
 * not be NaN (the order of NaN is unspecified).  ws may be NULL when the
 * size query returns 0.  Errors: NULL, SHAPE, WORKSPACE, HIP.
 */
dsa_status dsa_topk(const dsa_batch* batch, const float* scores, int64_t ld_scores,
                    int32_t top_k, int32_t* indices, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes dsa_sparse_attn needs (split partials across the index list). */
size_t dsa_sparse_attn_workspace_bytes(const dsa_batch* batch, const dsa_attn_args* attn,
                                       int32_t top_k);

/*
 * dsa_sparse_attn -- attention over the selected positions of the latent
 * cache ([A] §2: SFA reads only those positions; [D] §4.1: gathers the
 * selected positions from the main KV and runs chunked, parallel sparse
 * attention; [D] §5.1: the result depends only on the selected set).
 *
 * For each row r and head h, over the valid entries s of indices[r][0:top_k]
 * (0 <= s < L_r; others skipped):
 *   z_s = sm_scale * q[r][h][:] . kv[s][:],  p = softmax(z),
 *   out[r][h][:] = sum_s p_s * kv[s][0:d_v],  lse[r][h] = log sum_s exp(z_s).
 * Accumulation fp32, online softmax over chunks; out is rounded to the q
 * dtype (nearest-even for BF16).  Duplicate indices count as often as they
 * appear.  indices: device int32 [rows][top_k].  Errors: NULL, SHAPE,
 * UNSUPPORTED, WORKSPACE, HIP.
 */
dsa_status dsa_sparse_attn(const dsa_batch* batch, const dsa_attn_args* attn,
                           const int32_t* indices, int32_t top_k,
                           void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes dsa_forward needs (scores, indices when not returned, and
 * the attention partials). */
size_t dsa_forward_workspace_bytes(const dsa_batch* batch, const dsa_indexer_args* idx,
                                   const dsa_attn_args* attn, int32_t top_k);

/*
 * dsa_forward -- the whole stage: scoring -> weighting -> Top-K -> sparse
 * attention ([A] §4 "Indexer fusion" and its illustrative pipeline
 * fused_indexer then sfa; [D] §4.1).  The result equals dsa_indexer_scores,
 * then dsa_topk, then dsa_sparse_attn on the same inputs, bit for bit.  For
 * a few rows of at most 8192 positions (decode batches) the attention
 * launch selects the Top-K itself, so the stage is two launches plus the
 * split merge; otherwise the three run in turn.  indices_out: device int32
 * [rows][top_k] receiving the selected positions, or NULL.  Errors: as the
 * three calls, plus WORKSPACE.
 */
dsa_status dsa_forward(const dsa_batch* batch, const dsa_indexer_args* idx,
                       const dsa_attn_args* attn, int32_t top_k, int32_t* indices_out,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * dsa_forward_noalloc -- dsa_forward for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The same computation as dsa_forward (bit for bit), with
 * the workspace taken from the library's own per-GPU scratch array instead of
 * a caller buffer; the caller still passes every input and output.
 *
 * The array holds dsa_forward_noalloc_max_bytes() bytes (32 MiB) on every GPU
 * the library runs on, from the first call on that GPU until the process
 * ends.  A batch whose dsa_forward_workspace_bytes exceeds it returns
 * DSA_ERR_WORKSPACE before anything is launched (the decode workloads fit;
 * long prefills do not).  Calls on one GPU share its array, so calls that
 * overlap on one GPU (different streams, different host threads) race; calls
 * on one stream are ordered and safe.  Nothing here allocates: no hipMalloc,
 * no hipFree, no allocating library routine.  Errors: as dsa_forward, plus
 * HIP when the array's device address cannot be obtained.
 */
dsa_status dsa_forward_noalloc(const dsa_batch* batch, const dsa_indexer_args* idx,
                               const dsa_attn_args* attn, int32_t top_k, int32_t* indices_out,
                               void* stream);

/* Bytes of the per-GPU scratch array dsa_forward_noalloc works in. */
size_t dsa_forward_noalloc_max_bytes(void);

/*
 * dsa_cache_append -- write this step's index keys and latent KV rows into the
 * paged pools, quantizing them when the pool is quantized ([A] §5 "Layered
 * Quantization": dynamic quantization, scales computed in the operator that
 * writes the cache; [D] §4.2).
 *
 * Row r = b*n_q + i is the token at position s = L_b - n_q + i of sequence b
 * (the last position row r sees).  k_new[r][0:k->width] is stored at the
 * index-K pool row of s and kv_new[r][0:kv->width] at the latent pool row of
 * s; a row with s < 0 or an absent block is skipped.  Per pool format:
 *   BF16 or F32 (no scales): a bit-for-bit copy of k_new/kv_new, which have
 *       the pool's dtype (NaN payloads are kept as they are);
 *   E4M3 + F32 scale per `group` (a power of two, 4 to 256): scale =
 *       amax/448 (1 when amax = 0), code = e4m3(x/scale);
 *   E4M3 + E8M0 scale per `group` (32): e = floor(log2 amax) - 8 (-127 when
 *       amax = 0, clamped to [-127, 127]), code = e4m3(x * 2^-e), byte e + 127;
 * with amax over the group (a shorter last group when group does not divide
 * the width), the quotient clamped to +-448 and rounded to the nearest e4m3
 * (ties to even), all in fp32; quantized pools take BF16 input.  The pools'
 * `data` and `scales` are written (device memory the caller owns).
 * new_dtype: F32 (F32 pools) or BF16.  Widths: multiples of 4, at most 256
 * (index key) and 768 (latent row).  Errors: NULL, SHAPE, UNSUPPORTED, HIP.
 */
dsa_status dsa_cache_append(const dsa_batch* batch, const void* k_new, const void* kv_new,
                            dsa_dtype new_dtype, const dsa_cache* k, const dsa_cache* kv,
                            void* stream);

/* Indexer prolog inputs and outputs ([D] §4.2 "Three-Stream Coordination for
 * Indexer Preprocessing"; [A] §4 "Three-stream coordination in input
 * preparation"): what the indexer of one step needs, made from each query
 * token's hidden state. */
typedef struct {
    int32_t rows;               /* query tokens, at most 4194240 (0: nothing to do) */
    int32_t d_x;                /* hidden width: a positive multiple of 256        */
    int32_t n_heads;            /* H_I >= 1                                        */
    int32_t head_dim;           /* d_I: a multiple of 32, at most 256              */
    const void* x;              /* device bf16 [rows][d_x]: hidden states          */
    const void* w_q;            /* device bf16 [n_heads*head_dim][d_x]             */
    const void* w_h;            /* device bf16 [n_heads][d_x]                      */
    const void* k;              /* device bf16 [rows][head_dim]: new index keys    */
    const float* k_gain;        /* device fp32 [head_dim]: normalization gain      */
    float eps;                  /* normalization epsilon, finite and >= 0          */
    dsa_dtype q_dtype;          /* BF16, or E4M3 with E8M0 scales per 32 (MXFP8)   */
    void* q_out;                /* device [rows][n_heads][head_dim] in q_dtype     */
    void* q_scale_out;          /* device E8M0 [rows][n_heads][head_dim/32] (E4M3) */
    float* head_w_out;          /* device fp32 [rows][n_heads]                     */
    void* k_out;                /* device bf16 [rows][head_dim]: normalized keys   */
} dsa_prolog_args;

/*
 * dsa_indexer_prolog -- the indexer's input preparation ([D] §4.2: query
 * projection, key normalization, query quantization and head-weight
 * projection, the independent ones overlapped; [A] §5: projections in BF16,
 * the index query in MXFP8 with one scale per 32 elements).
 *
 *   q[r][n]      = sum_c w_q[n][c] * x[r][c]    (n = head*head_dim + channel)
 *   head_w[r][j] = sum_c w_h[j][c] * x[r][c]
 *   k_out[r][c]  = k[r][c] * k_gain[c] / sqrt(mean_c' k[r][c']^2 + eps)
 *
 * Projections accumulate in fp32.  q is stored nearest-even in BF16, or as
 * MXFP8 from the fp32 values: per 32 channels e = floor(log2 amax) - 8 (-127
 * when amax = 0, clamped to [-127, 127]), code = e4m3(x * 2^-e) with the
 * quotient clamped to +-448 (nearest, ties to even), scale byte e + 127 --
 * the layout dsa_indexer_args takes for an E4M3 query with E8M0 scales.
 * k_out is rounded nearest-even to BF16 and is what dsa_cache_append stores
 * as the index key (with eps = 0, an all-zero key gives NaN, 0/0).  All branches run in one launch on `stream`.  Alignment
 * (else SHAPE): x, w_q and w_h 16 bytes, q_out 8, head_w_out and k_gain 4,
 * k and k_out 2.  Errors: NULL, SHAPE, UNSUPPORTED, HIP.
 */
dsa_status dsa_indexer_prolog(const dsa_prolog_args* p, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
