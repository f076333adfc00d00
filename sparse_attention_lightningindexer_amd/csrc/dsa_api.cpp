// dsa_api.cpp -- the C ABI of libdsa (declared in include/dsa.h).
//
// Host-side only: argument validation (every check that needs no device data
// happens before anything is enqueued), workspace sizing and carving, and
// dispatch to the gfx950 kernels on the caller's stream.  No allocation, no
// synchronization, no global state.
#include <limits.h>
#include <stdint.h>
#include <stddef.h>

#include "dsa.h"
#include "kernels.hpp"

namespace {

constexpr int kMaxTopK = 4096;
constexpr int kMaxBatch = 65535;       // sequences form a grid dimension of the indexer
constexpr int64_t kMaxRows = 1 << 24;  // query rows (batch * n_q)
constexpr size_t kAlign = 256;
constexpr int kPrologChunk = 256;  // the prolog's hidden width must be a multiple of this

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

dsa_status check_batch(const dsa_batch* b) {
    if (b == nullptr) return DSA_ERR_NULL;
    if (b->batch < 0 || b->n_q < 1 || b->block_size != 64 || b->max_blocks < 1 || b->max_seq_len < 0)
        return DSA_ERR_SHAPE;
    if ((int64_t)b->max_seq_len > (int64_t)b->max_blocks * 64) return DSA_ERR_SHAPE;
    if (b->batch > kMaxBatch || (int64_t)b->batch * b->n_q > kMaxRows) return DSA_ERR_SHAPE;
    if (b->batch > 0 && (b->seq_lens == nullptr || b->block_table == nullptr)) return DSA_ERR_NULL;
    return DSA_OK;
}

// A pool's byte layout from its element strides (0: the dense layout).
// SHAPE when a stride is negative or too large, a row is narrower than the
// width, or an alignment the kernels rely on does not hold: rows of BF16 and
// E4M3 pools are read in 16-byte pieces, F32 rows and fp32 scales in 4 bytes.
dsa_status pool_layout(const dsa_cache* c, dsa::PoolLayout* L) {
    const int esz = c->dtype == DSA_F32 ? 4 : c->dtype == DSA_BF16 ? 2 : 1;
    const bool scaled = c->scale_kind != DSA_SCALE_NONE;
    const int ng = scaled && c->group > 0 ? (c->width + c->group - 1) / c->group : 0;
    const int ssz = c->scale_kind == DSA_SCALE_F32 ? 4 : 1;
    constexpr int64_t kMaxStride = int64_t(1) << 40;
    const int64_t in[4] = {c->block_stride, c->row_stride, c->scale_block_stride, c->scale_row_stride};
    for (int64_t v : in)
        if (v < 0 || v > kMaxStride) return DSA_ERR_SHAPE;
    const int64_t rs = c->row_stride != 0 ? c->row_stride : c->width;
    if (rs < c->width) return DSA_ERR_SHAPE;
    const int64_t bs = c->block_stride != 0 ? c->block_stride : 64 * rs;
    const int64_t srs = c->scale_row_stride != 0 ? c->scale_row_stride : ng;
    if (scaled && srs < ng) return DSA_ERR_SHAPE;
    const int64_t sbs = c->scale_block_stride != 0 ? c->scale_block_stride : 64 * srs;
    const int64_t align = esz == 4 ? 4 : 16;
    if ((uintptr_t)c->data % align != 0 || (rs * esz) % align != 0 || (bs * esz) % align != 0) return DSA_ERR_SHAPE;
    if (scaled && ssz == 4 && ((uintptr_t)c->scales % 4 != 0)) return DSA_ERR_SHAPE;
    L->bs = bs * esz;
    L->rs = rs * esz;
    L->sbs = sbs * ssz;
    L->srs = srs * ssz;
    return DSA_OK;
}

dsa::PoolLayout layout_of(const dsa_cache* c) {
    dsa::PoolLayout L{};
    (void)pool_layout(c, &L);  // validated before any launch
    return L;
}

dsa_status check_pool(const dsa_cache* c, int width) {
    if (c->data == nullptr) return DSA_ERR_NULL;
    if (c->num_blocks < 1 || c->width != width) return DSA_ERR_SHAPE;
    if (c->num_blocks * 64 > (int64_t)INT_MAX) return DSA_ERR_UNSUPPORTED;  // pool rows are int32
    dsa::PoolLayout L;
    return pool_layout(c, &L);
}

dsa_status check_indexer(const dsa_batch* b, const dsa_indexer_args* a) {
    if (a == nullptr) return DSA_ERR_NULL;
    if (b->batch > 0 && (a->q == nullptr || a->head_w == nullptr)) return DSA_ERR_NULL;
    dsa_status s = check_pool(&a->k, a->head_dim);
    if (s != DSA_OK) return s;
    if (a->k.dtype != a->dtype) return DSA_ERR_UNSUPPORTED;
    switch (a->dtype) {
    case DSA_F32:
        if (a->n_heads < 1 || a->n_heads > 16 || a->head_dim < 1 || a->head_dim > 128) return DSA_ERR_UNSUPPORTED;
        if (a->k.scale_kind != DSA_SCALE_NONE) return DSA_ERR_UNSUPPORTED;
        return DSA_OK;
    case DSA_BF16:
        if (a->n_heads != 64 || a->head_dim != 128) return DSA_ERR_UNSUPPORTED;
        if (a->k.scale_kind != DSA_SCALE_NONE) return DSA_ERR_UNSUPPORTED;
        // queries arrive in 16-byte pieces, head weights in 4-byte ones
        if ((uintptr_t)a->q % 16 != 0 || (uintptr_t)a->head_w % 4 != 0) return DSA_ERR_SHAPE;
        return DSA_OK;
    case DSA_E4M3:  // fp32 per 128 (one per head vector) or MXFP8 (E8M0 per 32)
        if (a->n_heads != 64 || a->head_dim != 128) return DSA_ERR_UNSUPPORTED;
        if (!((a->k.scale_kind == DSA_SCALE_F32 && a->k.group == 128) ||
              (a->k.scale_kind == DSA_SCALE_E8M0 && a->k.group == 32)))
            return DSA_ERR_UNSUPPORTED;
        if (a->k.scales == nullptr || (b->batch > 0 && a->q_scale == nullptr)) return DSA_ERR_NULL;
        // queries in 16-byte pieces; head weights and a head's scale (fp32, or its four E8M0 bytes) in 4
        if ((uintptr_t)a->q % 16 != 0 || ((uintptr_t)a->head_w | (uintptr_t)a->q_scale) % 4 != 0)
            return DSA_ERR_SHAPE;
        if (a->k.scale_kind == DSA_SCALE_E8M0) {  // a position's four E8M0 bytes are read as one dword
            const dsa::PoolLayout L = layout_of(&a->k);
            if ((uintptr_t)a->k.scales % 4 != 0 || L.srs % 4 != 0 || L.sbs % 4 != 0) return DSA_ERR_SHAPE;
        }
        return DSA_OK;
    default:
        return DSA_ERR_UNSUPPORTED;
    }
}

dsa_status check_attn(const dsa_batch* b, const dsa_attn_args* a) {
    if (a == nullptr) return DSA_ERR_NULL;
    if (b->batch > 0 && (a->q == nullptr || a->out == nullptr)) return DSA_ERR_NULL;
    dsa_status s = check_pool(&a->kv, a->kv.width);
    if (s != DSA_OK) return s;
    if (!(a->sm_scale > 0.f) || a->sm_scale > 3.0e38f) return DSA_ERR_SHAPE;  // finite and positive
    if (a->dtype == DSA_F32) {
        if (a->n_heads < 1 || a->n_heads > 16 || a->kv.width < 1 || a->kv.width > 128) return DSA_ERR_UNSUPPORTED;
        if (a->d_v < 1 || a->d_v > a->kv.width) return DSA_ERR_SHAPE;
        if (a->kv.dtype != DSA_F32 || a->kv.scale_kind != DSA_SCALE_NONE) return DSA_ERR_UNSUPPORTED;
        return DSA_OK;
    }
    if (a->dtype != DSA_BF16) return DSA_ERR_UNSUPPORTED;
    if (a->n_heads != 128 || a->kv.width != 576 || a->d_v != 512) return DSA_ERR_UNSUPPORTED;
    if (a->kv.dtype == DSA_BF16 && a->kv.scale_kind == DSA_SCALE_NONE) return DSA_OK;
    if (a->kv.dtype == DSA_E4M3 && ((a->kv.scale_kind == DSA_SCALE_E8M0 && a->kv.group == 32) ||
                                    (a->kv.scale_kind == DSA_SCALE_F32 && a->kv.group == 128)))
        return a->kv.scales == nullptr ? DSA_ERR_NULL : DSA_OK;
    return DSA_ERR_UNSUPPORTED;
}

dsa::IndexerLaunch indexer_launch(const dsa_batch* b, const dsa_indexer_args* a, float* scores, int64_t ld) {
    dsa::IndexerLaunch L{};
    L.dtype = a->dtype == DSA_F32 ? 0 : a->dtype == DSA_BF16 ? 1 : a->k.scale_kind == DSA_SCALE_E8M0 ? 3 : 2;
    L.q = a->q;
    L.q_scale = a->q_scale;
    L.w = a->head_w;
    L.kpool = a->k.data;
    L.kscale = a->k.scales;
    L.kl = layout_of(&a->k);
    L.seq_lens = b->seq_lens;
    L.table = b->block_table;
    L.max_blocks = b->max_blocks;
    L.num_blocks = a->k.num_blocks;
    L.batch = b->batch;
    L.n_q = b->n_q;
    L.max_seq_len = b->max_seq_len;
    L.H = a->n_heads;
    L.D = a->head_dim;
    L.scores = scores;
    L.ld = ld;
    return L;
}

dsa::AttnLaunch attn_launch(const dsa_batch* b, const dsa_attn_args* a, const int32_t* indices, int top_k,
                            float* ws) {
    dsa::AttnLaunch L{};
    L.q_dtype = a->dtype == DSA_F32 ? 0 : 1;
    L.kv_kind = a->kv.dtype == DSA_F32    ? 0
                : a->kv.dtype == DSA_BF16 ? 1
                : a->kv.scale_kind == DSA_SCALE_E8M0 ? 2
                                                      : 3;
    L.q = a->q;
    L.kv = a->kv.data;
    L.kvscale = a->kv.scales;
    L.kvl = layout_of(&a->kv);
    L.seq_lens = b->seq_lens;
    L.table = b->block_table;
    L.max_blocks = b->max_blocks;
    L.num_blocks = a->kv.num_blocks;
    L.batch = b->batch;
    L.n_q = b->n_q;
    L.max_seq_len = b->max_seq_len;
    L.H = a->n_heads;
    L.Dqk = a->kv.width;
    L.Dv = a->d_v;
    L.top_k = top_k;
    L.sm_scale = a->sm_scale;
    L.indices = const_cast<int32_t*>(indices);  // read only unless L.scores is set
    L.out = a->out;
    L.lse = a->lse;
    L.ws = ws;
    L.splits = a->dtype == DSA_F32 ? 1 : dsa::attn_splits(b->batch * b->n_q, top_k, a->kv.width);
    return L;
}

size_t attn_ws(const dsa_batch* b, const dsa_attn_args* a, int top_k) {
    if (a->dtype == DSA_F32) return 0;
    return dsa::attn_ws_bytes(b->batch * b->n_q, top_k, a->kv.width, a->n_heads, a->d_v);
}

int64_t forward_ld(const dsa_batch* b) { return ((int64_t)b->max_seq_len + 63) / 64 * 64; }

dsa_status hip_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

dsa_status forward_impl(const dsa_batch* batch, const dsa_indexer_args* idx, const dsa_attn_args* attn,
                        int32_t top_k, int32_t* indices_out, void* ws, size_t ws_bytes, void* stream);

}  // namespace

extern "C" {

const char* dsa_status_string(dsa_status s) {
    switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_NULL: return "DSA_ERR_NULL: a required pointer is NULL";
    case DSA_ERR_SHAPE: return "DSA_ERR_SHAPE: sizes inconsistent or out of range";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED: no kernel for this shape or dtype";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace missing or too small";
    case DSA_ERR_HIP: return "DSA_ERR_HIP: a HIP call or kernel launch failed";
    default: return "unknown dsa_status";
    }
}

int32_t dsa_version(void) { return 100; }

dsa_status dsa_indexer_scores(const dsa_batch* batch, const dsa_indexer_args* idx, float* scores,
                              int64_t ld_scores, void* stream) {
    dsa_status s = check_batch(batch);
    if (s != DSA_OK) return s;
    if ((s = check_indexer(batch, idx)) != DSA_OK) return s;
    if (batch->batch > 0 && scores == nullptr) return DSA_ERR_NULL;
    if (ld_scores < batch->max_seq_len) return DSA_ERR_SHAPE;
    return hip_status(dsa::launch_indexer(indexer_launch(batch, idx, scores, ld_scores), (hipStream_t)stream));
}

size_t dsa_topk_workspace_bytes(const dsa_batch* batch, int32_t top_k) {
    if (check_batch(batch) != DSA_OK || top_k < 1 || top_k > kMaxTopK) return 0;
    return dsa::topk_ws_bytes(batch->batch * batch->n_q, batch->max_seq_len, top_k);
}

dsa_status dsa_topk(const dsa_batch* batch, const float* scores, int64_t ld_scores, int32_t top_k,
                    int32_t* indices, void* ws, size_t ws_bytes, void* stream) {
    dsa_status s = check_batch(batch);
    if (s != DSA_OK) return s;
    if (top_k < 1 || top_k > kMaxTopK) return DSA_ERR_SHAPE;
    if (batch->batch > 0 && (scores == nullptr || indices == nullptr)) return DSA_ERR_NULL;
    if (ld_scores < batch->max_seq_len) return DSA_ERR_SHAPE;
    const size_t need = dsa::topk_ws_bytes(batch->batch * batch->n_q, batch->max_seq_len, top_k);
    if (need > 0 && (ws == nullptr || ws_bytes < need)) return DSA_ERR_WORKSPACE;
    dsa::TopkLaunch L{scores, ld_scores, batch->seq_lens, batch->batch, batch->n_q, batch->max_seq_len, top_k,
                      indices, (int32_t*)ws};
    return hip_status(dsa::launch_topk(L, (hipStream_t)stream));
}

size_t dsa_sparse_attn_workspace_bytes(const dsa_batch* batch, const dsa_attn_args* attn, int32_t top_k) {
    if (check_batch(batch) != DSA_OK || attn == nullptr || top_k < 1 || top_k > kMaxTopK) return 0;
    return attn_ws(batch, attn, top_k);
}

dsa_status dsa_sparse_attn(const dsa_batch* batch, const dsa_attn_args* attn, const int32_t* indices,
                           int32_t top_k, void* ws, size_t ws_bytes, void* stream) {
    dsa_status s = check_batch(batch);
    if (s != DSA_OK) return s;
    if ((s = check_attn(batch, attn)) != DSA_OK) return s;
    if (top_k < 1 || top_k > kMaxTopK) return DSA_ERR_SHAPE;
    if (batch->batch > 0 && indices == nullptr) return DSA_ERR_NULL;
    const size_t need = attn_ws(batch, attn, top_k);
    if (need > 0 && (ws == nullptr || ws_bytes < need)) return DSA_ERR_WORKSPACE;
    return hip_status(
        dsa::launch_sparse_attn(attn_launch(batch, attn, indices, top_k, (float*)ws), (hipStream_t)stream));
}

size_t dsa_forward_workspace_bytes(const dsa_batch* batch, const dsa_indexer_args* idx, const dsa_attn_args* attn,
                                   int32_t top_k) {
    if (check_batch(batch) != DSA_OK || idx == nullptr || attn == nullptr || top_k < 1 || top_k > kMaxTopK) return 0;
    const size_t rows = (size_t)batch->batch * batch->n_q;
    return align_up(sizeof(float) * rows * (size_t)forward_ld(batch)) + align_up(sizeof(int32_t) * rows * top_k) +
           align_up(attn_ws(batch, attn, top_k)) +
           align_up(dsa::topk_ws_bytes((int)rows, batch->max_seq_len, top_k));
}

dsa_status dsa_forward(const dsa_batch* batch, const dsa_indexer_args* idx, const dsa_attn_args* attn,
                       int32_t top_k, int32_t* indices_out, void* ws, size_t ws_bytes, void* stream) {
    return forward_impl(batch, idx, attn, top_k, indices_out, ws, ws_bytes, stream);
}

dsa_status dsa_forward_noalloc(const dsa_batch* batch, const dsa_indexer_args* idx, const dsa_attn_args* attn,
                               int32_t top_k, int32_t* indices_out, void* stream) {
    dsa_status s = check_batch(batch);
    if (s != DSA_OK) return s;
    if ((s = check_indexer(batch, idx)) != DSA_OK) return s;
    if ((s = check_attn(batch, attn)) != DSA_OK) return s;
    if (top_k < 1 || top_k > kMaxTopK) return DSA_ERR_SHAPE;
    if (dsa_forward_workspace_bytes(batch, idx, attn, top_k) > dsa::kScratchBytes) return DSA_ERR_WORKSPACE;
    void* ws = nullptr;
    if (dsa::scratch_for_current_device(&ws) != hipSuccess) return DSA_ERR_HIP;
    return forward_impl(batch, idx, attn, top_k, indices_out, ws, dsa::kScratchBytes, stream);
}

size_t dsa_forward_noalloc_max_bytes(void) { return dsa::kScratchBytes; }

}  // extern "C"

namespace {

dsa_status forward_impl(const dsa_batch* batch, const dsa_indexer_args* idx, const dsa_attn_args* attn,
                        int32_t top_k, int32_t* indices_out, void* ws, size_t ws_bytes, void* stream) {
    dsa_status s = check_batch(batch);
    if (s != DSA_OK) return s;
    if ((s = check_indexer(batch, idx)) != DSA_OK) return s;
    if ((s = check_attn(batch, attn)) != DSA_OK) return s;
    if (top_k < 1 || top_k > kMaxTopK) return DSA_ERR_SHAPE;
    const size_t need = dsa_forward_workspace_bytes(batch, idx, attn, top_k);
    if (ws == nullptr || ws_bytes < need) return DSA_ERR_WORKSPACE;
    const size_t rows = (size_t)batch->batch * batch->n_q;
    const int64_t ld = forward_ld(batch);
    char* p = (char*)ws;
    float* scores = (float*)p;
    p += align_up(sizeof(float) * rows * (size_t)ld);
    int32_t* idx_ws = (int32_t*)p;
    p += align_up(sizeof(int32_t) * rows * top_k);
    float* attn_ws_p = (float*)p;
    p += align_up(attn_ws(batch, attn, top_k));
    int32_t* topk_ws = (int32_t*)p;
    int32_t* indices = indices_out != nullptr ? indices_out : idx_ws;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = dsa::launch_indexer(indexer_launch(batch, idx, scores, ld), st);
    if (e != hipSuccess) return DSA_ERR_HIP;
    dsa::AttnLaunch A = attn_launch(batch, attn, indices, top_k, attn_ws_p);
    if (dsa::attn_fuses_topk(A)) {
        // each attention workgroup selects its row's Top-K from the scores and
        // writes the indices itself: one launch fewer, the same indices
        A.scores = scores;
        A.ld = ld;
        return hip_status(dsa::launch_sparse_attn(A, st));
    }
    dsa::TopkLaunch T{scores, ld, batch->seq_lens, batch->batch, batch->n_q, batch->max_seq_len, top_k, indices,
                      topk_ws};
    if ((e = dsa::launch_topk(T, st)) != hipSuccess) return DSA_ERR_HIP;
    return hip_status(dsa::launch_sparse_attn(A, st));
}

}  // namespace

extern "C" {

dsa_status dsa_cache_append(const dsa_batch* batch, const void* k_new, const void* kv_new, dsa_dtype new_dtype,
                            const dsa_cache* k, const dsa_cache* kv, void* stream) {
    dsa_status s = check_batch(batch);
    if (s != DSA_OK) return s;
    if (k == nullptr || kv == nullptr) return DSA_ERR_NULL;
    // pool format -> kernel kind (0 fp32, 1 bf16, 2 e4m3 + fp32 scale, 3 e4m3 + E8M0 scale), or -1
    auto kind_of = [&](const dsa_cache* c) -> int {
        if (c->dtype == DSA_F32 && c->scale_kind == DSA_SCALE_NONE) return new_dtype == DSA_F32 ? 0 : -1;
        if (new_dtype != DSA_BF16) return -1;
        if (c->dtype == DSA_BF16 && c->scale_kind == DSA_SCALE_NONE) return 1;
        if (c->dtype != DSA_E4M3) return -1;
        // groups are whole aligned lane groups of one wave: powers of two from 4 to 256
        if (c->scale_kind == DSA_SCALE_F32 && c->group >= 4 && c->group <= 256 && (c->group & (c->group - 1)) == 0)
            return 2;
        if (c->scale_kind == DSA_SCALE_E8M0 && c->group == 32) return 3;
        return -1;
    };
    const int kk = kind_of(k), kvk = kind_of(kv);
    if (kk < 0 || kvk < 0) return DSA_ERR_UNSUPPORTED;
    if (k->width < 4 || k->width % 4 != 0 || k->width > 256 || kv->width < 4 || kv->width % 4 != 0 ||
        kv->width > 768 || k->num_blocks < 1 || kv->num_blocks < 1)
        return DSA_ERR_SHAPE;
    if (k->num_blocks * 64 > (int64_t)INT_MAX || kv->num_blocks * 64 > (int64_t)INT_MAX) return DSA_ERR_UNSUPPORTED;
    if (batch->batch > 0 && (k_new == nullptr || kv_new == nullptr)) return DSA_ERR_NULL;
    if (k->data == nullptr || kv->data == nullptr) return DSA_ERR_NULL;
    if ((kk >= 2 && k->scales == nullptr) || (kvk >= 2 && kv->scales == nullptr)) return DSA_ERR_NULL;
    dsa::AppendLaunch L{};
    if ((s = pool_layout(k, &L.k_l)) != DSA_OK || (s = pool_layout(kv, &L.kv_l)) != DSA_OK) return s;
    // fp32 rows are written 16 bytes at a time
    for (const dsa_cache* c : {k, kv}) {
        const dsa::PoolLayout& Lc = c == k ? L.k_l : L.kv_l;
        if (c->dtype == DSA_F32 && ((uintptr_t)c->data % 16 != 0 || Lc.rs % 16 != 0 || Lc.bs % 16 != 0))
            return DSA_ERR_SHAPE;
    }
    L.in_f32 = new_dtype == DSA_F32;
    L.k_new = k_new;
    L.kv_new = kv_new;
    L.seq_lens = batch->seq_lens;
    L.table = batch->block_table;
    L.max_blocks = batch->max_blocks;
    L.batch = batch->batch;
    L.n_q = batch->n_q;
    L.max_seq_len = batch->max_seq_len;
    L.k_width = k->width;
    L.k_kind = kk;
    L.k_group = kk >= 2 ? k->group : 0;
    L.k_blocks = k->num_blocks;
    L.k_pool = const_cast<void*>(k->data);
    L.k_scales = const_cast<void*>(k->scales);
    L.kv_width = kv->width;
    L.kv_kind = kvk;
    L.kv_group = kvk >= 2 ? kv->group : 0;
    L.kv_blocks = kv->num_blocks;
    L.kv_pool = const_cast<void*>(kv->data);
    L.kv_scales = const_cast<void*>(kv->scales);
    return hip_status(dsa::launch_cache_append(L, (hipStream_t)stream));
}

dsa_status dsa_indexer_prolog(const dsa_prolog_args* p, void* stream) {
    if (p == nullptr) return DSA_ERR_NULL;
    if (p->rows < 0 || p->d_x < kPrologChunk || p->d_x % kPrologChunk != 0 || p->n_heads < 1 || p->head_dim < 32 ||
        p->head_dim % 32 != 0 || p->head_dim > 256 || !(p->eps >= 0.f) || p->eps > 3.0e38f)
        return DSA_ERR_SHAPE;
    // row tiles of up to 64 rows form the grid's second dimension (at most 65535)
    if ((int64_t)p->n_heads * p->head_dim > (int64_t)INT_MAX / 2 || p->rows > 65535 * 64) return DSA_ERR_SHAPE;
    if (p->q_dtype != DSA_BF16 && p->q_dtype != DSA_E4M3) return DSA_ERR_UNSUPPORTED;
    if (p->rows == 0) return DSA_OK;
    if (p->x == nullptr || p->w_q == nullptr || p->w_h == nullptr || p->k == nullptr || p->k_gain == nullptr ||
        p->q_out == nullptr || p->head_w_out == nullptr || p->k_out == nullptr ||
        (p->q_dtype == DSA_E4M3 && p->q_scale_out == nullptr))
        return DSA_ERR_NULL;
    // the projections' operands are read 16 bytes at a time; q is stored up to 8 bytes at a time
    if (((uintptr_t)p->x | (uintptr_t)p->w_q | (uintptr_t)p->w_h) % 16 != 0 || (uintptr_t)p->q_out % 8 != 0 ||
        ((uintptr_t)p->head_w_out | (uintptr_t)p->k_gain) % 4 != 0 || ((uintptr_t)p->k | (uintptr_t)p->k_out) % 2 != 0)
        return DSA_ERR_SHAPE;
    dsa::PrologLaunch L{};
    L.x = static_cast<const uint16_t*>(p->x);
    L.w_q = static_cast<const uint16_t*>(p->w_q);
    L.w_h = static_cast<const uint16_t*>(p->w_h);
    L.k = static_cast<const uint16_t*>(p->k);
    L.gain = p->k_gain;
    L.eps = p->eps;
    L.rows = p->rows;
    L.d_x = p->d_x;
    L.H_I = p->n_heads;
    L.d_I = p->head_dim;
    L.q_mx = p->q_dtype == DSA_E4M3;
    L.q_out = p->q_out;
    L.q_scale = static_cast<uint8_t*>(p->q_scale_out);
    L.head_w = p->head_w_out;
    L.k_norm = static_cast<uint16_t*>(p->k_out);
    return hip_status(dsa::launch_indexer_prolog(L, (hipStream_t)stream));
}

}  // extern "C"
