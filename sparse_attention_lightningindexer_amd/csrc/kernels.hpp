// kernels.hpp -- host-side launch descriptors of the gfx950 kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

constexpr int kTopkCacheMax = 16384;      // rows up to this length keep their keys in LDS
constexpr int kAttnMaxSplits = 32;        // split partials merged per row
constexpr int kAttnMaxSplitSlots = 2048;  // index slots one attention workgroup compacts

// A pool's layout in bytes: row (position o of block p) at p*bs + o*rs, its
// scales at p*sbs + o*srs.
struct PoolLayout {
    int64_t bs, rs, sbs, srs;
};

struct IndexerLaunch {
    int dtype;                 // 0 f32, 1 bf16, 2 e4m3 + fp32 per 128, 3 MXFP8 (e4m3 + e8m0 per 32)
    const void* q;
    const void* q_scale;       // fp32 [rows][heads] (2) or e8m0 [rows][heads][4] (3)
    const float* w;
    const void* kpool;
    const void* kscale;        // fp32 [pool rows] (2) or e8m0 [pool rows][4] (3)
    PoolLayout kl;             // index-K pool layout
    const int32_t* seq_lens;
    const int32_t* table;
    int max_blocks;
    int64_t num_blocks;
    int batch, n_q, max_seq_len, H, D;
    float* scores;
    int64_t ld;
};

struct TopkLaunch {
    const float* scores;
    int64_t ld;
    const int32_t* seq_lens;
    int batch, n_q, max_seq_len, top_k;
    int32_t* indices;
    int32_t* ws;               // segment candidates for long rows, topk_ws_bytes
};

struct AttnLaunch {
    int q_dtype;               // 0 f32, 1 bf16
    int kv_kind;               // 0 f32, 1 bf16, 2 MXFP8 (e4m3 + e8m0 per 32), 3 e4m3 + fp32 per 128
    const void* q;
    const void* kv;
    const void* kvscale;       // e8m0 [pool rows][18] (2) or fp32 [pool rows][5] (3)
    PoolLayout kvl;            // latent pool layout
    const int32_t* seq_lens;
    const int32_t* table;
    int max_blocks;
    int64_t num_blocks;
    int batch, n_q, max_seq_len, H, Dqk, Dv, top_k;
    float sm_scale;
    int32_t* indices;          // the index lists; written instead when scores is set
    void* out;
    float* lse;
    void* ws;                  // split partials, attn_ws_bytes
    int splits;
    const float* scores = nullptr;  // set: select each row's Top-K from these (attn_fuses_topk)
    int64_t ld = 0;
};

struct AppendLaunch {
    bool in_f32;               // new values in fp32 (else bf16)
    const void* k_new;         // [rows][k_width]
    const void* kv_new;        // [rows][kv_width]
    const int32_t* seq_lens;
    const int32_t* table;
    int max_blocks, batch, n_q, max_seq_len;
    int k_width, k_kind, k_group;     // kind: 0 fp32, 1 bf16, 2 e4m3 + fp32 scale, 3 e4m3 + E8M0 scale
    int64_t k_blocks;
    PoolLayout k_l;
    void* k_pool;
    void* k_scales;
    int kv_width, kv_kind, kv_group;
    int64_t kv_blocks;
    PoolLayout kv_l;
    void* kv_pool;
    void* kv_scales;
};

struct PrologLaunch {
    const uint16_t* x;         // bf16 [rows][d_x]
    const uint16_t* w_q;       // bf16 [H_I*d_I][d_x]
    const uint16_t* w_h;       // bf16 [H_I][d_x]
    const uint16_t* k;         // bf16 [rows][d_I]
    const float* gain;         // fp32 [d_I]
    float eps;
    int rows, d_x, H_I, d_I;
    bool q_mx;                 // q as e4m3 + E8M0 per 32 (else bf16)
    void* q_out;               // [rows][H_I*d_I]
    uint8_t* q_scale;          // [rows][H_I*d_I/32] when q_mx
    float* head_w;             // [rows][H_I]
    uint16_t* k_norm;          // bf16 [rows][d_I]
};

// The no-allocation entry point's device workspace: a file-scope array of
// this many bytes per GPU (scratch.hip); its device address for the current
// device, looked up once per device.
constexpr size_t kScratchBytes = size_t(32) << 20;
hipError_t scratch_for_current_device(void** ptr);
// Compute units of the current device (asked of the runtime once per device).
hipError_t compute_units(int* cus);

hipError_t launch_indexer(const IndexerLaunch& a, hipStream_t st);
hipError_t launch_indexer_prolog(const PrologLaunch& a, hipStream_t st);
hipError_t launch_cache_append(const AppendLaunch& a, hipStream_t st);
hipError_t launch_topk(const TopkLaunch& a, hipStream_t st);
hipError_t launch_sparse_attn(const AttnLaunch& a, hipStream_t st);
bool attn_fuses_topk(const AttnLaunch& a);

int attn_splits(int rows, int top_k, int Dqk);
size_t topk_ws_bytes(int rows, int max_seq_len, int top_k);
size_t attn_ws_bytes(int rows, int top_k, int Dqk, int H, int Dv);

}  // namespace dsa
