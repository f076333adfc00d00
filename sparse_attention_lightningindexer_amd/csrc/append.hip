// append.hip -- cache append with fused dynamic quantization for gfx950.
//
// Each decode step produces, per query token, one index key (d_I values) and
// one latent KV row (d_qk values).  They are written into the paged pools at
// the token's position, quantized on the way when the pool is quantized: the
// pages compute the scales inside the operator that produces the cache entry
// ("Day0 Inference Adaptation and Performance Optimization for a New
// Architecture Domestic Large Language Model on Ascend", §5 Layered
// Quantization: dynamic quantization; "Day0 Inference Adaptation and
// Performance Optimization for New-Architecture LLMs", §4.2).
//
// Formats of a pool (per group of G elements, a shorter last group when G
// does not divide the width), decided in fp32:
//   fp32 scale:  scale = amax/448 (1 when amax = 0), code = e4m3(x/scale)
//   E8M0 scale:  e = floor(log2 amax) - 8 (-127 when amax = 0), clamped to
//                [-127, 127], code = e4m3(x * 2^-e), byte e + 127
// The quotient is clamped to +-448 and rounded to the nearest e4m3 (ties to
// even) by the hardware conversion.  bf16 and fp32 pools are plain copies of
// their input, bit for bit (NaN payloads included).
//
// One workgroup of 256 threads per token: threads 0..63 take the index key,
// threads 64..255 the latent row, four values per thread, so a group of G
// values is G/4 consecutive lanes of one wave and its amax is a lane
// reduction.
#include "common.hpp"
#include "kernels.hpp"

namespace dsa {

namespace {

constexpr int kAppendThreads = 256;
constexpr int kKeyThreads = 64;  // the index key's threads (width <= 256)

__device__ __forceinline__ float lane_max(float v, int lanes) {  // over aligned groups of `lanes`
    for (int m = 1; m < lanes; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
    return v;
}

// e4m3 codes of four floats (already within +-448), nearest-even, packed.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -448.f), 448.f); }

// Writes this thread's four values x[0..3] (elements 4t .. 4t+3 of a width-wide
// vector) into pool row `prow`.  kind: 0 fp32 copy, 1 bf16 copy (of the input
// codes `raw`, not of x), 2 e4m3 with an fp32 scale per `group`, 3 e4m3 with
// an E8M0 scale per `group`.  Every lane of the wave calls this (the
// reductions are wave-wide); `active` says whether the thread holds values.
__device__ __forceinline__ void store_vector(const float (&x)[4], uint2 raw, bool active, int t, int width,
                                             int kind, int group, void* pool_row, void* scale_row) {
    if (kind == 0) {
        if (active)
            *reinterpret_cast<float4*>(static_cast<float*>(pool_row) + 4 * t) =
                make_float4(x[0], x[1], x[2], x[3]);
        return;
    }
    if (kind == 1) {
        if (active) *reinterpret_cast<uint2*>(static_cast<uint16_t*>(pool_row) + 4 * t) = raw;
        return;
    }
    float a = active ? fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3]))) : 0.f;
    a = lane_max(a, group / 4);
    const int gidx = (4 * t) / group;
    const bool first = active && (4 * t) % group == 0;
    uint32_t codes;
    if (kind == 2) {
        const float scale = a > 0.f ? a / 448.f : 1.f;
        codes = e4m3x4(clamp448(x[0] / scale), clamp448(x[1] / scale), clamp448(x[2] / scale),
                       clamp448(x[3] / scale));
        if (first) static_cast<float*>(scale_row)[gidx] = scale;
    } else {
        int e2 = 0;
        (void)frexpf(a, &e2);
        int e = a > 0.f ? e2 - 1 - 8 : -127;
        e = min(max(e, -127), 127);
        codes = e4m3x4(clamp448(ldexpf(x[0], -e)), clamp448(ldexpf(x[1], -e)), clamp448(ldexpf(x[2], -e)),
                       clamp448(ldexpf(x[3], -e)));
        if (first) static_cast<uint8_t*>(scale_row)[gidx] = (uint8_t)(e + 127);
    }
    if (active) *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(pool_row) + 4 * t) = codes;
}

template <class In>
__global__ __launch_bounds__(kAppendThreads) void cache_append_kernel(
    const In* __restrict__ k_new, const In* __restrict__ kv_new, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ table, int max_blocks, int n_q, int max_seq_len, int k_width, int k_kind,
    int k_group, int64_t k_blocks, PoolLayout k_l, void* k_pool, void* k_scales, int kv_width, int kv_kind,
    int kv_group, int64_t kv_blocks, PoolLayout kv_l, void* kv_pool, void* kv_scales) {
    const int r = blockIdx.x, b = r / n_q, i = r % n_q;
    const int s = clamp_len(seq_lens, b, max_seq_len) - n_q + i;  // this token's position
    if (s < 0) return;  // block-uniform
    const bool key = threadIdx.x < kKeyThreads;
    const int t = key ? threadIdx.x : threadIdx.x - kKeyThreads;
    const int width = key ? k_width : kv_width;
    const bool active = 4 * t < width;
    const int64_t pb = phys_block(table, max_blocks, b, s / kBlock, key ? k_blocks : kv_blocks);
    if (pb < 0) return;  // absent block: nothing is written (uniform per pool, hence per wave)
    const PoolLayout& Lp = key ? k_l : kv_l;
    const int64_t roff = pb * Lp.bs + (s % kBlock) * Lp.rs;    // this token's row, in bytes
    const int64_t soff = pb * Lp.sbs + (s % kBlock) * Lp.srs;  // and its scales
    float x[4] = {0.f, 0.f, 0.f, 0.f};
    uint2 raw = make_uint2(0u, 0u);  // bf16 input codes, stored as they are into a bf16 pool
    if (active) {
        const In* src = (key ? k_new + (int64_t)r * k_width : kv_new + (int64_t)r * kv_width) + 4 * t;
        if constexpr (sizeof(In) == 2) {
            const uint2 v = *reinterpret_cast<const uint2*>(src);
            raw = v;
            x[0] = bf16_bits_to_f32((uint16_t)(v.x & 0xffffu));
            x[1] = bf16_bits_to_f32((uint16_t)(v.x >> 16));
            x[2] = bf16_bits_to_f32((uint16_t)(v.y & 0xffffu));
            x[3] = bf16_bits_to_f32((uint16_t)(v.y >> 16));
        } else {
            const float4 v = *reinterpret_cast<const float4*>(src);
            x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
        }
    }
    if (key)
        store_vector(x, raw, active, t, k_width, k_kind, k_group, static_cast<uint8_t*>(k_pool) + roff,
                     static_cast<uint8_t*>(k_scales) + soff);
    else
        store_vector(x, raw, active, t, kv_width, kv_kind, kv_group, static_cast<uint8_t*>(kv_pool) + roff,
                     static_cast<uint8_t*>(kv_scales) + soff);
}

}  // namespace

hipError_t launch_cache_append(const AppendLaunch& a, hipStream_t st) {
    const int rows = a.batch * a.n_q;
    if (rows == 0) return hipSuccess;
    if (a.in_f32)
        hipLaunchKernelGGL(cache_append_kernel<float>, dim3(rows), dim3(kAppendThreads), 0, st,
                           (const float*)a.k_new, (const float*)a.kv_new, a.seq_lens, a.table, a.max_blocks,
                           a.n_q, a.max_seq_len, a.k_width, a.k_kind, a.k_group, a.k_blocks, a.k_l, a.k_pool,
                           a.k_scales, a.kv_width, a.kv_kind, a.kv_group, a.kv_blocks, a.kv_l, a.kv_pool,
                           a.kv_scales);
    else
        hipLaunchKernelGGL(cache_append_kernel<uint16_t>, dim3(rows), dim3(kAppendThreads), 0, st,
                           (const uint16_t*)a.k_new, (const uint16_t*)a.kv_new, a.seq_lens, a.table,
                           a.max_blocks, a.n_q, a.max_seq_len, a.k_width, a.k_kind, a.k_group, a.k_blocks,
                           a.k_l, a.k_pool, a.k_scales, a.kv_width, a.kv_kind, a.kv_group, a.kv_blocks, a.kv_l,
                           a.kv_pool, a.kv_scales);
    return hipGetLastError();
}

}  // namespace dsa
