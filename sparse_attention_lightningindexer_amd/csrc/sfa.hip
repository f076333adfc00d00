// sfa.hip -- Sparse Flash Attention over the MLA latent cache for gfx950.
//
// For each query row, attention over only the positions the indexer kept,
// read from the paged latent KV cache ("Day0 Inference Adaptation and
// Performance Optimization for a New Architecture Domestic Large Language
// Model on Ascend", §2 Sparse Attention and §4 Sparse attention read), in the
// chunked, IO-aware form the pages describe ("Day0 Inference Adaptation and
// Performance Optimization for New-Architecture LLMs", §2.2 and §4.1).  One
// latent row [latent 512 | rope 64] per position is shared by all 128 heads:
// K is the whole row, V its first 512 channels.
//
// Kernel structure (128 heads, d_qk 576, d_v 512), one workgroup of 8 waves
// per (row, split of the index list):
//   0. the split's index slots are validated (0 <= s < L_r, block present)
//      and compacted in order into LDS as pool-row numbers;
//   1. per chunk of 32 positions the latent rows are gathered straight into
//      LDS (global_load_lds, double-buffered, 16-byte units XOR-swizzled by
//      row so the MFMA operand reads are bank-conflict free).  An MXFP8 cache
//      is dequantized (e4m3 * 2^(e8m0-127), exact in bf16) on the way in;
//   2. wave w owns heads 16w..16w+15: S^T = K . Q^T on MFMA with Q held in
//      registers for the whole kernel;
//   3. online softmax in the log2 domain, per head, in registers; the
//      running maximum is only moved when it grows by more than 2^8, which
//      changes rounding only (numerator and denominator share it);
//   4. O^T += V^T . P^T on MFMA: P is already laid out as the B operand, and
//      V^T comes from LDS with the transposing read ds_read_b64_tr_b16;
//   5. the row's result (or the split's normalized partial and its LSE) is
//      written; a combine kernel merges the splits by LSE.
#include "common.hpp"
#include "kernels.hpp"

namespace dsa {

constexpr int kH = 128, kDqk = 576, kDv = 512, kCh = 32;
constexpr int kRowB = kDqk * 2;        // bytes per bf16 latent row
constexpr int kUnits = kRowB / 16;     // 16-byte units per row (72)
constexpr int kTileB = kCh * kRowB;    // 36864 bytes per chunk
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescale = 8.0f;       // move the running max when it grows by > 2^8

// LDS byte offset of 16-byte unit u of tile row `row`.
__device__ __forceinline__ int lds_unit(int row, int u) { return row * kRowB + ((u ^ (row & 7)) << 4); }

// E8M0 byte -> fp32 2^(b-127) (b = 0 gives the subnormal 2^-127; 255 is NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
    if (b == 0u) return __uint_as_float(0x00400000u);
    if (b == 255u) return __uint_as_float(0x7fc00000u);
    return __uint_as_float(b << 23);
}

// 16 e4m3 codes (one 16-byte unit) times a power-of-two scale -> 16 bf16 (exact).
__device__ __forceinline__ void dequant_unit(i32x4 codes, float scale, i32x4& lo, i32x4& hi) {
    uint32_t packed[8];
    for (int w = 0; w < 4; ++w) {
        const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(codes[w], false);
        const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(codes[w], true);
        const uint32_t b0 = __float_as_uint(a[0] * scale) >> 16, b1 = __float_as_uint(a[1] * scale) >> 16;
        const uint32_t b2 = __float_as_uint(c[0] * scale) >> 16, b3 = __float_as_uint(c[1] * scale) >> 16;
        packed[2 * w] = b0 | (b1 << 16);
        packed[2 * w + 1] = b2 | (b3 << 16);
    }
    lo = i32x4{(int)packed[0], (int)packed[1], (int)packed[2], (int)packed[3]};
    hi = i32x4{(int)packed[4], (int)packed[5], (int)packed[6], (int)packed[7]};
}

template <bool MX>
__global__ __launch_bounds__(512, 1) void sfa_mla_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv, const uint8_t* __restrict__ kvscale,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ table, int max_blocks,
    int64_t num_blocks, int n_q, int max_seq_len, int rows, const int32_t* __restrict__ indices,
    int top_k, int per_split, int splits, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ ws_o, float* __restrict__ ws_lse) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[2][kTileB];
    __shared__ __attribute__((aligned(16))) uint8_t stage[MX ? kCh * kDqk : 16];  // fp8 codes of the next chunk
    __shared__ int32_t prow[kAttnMaxSplitSlots];
    __shared__ int wave_cnt[8];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, j = lane & 15;

    // work item: with splits, the splits of one row share an XCD (ids equal mod 8)
    int row, split;
    if (splits == 1) {
        row = rows - 1 - (int)blockIdx.x;  // longest histories first in prefill
        split = 0;
    } else {
        const int x = blockIdx.x & 7, jj = blockIdx.x >> 3;
        row = (jj / splits) * 8 + x;
        split = jj % splits;
    }
    if (row >= rows) return;  // padding of the XCD-aware grid (block-uniform)
    const int b = row / n_q, qi = row % n_q;
    const int L = history_len(clamp_len(seq_lens, b, max_seq_len), n_q, qi);
    const int slot0 = split * per_split;
    const int slot1 = min(top_k, slot0 + per_split);

    // 0. ordered compaction of the valid index slots into pool-row numbers
    int n_valid = 0;
    for (int base = slot0; base < slot1; base += 512) {
        const int t = base + tid;
        const int s = t < slot1 ? indices[(int64_t)row * top_k + t] : -1;
        int pr = -1;
        if (s >= 0 && s < L) {
            const int64_t p = phys_block(table, max_blocks, b, s / kBlock, num_blocks);
            if (p >= 0) pr = (int)(p * kBlock + (s % kBlock));
        }
        const uint64_t m = ballot(pr >= 0);
        if (lane == 0) wave_cnt[wave] = __popcll(m);
        __syncthreads();
        int before = 0, tot = 0;
        for (int w = 0; w < 8; ++w) {
            before += w < wave ? wave_cnt[w] : 0;
            tot += wave_cnt[w];
        }
        if (pr >= 0) prow[n_valid + before + lanes_below(m)] = pr;
        n_valid += tot;
        __syncthreads();
    }
    const int nchunks = (n_valid + kCh - 1) / kCh;

    // Q^T fragments of this wave's 16 heads: lane holds q[h0 + j][32ks + 8g .. +8]
    const int h0 = 16 * wave;
    bf16x8 qf[kDqk / 32];
    {
        const uint16_t* qrow = q + ((int64_t)row * kH + h0 + j) * kDqk + 8 * g;
        for (int ks = 0; ks < kDqk / 32; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
    }

    f32x4 o[kDv / 16];
    for (int t = 0; t < kDv / 16; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    // 1. chunk gather.  bf16: 36 wave-instructions of 64 x 16 B straight into LDS.
    //    MXFP8: the codes (18 wave-instructions) go straight into a staging area,
    //    the E8M0 scales of the thread's three units into registers; after the
    //    chunk's compute they are dequantized into the bf16 tile.
    constexpr int kMxUnits = kCh * (kDqk / 16);   // 1152 code units per chunk
    constexpr int kMxPer = (kMxUnits + 511) / 512; // 3 per thread
    auto chunk_row = [&](int c, int r_) -> int {  // pool row of chunk row r_ (tail rows repeat a valid one)
        const int t = c * kCh + r_;
        return prow[t < n_valid ? t : c * kCh];
    };
    auto issue_gather = [&](int c, int buf) {
        if constexpr (!MX) {
            for (int k = wave; k < kTileB / (16 * kWave); k += 8) {
                const int U = k * kWave + lane;
                const int r_ = U / kUnits, col = (U % kUnits) ^ (r_ & 7);
                const uint8_t* src = kv + (int64_t)chunk_row(c, r_) * kRowB + col * 16;
                __builtin_amdgcn_global_load_lds((const void*)src, (DSA_LDS void*)(&tile[buf][k * kWave * 16]),
                                                 16, 0, 0);
            }
        } else {
            for (int k = wave; k < kMxUnits / kWave; k += 8) {
                const int U = k * kWave + lane;
                const int r_ = U / (kDqk / 16), cu = U % (kDqk / 16);
                const uint8_t* src = kv + (int64_t)chunk_row(c, r_) * kDqk + cu * 16;
                __builtin_amdgcn_global_load_lds((const void*)src, (DSA_LDS void*)(&stage[k * kWave * 16]), 16, 0, 0);
            }
        }
    };
    auto finish_gather = [&](int c, int buf) {  // MXFP8 only: staging -> dequantized bf16 tile
        if constexpr (MX) {
            float sc[kMxPer];
            for (int u = 0; u < kMxPer; ++u) {
                const int U = tid + 512 * u;
                const int r_ = U / (kDqk / 16), cu = U % (kDqk / 16);
                sc[u] = U < kMxUnits ? e8m0_to_f32(kvscale[(int64_t)chunk_row(c, r_) * (kDqk / 32) + cu / 2]) : 0.f;
            }
            __builtin_amdgcn_s_waitcnt(0x0f70);
            __syncthreads();  // staging complete
#pragma unroll 1
            for (int u = 0; u < kMxPer; ++u) {
                const int U = tid + 512 * u;
                if (U < kMxUnits) {
                    const int r_ = U / (kDqk / 16), cu = U % (kDqk / 16);
                    i32x4 lo, hi;
                    dequant_unit(*reinterpret_cast<const i32x4*>(&stage[U * 16]), sc[u], lo, hi);
                    *reinterpret_cast<i32x4*>(&tile[buf][lds_unit(r_, 2 * cu)]) = lo;
                    *reinterpret_cast<i32x4*>(&tile[buf][lds_unit(r_, 2 * cu + 1)]) = hi;
                }
            }
        }
    };

    if (nchunks > 0) {
        issue_gather(0, 0);
        finish_gather(0, 0);
    }
    for (int c = 0; c < nchunks; ++c) {
        const int buf = c & 1;
        __builtin_amdgcn_s_waitcnt(0x0f70);  // this wave's gathers into `buf` have landed
        __syncthreads();
        if (c + 1 < nchunks) issue_gather(c + 1, buf ^ 1);
        const uint8_t* T = tile[buf];

        // 2. S^T = K . Q^T : lane holds S[head j][pos 16mt + 4g + i].  Unit
        //    4ks + g of row r sits at ((4(ks&1) + g) ^ (r&7)) + 8(ks>>1): two lane
        //    offsets per M-tile plus a compile-time displacement.
        f32x4 s[2];
        for (int mt = 0; mt < 2; ++mt) {
            s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int r_ = 16 * mt + j;
            const uint8_t* base0 = T + r_ * kRowB + ((g ^ (r_ & 7)) << 4);
            const uint8_t* base1 = T + r_ * kRowB + (((4 + g) ^ (r_ & 7)) << 4);
#pragma unroll
            for (int ks = 0; ks < kDqk / 32; ++ks) {
                const uint8_t* p_ = ((ks & 1) ? base1 : base0) + 128 * (ks >> 1);
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(p_);
                s[mt] = mfma_bf16(a, qf[ks], s[mt]);
            }
        }

        // 3. online softmax for head h0 + j over this chunk's 32 positions
        float t[8];
        float cmax = -INFINITY;
        for (int mt = 0; mt < 2; ++mt)
            for (int i = 0; i < 4; ++i) {
                const bool ok = c * kCh + 16 * mt + 4 * g + i < n_valid;
                const float v = ok ? s[mt][i] * scale_log2 : -INFINITY;
                t[4 * mt + i] = v;
                cmax = fmaxf(cmax, v);
            }
        cmax = max_over_groups(cmax);
        float alpha = 1.f;
        if (cmax > m_run + kRescale || (m_run == -INFINITY && cmax > -INFINITY)) {
            alpha = m_run == -INFINITY ? 0.f : exp2f(m_run - cmax);
            m_run = cmax;
        }
        uint16_t pb[8];
        float psum = 0.f;
        for (int e = 0; e < 8; ++e) {
            const float p = t[e] == -INFINITY ? 0.f : exp2f(t[e] - m_run);
            pb[e] = f32_to_bf16_bits(p);   // P operand of the PV product
            psum += p;                     // the denominator (and lse) keep fp32 p
        }
        l_run = l_run * alpha + sum_over_groups(psum);
        if (ballot(alpha != 1.f) != 0ull) {
            for (int d = 0; d < kDv / 16; ++d)
                for (int i = 0; i < 4; ++i) o[d][i] *= alpha;
        }
        bf16x8 pf;
        {
            uint32_t w4[4] = {pb[0] | ((uint32_t)pb[1] << 16), pb[2] | ((uint32_t)pb[3] << 16),
                              pb[4] | ((uint32_t)pb[5] << 16), pb[6] | ((uint32_t)pb[7] << 16)};
            pf = *reinterpret_cast<const bf16x8*>(w4);
        }

        // 4. O^T += V^T . P^T; V^T fragment via two transposing LDS reads:
        //    lane j of group g addresses row 16h + 4g + j/4, channels 16d + 4(j%4),
        //    i.e. unit 2d + (j%4)/2: four lane offsets (d mod 4) per row plus a
        //    compile-time displacement of 128 bytes per 4 d.
        {
            const int e_ = j >> 2, q4 = j & 3;
            const int r0 = 4 * g + e_, r1 = 16 + 4 * g + e_;
            const int byte = (q4 & 1) * 8;
            const uint8_t* b0[4];
            const uint8_t* b1[4];
            for (int dd = 0; dd < 4; ++dd) {
                const int u = 2 * dd + (q4 >> 1);
                b0[dd] = T + r0 * kRowB + ((u ^ (r0 & 7)) << 4) + byte;
                b1[dd] = T + r1 * kRowB + ((u ^ (r1 & 7)) << 4) + byte;
            }
#pragma unroll
            for (int d = 0; d < kDv / 16; ++d) {
                const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (DSA_LDS v4i16*)(b0[d & 3] + 128 * (d >> 2)));
                const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (DSA_LDS v4i16*)(b1[d & 3] + 128 * (d >> 2)));
                const v4i16 both[2] = {lo, hi};
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(both);
                o[d] = mfma_bf16(a, pf, o[d]);
            }
        }
        // buf^1 was last read in chunk c-1, before this iteration's barrier; the
        // staging area is refilled only after the next barrier
        if (MX && c + 1 < nchunks) finish_gather(c + 1, buf ^ 1);
    }

    // 5. results: lane holds O^T[16d + 4g + i][head h0 + j]
    const float inv_l = l_run > 0.f ? 1.f / l_run : 0.f;
    const float row_lse = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
    const int h = h0 + j;
    if (splits == 1) {
        uint16_t* orow = out + ((int64_t)row * kH + h) * kDv + 4 * g;
        for (int d = 0; d < kDv / 16; ++d) {
            const uint32_t lo = f32_to_bf16_bits(o[d][0] * inv_l) | ((uint32_t)f32_to_bf16_bits(o[d][1] * inv_l) << 16);
            const uint32_t hi = f32_to_bf16_bits(o[d][2] * inv_l) | ((uint32_t)f32_to_bf16_bits(o[d][3] * inv_l) << 16);
            *reinterpret_cast<uint2*>(orow + 16 * d) = make_uint2(lo, hi);
        }
        if (lse != nullptr && g == 0) lse[(int64_t)row * kH + h] = row_lse;
    } else {
        const int64_t part = (int64_t)row * splits + split;
        float* orow = ws_o + (part * kH + h) * kDv + 4 * g;
        for (int d = 0; d < kDv / 16; ++d)
            *reinterpret_cast<f32x4*>(orow + 16 * d) =
                f32x4{o[d][0] * inv_l, o[d][1] * inv_l, o[d][2] * inv_l, o[d][3] * inv_l};
        if (g == 0) ws_lse[part * kH + h] = row_lse;
    }
}

// Merge split partials: out = sum_s exp(lse_s - LSE) * O_s, LSE = log sum_s exp(lse_s).
// grid (rows, H/4), block 256: wave w -> head 4*blockIdx.y + w, lane -> 8 channels,
// so every load instruction of a wave reads 2 KB of contiguous partials.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void sfa_combine_kernel(const float* __restrict__ ws_o,
                                                          const float* __restrict__ ws_lse, int splits,
                                                          int H, int Dv, void* __restrict__ out,
                                                          float* __restrict__ lse) {
    const int row = blockIdx.x;
    const int h = 4 * blockIdx.y + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (h >= H) return;
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, ws_lse[((int64_t)row * splits + s) * H + h]);
    float W = 0.f;
    for (int s = 0; s < splits; ++s) {
        const float ls = ws_lse[((int64_t)row * splits + s) * H + h];
        W += (M == -INFINITY || ls == -INFINITY) ? 0.f : expf(ls - M);
    }
    const float inv = W > 0.f ? 1.f / W : 0.f;
    for (int d = 8 * lane; d < Dv; d += 8 * 64) {
        f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < splits; ++s) {
            const float ls = ws_lse[((int64_t)row * splits + s) * H + h];
            if (M == -INFINITY || ls == -INFINITY) continue;
            const float wgt = expf(ls - M);
            const float* src = ws_o + (((int64_t)row * splits + s) * H + h) * Dv + d;
            const f32x4 v0 = *reinterpret_cast<const f32x4*>(src);
            const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + 4);
            for (int i = 0; i < 4; ++i) {
                a0[i] = fmaf(wgt, v0[i], a0[i]);
                a1[i] = fmaf(wgt, v1[i], a1[i]);
            }
        }
        if constexpr (OUT_BF16) {
            uint16_t* o = (uint16_t*)out + ((int64_t)row * H + h) * Dv + d;
            uint32_t w4[4];
            for (int i = 0; i < 2; ++i) {
                w4[i] = f32_to_bf16_bits(a0[2 * i] * inv) | ((uint32_t)f32_to_bf16_bits(a0[2 * i + 1] * inv) << 16);
                w4[2 + i] = f32_to_bf16_bits(a1[2 * i] * inv) | ((uint32_t)f32_to_bf16_bits(a1[2 * i + 1] * inv) << 16);
            }
            *reinterpret_cast<uint4*>(o) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
        } else {
            float* o = (float*)out + ((int64_t)row * H + h) * Dv + d;
            *reinterpret_cast<f32x4*>(o) = f32x4{a0[0] * inv, a0[1] * inv, a0[2] * inv, a0[3] * inv};
            *reinterpret_cast<f32x4*>(o + 4) = f32x4{a1[0] * inv, a1[1] * inv, a1[2] * inv, a1[3] * inv};
        }
    }
    if (lse != nullptr && lane == 0) lse[(int64_t)row * H + h] = W > 0.f ? M + logf(W) : -INFINITY;
}

// fp32 attention for small shapes: one wave per (head, row); logits of the
// row's valid positions in LDS, two-pass softmax, lanes over value channels.
__global__ __launch_bounds__(64) void sfa_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kv, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ table, int max_blocks, int64_t num_blocks, int n_q, int max_seq_len,
    const int32_t* __restrict__ indices, int top_k, int H, int Dqk, int Dv, float sm_scale,
    float* __restrict__ out, float* __restrict__ lse) {
    extern __shared__ float sh[];  // [top_k] logits, then [top_k] pool rows (as int)
    float* z = sh;
    int* pr = (int*)(sh + top_k);
    const int h = blockIdx.x, row = blockIdx.y, lane = threadIdx.x;
    const int b = row / n_q, qi = row % n_q;
    const int L = history_len(clamp_len(seq_lens, b, max_seq_len), n_q, qi);
    int n = 0;
    for (int base = 0; base < top_k; base += 64) {
        const int t = base + lane;
        const int s = t < top_k ? indices[(int64_t)row * top_k + t] : -1;
        int p_ = -1;
        if (s >= 0 && s < L) {
            const int64_t p = phys_block(table, max_blocks, b, s / kBlock, num_blocks);
            if (p >= 0) p_ = (int)(p * kBlock + s % kBlock);
        }
        const uint64_t m = ballot(p_ >= 0);
        if (p_ >= 0) pr[n + lanes_below(m)] = p_;
        n += __popcll(m);
    }
    __syncthreads();
    const float* qh = q + ((int64_t)row * H + h) * Dqk;
    float mx = -INFINITY;
    for (int t = lane; t < n; t += 64) {
        const float* k = kv + (int64_t)pr[t] * Dqk;
        float acc = 0.f;
        for (int c = 0; c < Dqk; ++c) acc = fmaf(qh[c], k[c], acc);
        z[t] = acc * sm_scale;
        mx = fmaxf(mx, z[t]);
    }
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    float sum = 0.f;
    for (int t = lane; t < n; t += 64) {
        z[t] = expf(z[t] - mx);
        sum += z[t];
    }
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
    __syncthreads();
    const float inv = n > 0 ? 1.f / sum : 0.f;
    float* oh = out + ((int64_t)row * H + h) * Dv;
    for (int d = lane; d < Dv; d += 64) {
        float acc = 0.f;
        for (int t = 0; t < n; ++t) acc = fmaf(z[t], kv[(int64_t)pr[t] * Dqk + d], acc);
        oh[d] = acc * inv;
    }
    if (lse != nullptr && lane == 0) lse[(int64_t)row * H + h] = n > 0 ? mx + logf(sum) : -INFINITY;
}

// ---------------------------------------------------------------- launchers

int attn_splits(int rows, int top_k, int Dqk) {
    if (Dqk != kDqk) return 1;
    const int nchunks = (top_k + kCh - 1) / kCh;
    int s = rows >= 256 ? 1 : (256 + rows - 1) / rows;
    s = s > nchunks ? nchunks : s;
    s = s > kAttnMaxSplits ? kAttnMaxSplits : s;
    // each split must fit its compacted slot list in LDS
    while ((top_k + s - 1) / s > kAttnMaxSplitSlots) ++s;
    return s < 1 ? 1 : s;
}

int attn_per_split(int top_k, int splits) {
    const int nchunks = (top_k + kCh - 1) / kCh;
    return ((nchunks + splits - 1) / splits) * kCh;
}

hipError_t launch_sparse_attn(const AttnLaunch& a, hipStream_t st) {
    const int rows = a.batch * a.n_q;
    if (rows == 0) return hipSuccess;
    if (a.q_dtype == 0) {
        const size_t sh = (size_t)a.top_k * (sizeof(float) + sizeof(int));
        hipLaunchKernelGGL(sfa_f32_kernel, dim3(a.H, rows), dim3(64), sh, st, (const float*)a.q,
                           (const float*)a.kv, a.seq_lens, a.table, a.max_blocks, a.num_blocks, a.n_q,
                           a.max_seq_len, a.indices, a.top_k, a.H, a.Dqk, a.Dv, a.sm_scale, (float*)a.out,
                           a.lse);
        return hipGetLastError();
    }
    const int splits = a.splits;
    const int per = splits == 1 ? a.top_k : attn_per_split(a.top_k, splits);
    const int grid = splits == 1 ? rows : ((rows + 7) / 8) * 8 * splits;
    const float scale_log2 = a.sm_scale * kLog2e;
    float* ws_lse = splits == 1 ? nullptr : a.ws + (size_t)rows * splits * kH * kDv;
    if (a.kv_kind == 2)
        hipLaunchKernelGGL((sfa_mla_kernel<true>), dim3(grid), dim3(512), 0, st, (const uint16_t*)a.q,
                           (const uint8_t*)a.kv, a.kvscale, a.seq_lens, a.table, a.max_blocks, a.num_blocks,
                           a.n_q, a.max_seq_len, rows, a.indices, a.top_k, per, splits, scale_log2,
                           (uint16_t*)a.out, a.lse, a.ws, ws_lse);
    else
        hipLaunchKernelGGL((sfa_mla_kernel<false>), dim3(grid), dim3(512), 0, st, (const uint16_t*)a.q,
                           (const uint8_t*)a.kv, a.kvscale, a.seq_lens, a.table, a.max_blocks, a.num_blocks,
                           a.n_q, a.max_seq_len, rows, a.indices, a.top_k, per, splits, scale_log2,
                           (uint16_t*)a.out, a.lse, a.ws, ws_lse);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    hipLaunchKernelGGL((sfa_combine_kernel<true>), dim3(rows, kH / 4), dim3(256), 0, st, a.ws, ws_lse, splits, kH,
                       kDv, a.out, a.lse);
    return hipGetLastError();
}

size_t attn_ws_bytes(int rows, int top_k, int Dqk, int H, int Dv) {
    const int s = attn_splits(rows, top_k, Dqk);
    if (s == 1) return 0;
    return sizeof(float) * (size_t)rows * s * H * ((size_t)Dv + 1);
}

}  // namespace dsa
