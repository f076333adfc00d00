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

// Work decomposition: one workgroup per (row, half of the heads, split of the
// index list).  The two head halves write disjoint outputs (no merge); only
// position splits produce partials, merged by LSE afterwards.  The workgroups
// of one row are consecutive on one XCD, so the two halves' gathers of the
// same latent rows meet in that XCD's L2.
//
// Workgroup: 4 waves, one per SIMD (the whole register file each), 64 heads.
// Per chunk of 32 positions:
//   QK   wave w owns heads 32(w&1) .. +31 of the half and positions 16(w>>1)
//        .. +15 of the chunk: S^T = K . Q^T with Q^T resident in registers,
//        each K fragment read from LDS feeding two MFMAs; the two waves of a
//        head pair exchange their partial row maxima through LDS, then each
//        writes its bf16 probabilities P[head][pos] and keeps a partial
//        denominator (summed at the end);
//   PV   wave w owns value channels 128w .. 128w+127 for the half's 64 heads:
//        O^T[d][h] += V^T . P^T, each V^T fragment (transposing LDS read)
//        feeding 4 MFMAs and each P^T fragment 8.
// LDS (one workgroup per CU): 3 x 36 KiB gather ring (bf16 cache), or 3 x
// 18.75 KiB fp8 staging + 2 bf16 tiles (MXFP8 cache); + P 5 KiB + slot list 8 KiB.
constexpr int kWaves = 4, kThreads = kWaves * kWave;
constexpr int kHalf = kH / 2;                   // heads per workgroup
constexpr int kDvPerWave = kDv / kWaves;        // 128 value channels = 8 D-tiles
constexpr int kRing = 3;                        // chunks resident in LDS (bf16 cache)
constexpr int kMxRing = 3;                      // fp8 staging slots (MXFP8 cache)
constexpr int kMxCodeB = kCh * kDqk;            // fp8 codes of a chunk (18432 B)
constexpr int kMxScaleW = 24;                   // bytes of an aligned window holding a row's 18 scales
constexpr int kMxStageB = kMxCodeB + kCh * kMxScaleW;
constexpr int kGatherK = kTileB / (16 * kWave);          // 36 wave-instructions per bf16 chunk
constexpr int kMxCodeK = kMxCodeB / (16 * kWave);        // 18 per fp8 chunk
constexpr int kMxScaleK = kCh * kMxScaleW / (4 * kWave); // 3 (dword lanes), waves 1..3
constexpr int kPRow = kCh * 2 + 16;             // bytes per head row of P (64 + 16 pad)

template <bool MX>
__global__ __launch_bounds__(kThreads, 1) void sfa_mla_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv, const uint8_t* __restrict__ kvscale,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ table, int max_blocks,
    int64_t num_blocks, int n_q, int max_seq_len, int rows, const int32_t* __restrict__ indices,
    int top_k, int per_split, int splits, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ ws_o, float* __restrict__ ws_lse) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[MX ? 2 : kRing][kTileB];
    __shared__ __attribute__((aligned(16))) uint8_t stage[MX ? kMxRing : 1][MX ? kMxStageB : 16];
    __shared__ __attribute__((aligned(16))) uint8_t pbuf[2][kHalf * kPRow];  // P[head][pos] bf16, by chunk parity
    __shared__ float alpha_s[2][kHalf];  // rescale factor per head, by chunk parity
    __shared__ float pmax_s[2][kHalf]; // chunk maximum per head over each position half
    __shared__ float lpart_s[2][kHalf]; // final partial denominators per position half
    __shared__ int rescale_chunk[2];  // the chunk (by parity) whose factors are not all 1
    __shared__ int32_t prow[kAttnMaxSplitSlots];
    __shared__ int wave_cnt[kWaves];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, j = lane & 15;

    // work item (row, half, split); ids equal mod 8 share an XCD, and a row's
    // 2*splits workgroups are consecutive on it.  Rows run longest-first.
    const int per_row = 2 * splits;
    const int x = blockIdx.x & 7, jj = blockIdx.x >> 3;
    const int rows_pad = (rows + 7) & ~7;
    const int row = rows_pad - 1 - ((jj / per_row) * 8 + x);
    const int half = (jj % per_row) & 1, split = (jj % per_row) >> 1;
    if (row < 0 || row >= rows) return;  // padding of the grid (block-uniform)
    const int hb = half * kHalf;         // first head of this workgroup
    const int b = row / n_q, qi = row % n_q;
    const int L = history_len(clamp_len(seq_lens, b, max_seq_len), n_q, qi);
    const int slot0 = split * per_split;
    const int slot1 = min(top_k, slot0 + per_split);

    // QK role of this wave: head pair hq (32 heads) x position half ph.  Q^T
    // fragments: qf[ht][ks] holds q[hb + 32hq + 16ht + j][32ks + 8g .. +8].
    // Loaded first so that they retire, with the index loads below, before the
    // gather ring starts (a wait for them inside the loop would drain it).
    const int hq = wave & 1, ph = wave >> 1;
    const int hl0 = 32 * hq;             // first head of the pair, within the half
    bf16x8 qf[2][kDqk / 32];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
        const uint16_t* qrow = q + ((int64_t)row * kH + hb + hl0 + 16 * ht + j) * kDqk + 8 * g;
#pragma unroll
        for (int ks = 0; ks < kDqk / 32; ++ks) qf[ht][ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
    }

    // 0. ordered compaction of the valid index slots into pool-row numbers
    int n_valid = 0;
    for (int base = slot0; base < slot1; base += kThreads) {
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
        for (int w = 0; w < kWaves; ++w) {
            before += w < wave ? wave_cnt[w] : 0;
            tot += wave_cnt[w];
        }
        if (pr >= 0) prow[n_valid + before + lanes_below(m)] = pr;
        n_valid += tot;
        __syncthreads();
    }
    const int nchunks = (n_valid + kCh - 1) / kCh;
    if (tid < 2) rescale_chunk[tid] = -1;  // visible after the first barrier of the ring
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): q and index loads retired (known to the compiler)

    // O^T accumulators: o[dt][ht] holds O^T[128w + 16dt + 4g + i][head hb + 16ht + j]
    f32x4 o[kDvPerWave / 16][kHalf / 16];
#pragma unroll
    for (int dt = 0; dt < kDvPerWave / 16; ++dt)
#pragma unroll
        for (int ht = 0; ht < kHalf / 16; ++ht) o[dt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
    // softmax state of heads hl0 + 16ht + j (the same m in both waves of the
    // pair; l over this wave's position half only)
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

    auto chunk_row = [&](int c, int r_) -> int {  // pool row of chunk row r_ (tail rows repeat a valid one)
        const int t = c * kCh + r_;
        return prow[t < n_valid ? t : c * kCh];
    };
    // Gathers issued per chunk by this wave (wave-instructions k = wave + 4i).
    constexpr int kBfPer = kGatherK / kWaves;                                                       // 9
    const int nk_mx = (kMxCodeK - wave + kWaves - 1) / kWaves + (wave >= kWaves - kMxScaleK ? 1 : 0); // 5 or 6
    const int per_chunk = MX ? nk_mx : kBfPer;

    // 1. bf16 cache: the chunk's 32 latent rows straight into a ring tile.
    //    Unit U (row U/72, column U%72) of the tile holds global column
    //    (U%72) ^ (row & 7): the XOR swizzle keeps the operand reads conflict free.
    auto issue_bf16 = [&](int c, int buf) {
        int pr[kBfPer];
#pragma unroll
        for (int i = 0; i < kBfPer; ++i) pr[i] = chunk_row(c, ((wave + kWaves * i) * kWave + lane) / kUnits);
        const uint32_t base = lds_addr(&tile[buf][0]);
#pragma unroll
        for (int i = 0; i < kBfPer; ++i) {
            const int k = wave + kWaves * i;
            const int U = k * kWave + lane;
            const int r_ = U / kUnits, col = (U % kUnits) ^ (r_ & 7);
            lds_gather16(kv + (int64_t)pr[i] * kRowB + col * 16, base + k * kWave * 16);
        }
    };
    // 1'. MXFP8 cache: codes [32][576] and, per row, the 4-byte-aligned 24-byte
    //     window of the scale pool that holds its 18 E8M0 scales.
    const int64_t scale_bytes = num_blocks * kBlock * (kDqk / 32);
    auto scale_window = [&](int pr) -> int64_t {
        const int64_t w = ((int64_t)pr * (kDqk / 32)) & ~(int64_t)3;
        return w + kMxScaleW <= scale_bytes ? w : scale_bytes - kMxScaleW;
    };
    auto issue_mx = [&](int c, int sb) {
        const uint32_t base = lds_addr(&stage[sb][0]);
        int pr[5];
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int k = wave + kWaves * i;
            if (k < kMxCodeK) pr[i] = chunk_row(c, (k * kWave + lane) / (kDqk / 16));
        }
        const int sk = wave - (kWaves - kMxScaleK);
        int spr = 0;
        if (sk >= 0) spr = chunk_row(c, (sk * kWave + lane) / (kMxScaleW / 4));
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int k = wave + kWaves * i;
            if (k < kMxCodeK) {
                const int cu = (k * kWave + lane) % (kDqk / 16);
                lds_gather16(kv + (int64_t)pr[i] * kDqk + cu * 16, base + k * kWave * 16);
            }
        }
        if (sk >= 0) {
            const int dw = (sk * kWave + lane) % (kMxScaleW / 4);
            lds_gather4(kvscale + scale_window(spr) + 4 * dw, base + kMxCodeB + sk * kWave * 4);
        }
    };
    // staged fp8 chunk -> dequantized bf16 tile (all threads)
    auto convert_mx = [&](int c, int sb, int tb) {
#pragma unroll 1
        for (int u = 0; u < (kMxCodeB / 16 + kThreads - 1) / kThreads; ++u) {
            const int U = tid + kThreads * u;
            if (U < kMxCodeB / 16) {
                const int r_ = U / (kDqk / 16), cu = U % (kDqk / 16);
                const int pr = chunk_row(c, r_);
                const int off = (int)((int64_t)pr * (kDqk / 32) - scale_window(pr));
                const float sc = e8m0_to_f32(stage[sb][kMxCodeB + r_ * kMxScaleW + off + cu / 2]);
                i32x4 lo, hi;
                dequant_unit(*reinterpret_cast<const i32x4*>(&stage[sb][U * 16]), sc, lo, hi);
                *reinterpret_cast<i32x4*>(&tile[tb][lds_unit(r_, 2 * cu)]) = lo;
                *reinterpret_cast<i32x4*>(&tile[tb][lds_unit(r_, 2 * cu + 1)]) = hi;
            }
        }
    };

    // 2. QK of this wave's 32 heads x 16 positions, then the softmax of the
    //    chunk with the partner wave (same heads, other position half).
    //    Lane holds S[head hl0 + 16ht + j][pos 16ph + 4g + i] in s[ht][i].
    auto qk = [&](const uint8_t* T) -> auto {
        // The 18 K fragments of the wave's 16 rows are read in two batches of 9,
        // each batch issued ahead of its MFMAs so that LDS latencies overlap.
        // Unit 4ks + g of row r sits at ((4(ks&1) + g) ^ (r&7)) + 8(ks>>1).
        constexpr int KB = kDqk / 64;  // 9
        const int r_ = 16 * ph + j;
        const uint8_t* base0 = T + r_ * kRowB + ((g ^ (r_ & 7)) << 4);
        const uint8_t* base1 = T + r_ * kRowB + (((4 + g) ^ (r_ & 7)) << 4);
        f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int bh = 0; bh < 2; ++bh) {
            bf16x8 ka[KB];
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) {
                const int ks = bh * KB + kk;
                ka[kk] = *reinterpret_cast<const bf16x8*>(((ks & 1) ? base1 : base0) + 128 * (ks >> 1));
            }
            issue_fence();
#pragma unroll
            for (int kk = 0; kk < KB; ++kk)
#pragma unroll
                for (int ht = 0; ht < 2; ++ht) s[ht] = mfma_bf16(ka[kk], qf[ht][bh * KB + kk], s[ht]);
        }
        struct S2 { f32x4 v[2]; };
        return S2{{s[0], s[1]}};
    };
    auto softmax = [&](const f32x4 (&s)[2], int c) {
        float t[2][4];
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
            float cmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = c * kCh + 16 * ph + 4 * g + i < n_valid;
                t[ht][i] = ok ? s[ht][i] * scale_log2 : -INFINITY;
                cmax = fmaxf(cmax, t[ht][i]);
            }
            cmax = max_over_groups(cmax);
            if (g == 0) pmax_s[ph][hl0 + 16 * ht + j] = cmax;
        }
        sync_lds();  // partial maxima of both position halves are in LDS
        bool rescale = false;
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
            const int hl = hl0 + 16 * ht + j;
            const float cmax = fmaxf(pmax_s[0][hl], pmax_s[1][hl]);
            float alpha = 1.f;
            if (cmax > m_run[ht] + kRescale || (m_run[ht] == -INFINITY && cmax > -INFINITY)) {
                alpha = m_run[ht] == -INFINITY ? 0.f : exp2f(m_run[ht] - cmax);
                m_run[ht] = cmax;
            }
            rescale |= alpha != 1.f;
            float psum = 0.f;
            uint32_t w2[2];
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                const float p0 = t[ht][i] == -INFINITY ? 0.f : exp2f(t[ht][i] - m_run[ht]);
                const float p1 = t[ht][i + 1] == -INFINITY ? 0.f : exp2f(t[ht][i + 1] - m_run[ht]);
                w2[i / 2] = f32_to_bf16_bits(p0) | ((uint32_t)f32_to_bf16_bits(p1) << 16);  // P operand
                psum += p0 + p1;                                                          // fp32 denominator
            }
            *reinterpret_cast<uint2*>(pbuf[c & 1] + hl * kPRow + 2 * (16 * ph + 4 * g)) = make_uint2(w2[0], w2[1]);
            l_run[ht] = l_run[ht] * alpha + sum_over_groups(psum);
            if (ph == 0 && g == 0) alpha_s[c & 1][hl] = alpha;
        }
        if (ph == 0 && ballot(rescale) != 0ull && lane == 0) rescale_chunk[c & 1] = c;  // every writer stores c
    };

    // 3. PV on this wave's 128 value channels for the half's 64 heads.  V^T
    //    fragment: lane j of group g addresses row 8g + 4h + j/4, channels
    //    d0 + 4(j%4) (two transposing reads give positions 8g .. 8g+7 in
    //    order); P^T fragment: lane reads P[head 16ht + j][pos 8g .. 8g+7].
    auto pv = [&](const uint8_t* T, int c) {
        if (rescale_chunk[c & 1] == c) {  // workgroup-uniform
#pragma unroll
            for (int ht = 0; ht < kHalf / 16; ++ht) {
                const float al = alpha_s[c & 1][16 * ht + j];
#pragma unroll
                for (int dt = 0; dt < kDvPerWave / 16; ++dt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[dt][ht][i] *= al;
            }
        }
        bf16x8 pf[kHalf / 16];
#pragma unroll
        for (int ht = 0; ht < kHalf / 16; ++ht)
            pf[ht] = *reinterpret_cast<const bf16x8*>(pbuf[c & 1] + (16 * ht + j) * kPRow + 16 * g);
        const int e_ = j >> 2, q4 = j & 3;
        const int r0 = 8 * g + e_, r1 = 8 * g + 4 + e_;
#pragma unroll
        for (int bh = 0; bh < 2; ++bh) {
            bf16x8 vf[kDvPerWave / 32];
#pragma unroll
            for (int dd = 0; dd < kDvPerWave / 32; ++dd) {
                const int dt = bh * (kDvPerWave / 32) + dd;
                const int ch = wave * kDvPerWave + 16 * dt + 4 * q4;   // channel this lane addresses
                const int unit = ch >> 3, byte = (ch & 7) * 2;
                const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (DSA_LDS v4i16*)(T + r0 * kRowB + ((unit ^ (r0 & 7)) << 4) + byte));
                const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (DSA_LDS v4i16*)(T + r1 * kRowB + ((unit ^ (r1 & 7)) << 4) + byte));
                const v4i16 both[2] = {lo, hi};
                vf[dd] = *reinterpret_cast<const bf16x8*>(both);
            }
            issue_fence();
#pragma unroll
            for (int dd = 0; dd < kDvPerWave / 32; ++dd)
#pragma unroll
                for (int ht = 0; ht < kHalf / 16; ++ht)
                    o[bh * (kDvPerWave / 32) + dd][ht] = mfma_bf16(vf[dd], pf[ht], o[bh * (kDvPerWave / 32) + dd][ht]);
        }
    };

    // The gather ring: chunk c lives in ring slot c % R; at the top of
    // iteration c this wave has issued the chunks up to c + R - 2 (bf16) or
    // c + R - 1 (MXFP8, where the extra slot is the bf16 tile being filled).
    if constexpr (!MX) {
        // Software pipeline: iteration c runs QK(c), then PV(c-1), then the
        // softmax of chunk c, so that the softmax's dependent VALU chain runs
        // while the matrix core executes PV(c-1).  Slots: c-1 (PV), c (QK),
        // c+1 (in flight).
        if (nchunks > 0) issue_bf16(0, 0);
        for (int c = 0; c < nchunks; ++c) {
            wait_vmcnt(0);  // chunk c has landed
            sync_lds();     // ... for every wave; softmax(c-1) wrote P and alpha; slot (c+1) % R is free
            if (c + 1 < nchunks) issue_bf16(c + 1, (c + 1) % kRing);
            const auto sc = qk(tile[c % kRing]);
            if (c > 0) pv(tile[(c - 1) % kRing], c - 1);
            softmax(sc.v, c);
        }
        if (nchunks > 0) {
            sync_lds();
            pv(tile[(nchunks - 1) % kRing], nchunks - 1);
        }
    } else {
        for (int c = 0; c < kMxRing && c < nchunks; ++c) issue_mx(c, c);
        if (nchunks > 0) {
            wait_vmcnt(per_chunk * min(kMxRing - 1, nchunks - 1));
            sync_lds();
            convert_mx(0, 0, 0);
        }
        for (int c = 0; c < nchunks; ++c) {
            const uint8_t* T = tile[c & 1];
            if (c + 1 < nchunks) wait_vmcnt(per_chunk * min(kMxRing - 2, nchunks - 2 - c));  // chunk c+1 staged
            sync_lds();  // tile c%2 converted; tile (c+1)%2, stage c%R and P are free
            if (c + kMxRing < nchunks) issue_mx(c + kMxRing, c % kMxRing);
            if (c + 1 < nchunks) convert_mx(c + 1, (c + 1) % kMxRing, (c + 1) & 1);
            const auto sc = qk(T);
            softmax(sc.v, c);
            sync_lds();
            pv(T, c);
        }
    }

    // 4. results.  The denominators of the two position halves are summed.
    if (g == 0) {
        lpart_s[ph][hl0 + j] = l_run[0];
        lpart_s[ph][hl0 + 16 + j] = l_run[1];
        if (ph == 0) {
            pmax_s[0][hl0 + j] = m_run[0];
            pmax_s[0][hl0 + 16 + j] = m_run[1];
        }
    }
    __syncthreads();
    const int64_t part = (int64_t)row * splits + split;
#pragma unroll
    for (int ht = 0; ht < kHalf / 16; ++ht) {
        const int h = hb + 16 * ht + j;
        const float lsum = lpart_s[0][16 * ht + j] + lpart_s[1][16 * ht + j];
        const float inv_l = lsum > 0.f ? 1.f / lsum : 0.f;
        const int d0 = wave * kDvPerWave + 4 * g;
        if (splits == 1) {
            uint16_t* orow = out + ((int64_t)row * kH + h) * kDv + d0;
#pragma unroll
            for (int dt = 0; dt < kDvPerWave / 16; ++dt) {
                const f32x4 v = o[dt][ht];
                const uint32_t lo = f32_to_bf16_bits(v[0] * inv_l) | ((uint32_t)f32_to_bf16_bits(v[1] * inv_l) << 16);
                const uint32_t hi = f32_to_bf16_bits(v[2] * inv_l) | ((uint32_t)f32_to_bf16_bits(v[3] * inv_l) << 16);
                *reinterpret_cast<uint2*>(orow + 16 * dt) = make_uint2(lo, hi);
            }
        } else {
            float* orow = ws_o + (part * kH + h) * kDv + d0;
#pragma unroll
            for (int dt = 0; dt < kDvPerWave / 16; ++dt) {
                const f32x4 v = o[dt][ht];
                *reinterpret_cast<f32x4*>(orow + 16 * dt) = f32x4{v[0] * inv_l, v[1] * inv_l, v[2] * inv_l, v[3] * inv_l};
            }
        }
    }
    if (tid < kHalf) {
        const float lsum = lpart_s[0][tid] + lpart_s[1][tid];
        const float hl_lse = lsum > 0.f ? (pmax_s[0][tid] + log2f(lsum)) * kLn2 : -INFINITY;
        if (splits == 1) {
            if (lse != nullptr) lse[(int64_t)row * kH + hb + tid] = hl_lse;
        } else {
            ws_lse[part * kH + hb + tid] = hl_lse;
        }
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
    // two head halves per row already; split the index list until ~256 workgroups
    int s = rows >= 128 ? 1 : (128 + rows - 1) / rows;
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
    const int grid = ((rows + 7) / 8) * 8 * 2 * splits;   // (row, head half, split)
    const float scale_log2 = a.sm_scale * kLog2e;
    float* ws_lse = splits == 1 ? nullptr : a.ws + (size_t)rows * splits * kH * kDv;
    if (a.kv_kind == 2)
        hipLaunchKernelGGL((sfa_mla_kernel<true>), dim3(grid), dim3(kThreads), 0, st, (const uint16_t*)a.q,
                           (const uint8_t*)a.kv, a.kvscale, a.seq_lens, a.table, a.max_blocks, a.num_blocks,
                           a.n_q, a.max_seq_len, rows, a.indices, a.top_k, per, splits, scale_log2,
                           (uint16_t*)a.out, a.lse, a.ws, ws_lse);
    else
        hipLaunchKernelGGL((sfa_mla_kernel<false>), dim3(grid), dim3(kThreads), 0, st, (const uint16_t*)a.q,
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
