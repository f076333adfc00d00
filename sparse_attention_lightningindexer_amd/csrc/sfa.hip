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
// Kernel structure (128 heads, d_qk 576, d_v 512), one workgroup of 4 waves
// per (row, half of the heads, split of the index list):
//   0. the split's index slots are validated (0 <= s < L_r, block present)
//      and compacted in order into LDS as pool-row numbers;
//   1. per chunk of 32 positions the latent rows are gathered through
//      registers into a 4-tile LDS ring (16-byte units XOR-swizzled by row so
//      the MFMA operand reads are bank-conflict free).  An MXFP8 cache is
//      dequantized (e4m3 * 2^(e8m0-127), exact in bf16) on the way in;
//   2. S^T = K . Q^T on MFMA with Q held in registers for the whole kernel;
//   3. softmax in the log2 domain, per head, in registers, relative to a
//      fixed reference (the first chunk's maximum; an exact second pass if a
//      later logit exceeds it by more than 2^32), so the accumulators are
//      never rescaled;
//   4. O^T += V^T . P^T on MFMA: P is laid out in LDS as the B operand, and
//      V^T comes from LDS with the transposing read ds_read_b64_tr_b16;
//   5. the row's result (or the split's normalized partial and its LSE) is
//      written; a combine kernel merges the splits by LSE.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace dsa {

constexpr int kH = 128, kDqk = 576, kDv = 512, kCh = 32;
constexpr int kRowB = kDqk * 2;        // bytes per bf16 latent row
constexpr int kTileB = kCh * kRowB;    // 36864 bytes per chunk
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSlack = 32.0f;        // probabilities may exceed 1 by up to 2^32 (log2 units)

// LDS byte offset of 16-byte unit u of tile row `row`: the low three unit bits
// are XORed with bits 1..3 of the row.  With the 1152-byte row stride this
// keeps the 16-row fragment reads (16 lanes per LDS pass, 64 banks) and whole-
// row stores free of bank conflicts, and changes units only within aligned
// groups of eight (so offsets of 8 units stay immediates).
__device__ __forceinline__ int row_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int lds_unit(int row, int u) { return row * kRowB + ((u ^ row_swz(row)) << 4); }

// 16 e4m3 codes (one 16-byte unit) times the power of two 2^(e8m0 - 127) ->
// 16 bf16 (exact): the scaled conversion takes the scale's exponent field as
// the E8M0 byte, two codes per instruction.
__device__ __forceinline__ void dequant_unit_mx(i32x4 codes, uint32_t e8m0, i32x4& lo, i32x4& hi) {
    const float scale = __uint_as_float(e8m0 << 23);  // only the exponent field is read
    uint32_t packed[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        packed[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[w], scale, false));
        packed[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[w], scale, true));
    }
    lo = i32x4{(int)packed[0], (int)packed[1], (int)packed[2], (int)packed[3]};
    hi = i32x4{(int)packed[4], (int)packed[5], (int)packed[6], (int)packed[7]};
}

// 16 e4m3 codes times an fp32 scale -> 16 bf16: the fp32 product, rounded to
// nearest-even bf16 (not exact; defined below, after pack_bf16x2).
__device__ __forceinline__ void dequant_unit_rne(i32x4 codes, float scale, i32x4& lo, i32x4& hi);

// Work decomposition: one workgroup per (row, half of the heads, split of the
// index list).  The two head halves write disjoint outputs (no merge); only
// position splits produce partials, merged by LSE afterwards.  The workgroups
// of one row are consecutive on one XCD, so the two halves' gathers of the
// same latent rows meet in that XCD's L2.
//
// Workgroup: 8 waves, two per SIMD (waves w and w+4 share SIMD w), 64 heads,
// in two roles.  A wave's own MFMAs and vector-ALU work do not overlap on this
// chip, but the MFMAs of one wave and the ALU work of the other wave on the
// same SIMD do; each SIMD therefore holds one wave of each role.  Per chunk of
// 32 positions:
//   QK   waves 0..3 own heads 16w .. 16w+15 of the half over all 32 positions:
//        S^T = K . Q^T with Q^T resident in registers; the row maxima and the
//        softmax of the chunk are local to the wave, which writes bf16
//        P[head][pos] to LDS;
//   PV   waves 4..7 own value channels 128(w-4) .. +127 for all 64 heads:
//        O^T[d][h] += V^T . P^T, each V^T fragment (transposing LDS read)
//        feeding 4 MFMAs and each P^T fragment 8;
//   all  eight waves gather the chunk's latent rows through registers, four
//        rows each (row r of wave w in register r, chunk c in lane c).
// The QK waves run one chunk ahead: in iteration c they compute QK(c) and the
// softmax of chunk c-1, while the PV waves compute PV(c-2).  One barrier per
// chunk hands tiles and P over.  Chunks are loaded two iterations before they
// are stored and stored one iteration before their QK.  LDS (one workgroup
// per CU): 4 x 36 KiB tiles + P 10 KiB; the slot list of the compaction lives
// in the fourth tile until the gathers start.
constexpr int kWaves = 8, kThreads = kWaves * kWave;
constexpr int kHalf = kH / 2;                   // heads per workgroup
constexpr int kRoleWaves = kWaves / 2;          // waves per role
constexpr int kQkHeads = kHalf / kRoleWaves;    // 16 heads per QK wave
constexpr int kDvPerPv = kDv / kRoleWaves;      // 128 value channels = 8 D-tiles per PV wave
constexpr int kRing = 4;                        // bf16 tiles resident in LDS
constexpr int kPRow = kCh * 2 + 16;             // bytes per head row of P (64 + 16 pad)
constexpr int kMxUnitsRow = kDqk / 16;          // 36 16-code units per MXFP8 row
constexpr int kStRows = kCh / kWaves;           // chunk rows gathered per wave
constexpr int kFusedTopkKpt = 16;               // keys per thread of the fused Top-K (rows up to 8192)

// two floats -> two bfloat16 (round to nearest even) packed in 32 bits
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 h2 __attribute__((ext_vector_type(2)));
    const h2 h = __builtin_convertvector((f2){a, b}, h2);
    return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ void dequant_unit_rne(i32x4 codes, float scale, i32x4& lo, i32x4& hi) {
    uint32_t packed[8];
    for (int w = 0; w < 4; ++w) {
        const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(codes[w], false);
        const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(codes[w], true);
        packed[2 * w] = pack_bf16x2(a[0] * scale, a[1] * scale);
        packed[2 * w + 1] = pack_bf16x2(c[0] * scale, c[1] * scale);
    }
    lo = i32x4{(int)packed[0], (int)packed[1], (int)packed[2], (int)packed[3]};
    hi = i32x4{(int)packed[4], (int)packed[5], (int)packed[6], (int)packed[7]};
}

// KV: 1 bf16, 2 MXFP8 (e4m3 + E8M0 per 32), 3 e4m3 + fp32 scale per 128.
// DENSE: the pool has the dense layout, so a row's place is a constant
// multiple of its number (no per-row stride arithmetic).
// TK: 0, the index lists are given (`indices`); else the fused form, in which
// every workgroup selects its row's top_k positions itself from the indexer's
// scores (TK keys per thread, rows up to 512 * TK positions), keeps its
// split's slots, and writes them to `indices` (head half 0).  The selection
// is the Top-K kernels' own (select.hpp), so the indices are the same
// ("Day0 Inference Adaptation and Performance Optimization for
// New-Architecture LLMs", §4.1: the top-k step feeds the sparse core).
template <int KV, bool DENSE, int TK>
__global__ __launch_bounds__(kThreads, 1) void sfa_mla_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv, const void* __restrict__ kvscale,
    PoolLayout kvl, const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ table, int max_blocks,
    int64_t num_blocks, int n_q, int max_seq_len, int rows, int32_t* __restrict__ indices,
    int top_k, int per_split, int splits, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse, uint16_t* __restrict__ ws_o, float* __restrict__ ws_lse,
    const float* __restrict__ scores, int64_t ld) {
    constexpr bool MX = KV != 1;  // e4m3 codes, dequantized to bf16 while staged
    __shared__ __attribute__((aligned(16))) uint8_t tile[kRing][kTileB];
    __shared__ __attribute__((aligned(16))) uint8_t pbuf[2][kHalf * kPRow];  // P[head][pos] bf16, by chunk parity
    __shared__ float l_s[kHalf], m_s[kHalf];
    __shared__ int overflow;             // some logit exceeded its reference by more than 2^kSlack
    __shared__ int wave_cnt[kWaves];
    int32_t* const prow = reinterpret_cast<int32_t*>(&tile[kRing - 1][0]);  // slot list (prologue only)
    static_assert(kAttnMaxSplitSlots * 4 <= kTileB, "slot list fits in one tile");

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

    // 0. ordered compaction of the valid index slots into pool-row numbers.
    //    All of the split's indices are loaded first, then all of their table
    //    entries (two memory round trips in total), then compacted.
    //    Run by both roles; the QK waves issue their query loads once the
    //    indices and table entries have arrived, so the queries arrive during
    //    the compaction without delaying it.  It ends with a barrier, after
    //    which every wave loads the pool rows of its chunk rows (vid).
    const int srow0 = kStRows * wave;  // the wave's first chunk row (staging, below)
    int n_valid = 0, nchunks = 0;
    int vid[kStRows];  // pool row of chunk row srow0 + r of chunk c, in lane c
    auto compact = [&](auto&& after_reads) __attribute__((always_inline)) {
        constexpr int kSlotIters = kAttnMaxSplitSlots / kThreads;
        // The sequence's block-table row goes to LDS beside the slot list
        // (when it fits), loaded together with the indices: then the
        // compaction costs one memory round trip instead of two.
        constexpr int kTabMax = (kTileB - kAttnMaxSplitSlots * 4) / 4;
        int32_t* const tab_s = prow + kAttnMaxSplitSlots;
        const int nb = (L + kBlock - 1) / kBlock;  // blocks of the history (<= max_blocks)
        const bool tab_lds = nb <= kTabMax;        // workgroup-uniform
        int pr_[kSlotIters];
        {
            // reads are unconditional (clamped to in-range slots and blocks) so
            // that each round trip is one batch of loads
            int sv[kSlotIters];
            if constexpr (TK == 0) {
#pragma unroll
                for (int k = 0; k < kSlotIters; ++k) {
                    const int t = slot0 + kThreads * k + tid;
                    const int v = indices[(int64_t)row * top_k + min(t, top_k - 1)];
                    sv[k] = t < slot1 && v >= 0 && v < L ? v : -1;
                }
                if (tab_lds)
                    for (int jb = tid; jb < nb; jb += kThreads)
                        tab_s[jb] = (int)phys_block(table, max_blocks, b, jb, num_blocks);
                if (tab_lds) __syncthreads();
                // the indices and table entries have arrived; later loads (the QK
                // waves' query) now overlap the compaction instead of delaying it
                after_reads();
            } else {
                // The row's Top-K, selected here: the table entries, the row's
                // score keys and (QK waves) the queries are all issued first, so
                // the queries arrive during the selection, whose barriers wait
                // for LDS only.  The split's positions go to spos (tile 0),
                // the selection's histogram to tile 1.
                int32_t* const spos = reinterpret_cast<int32_t*>(&tile[0][0]);
                auto& ssh = *reinterpret_cast<SelectShared<kThreads>*>(&tile[1][0]);
                static_assert(sizeof(SelectShared<kThreads>) <= kTileB, "select state fits in one tile");
                static_assert(kAttnMaxSplitSlots * 4 <= kTileB, "split positions fit in one tile");
                int32_t* const iout = indices + (int64_t)row * top_k;
                const bool whole = L <= top_k;  // the whole history is kept (workgroup-uniform)
                uint32_t key[TK];
                if (!whole) load_keys<TK>(scores + (int64_t)row * ld, TK * kWave * wave, L, lane, key);
                if (tab_lds)
                    for (int jb = tid; jb < nb; jb += kThreads)
                        tab_s[jb] = (int)phys_block(table, max_blocks, b, jb, num_blocks);
                after_reads();
                if (whole) {
                    for (int t = slot0 + tid; t < slot1; t += kThreads) spos[t - slot0] = t < L ? t : -1;
                } else {
                    clear_hist<kThreads, true>(ssh);
                    block_select<kThreads, TK, true>(ssh, key, top_k, [&](int place, int, int slot) {
                        if (place >= slot0 && place < slot1) spos[place - slot0] = slot;
                    });
                }
                sync_lds();  // spos and the table row are in LDS
                // the head-half-0 workgroups write their split's indices, one
                // coalesced store per thread (not scattered through the emit)
#pragma unroll
                for (int k = 0; k < kSlotIters; ++k) {
                    const int t = slot0 + kThreads * k + tid;
                    const int v = t < slot1 ? spos[t - slot0] : -1;
                    if (half == 0 && t < slot1) iout[t] = v;
                    sv[k] = v >= 0 && v < L ? v : -1;
                }
            }
#pragma unroll
            for (int k = 0; k < kSlotIters; ++k) {
                const int sk = sv[k];
                const int jb = sk < 0 ? 0 : sk / kBlock;
                const int64_t p = tab_lds ? (int64_t)tab_s[jb] : phys_block(table, max_blocks, b, jb, num_blocks);
                pr_[k] = (sk >= 0 && p >= 0) ? (int)(p * kBlock + (sk % kBlock)) : -1;
            }
        }
        n_valid = 0;
#pragma unroll
        for (int k = 0; k < kSlotIters; ++k) {
            if (slot0 + kThreads * k >= slot1) break;  // workgroup-uniform
            const int pr = pr_[k];
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
        nchunks = (n_valid + kCh - 1) / kCh;
        // pad the last chunk with a valid row, so every chunk row names real data
        if (tid < nchunks * kCh - n_valid) prow[n_valid + tid] = prow[0];
        if (tid == 0) overflow = 0;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < kStRows; ++r) vid[r] = lane < nchunks ? prow[lane * kCh + srow0 + r] : 0;
    };

    // 1. Staging, by every wave: wave w owns chunk rows 4w .. 4w+3.  bf16: each
    //    row's 512 latent channels are one 64-lane x 16-byte load from a row
    //    base in scalar registers; the rope units 64 + lane%8 of the four rows
    //    follow as one load (lanes 32..63 repeat lanes 0..31).  MXFP8: unit
    //    U = 64i + lane of the wave's 4 rows x 36 units (row U/36, 16 codes
    //    U%36; the third load's lanes past unit 143 repeat it) with its E8M0
    //    scale byte, dequantized (exact) to two bf16 units when stored.  Rows
    //    are stored at their XOR-swizzled places.
    constexpr int kMxPer = (kStRows * kMxUnitsRow + kWave - 1) / kWave;  // 3 MXFP8 loads per chunk
    constexpr int kStN = MX ? kMxPer : kStRows + 1;
    struct Stage {
        i32x4 v[kStN];
        uint32_t sc[MX ? kMxPer : 1];
    };
    // pool row of chunk row srow0 + r of chunk c (wave-uniform)
    auto sid = [&](int c, int r) __attribute__((always_inline)) -> int {
        return __builtin_amdgcn_readlane(vid[r], c);
    };
    // byte offsets of pool row pr (block pr/64, position pr%64) and of its scales
    auto row_off = [&](int pr) __attribute__((always_inline)) -> int64_t {
        if constexpr (DENSE) return (int64_t)pr * (MX ? kDqk : kRowB);
        else return (int64_t)(pr >> 6) * kvl.bs + (int64_t)(pr & 63) * kvl.rs;
    };
    auto scale_off = [&](int pr) __attribute__((always_inline)) -> int64_t {
        if constexpr (DENSE) return (int64_t)pr * (KV == 2 ? kDqk / 32 : 5 * 4);
        else return (int64_t)(pr >> 6) * kvl.sbs + (int64_t)(pr & 63) * kvl.srs;
    };
    const int rope_r = (lane & 31) >> 3;  // the row of the lane's rope unit
    auto load_chunk = [&](int c, Stage& st) __attribute__((always_inline)) {
        int rid[kStRows];
#pragma unroll
        for (int r = 0; r < kStRows; ++r) rid[r] = sid(c, r);
        if constexpr (!MX) {
#pragma unroll
            for (int r = 0; r < kStRows; ++r)
                st.v[r] = *reinterpret_cast<const i32x4*>(kv + row_off(rid[r]) + lane * 16);
            int id = rid[0];
#pragma unroll
            for (int m = 1; m < kStRows; ++m) id = rope_r == m ? rid[m] : id;
            st.v[kStRows] = *reinterpret_cast<const i32x4*>(kv + row_off(id) + 16 * (64 + (lane & 7)));
        } else {
#pragma unroll
            for (int i = 0; i < kMxPer; ++i) {
                const int U = min(kWave * i + lane, kStRows * kMxUnitsRow - 1);
                const int r = U / kMxUnitsRow, u = U - r * kMxUnitsRow;
                int id = rid[0];
#pragma unroll
                for (int m = 1; m < kStRows; ++m) id = r == m ? rid[m] : id;
                st.v[i] = *reinterpret_cast<const i32x4*>(kv + row_off(id) + u * 16);
                const uint8_t* sp = static_cast<const uint8_t*>(kvscale) + scale_off(id);
                if constexpr (KV == 2)  // E8M0 of the 32-code group u/2
                    st.sc[i] = sp[u >> 1];
                else  // fp32 of the 128-code group u/8 (five per row, the last one the rope)
                    st.sc[i] = __float_as_uint(reinterpret_cast<const float*>(sp)[u >> 3]);
            }
        }
    };
    auto store_chunk = [&](int slot, const Stage& st) __attribute__((always_inline)) {
        uint8_t* T = tile[slot];
        if constexpr (!MX) {
            uint8_t* Tw = T + srow0 * kRowB;
#pragma unroll
            for (int r = 0; r < kStRows; ++r)
                *reinterpret_cast<i32x4*>(Tw + r * kRowB + ((lane ^ row_swz(srow0 + r)) << 4)) = st.v[r];
            *reinterpret_cast<i32x4*>(T + lds_unit(srow0 + rope_r, 64 + (lane & 7))) = st.v[kStRows];
        } else {
#pragma unroll
            for (int i = 0; i < kMxPer; ++i) {
                const int U = min(kWave * i + lane, kStRows * kMxUnitsRow - 1);
                const int r = U / kMxUnitsRow, u = U - r * kMxUnitsRow;
                i32x4 lo, hi;
                if constexpr (KV == 2) dequant_unit_mx(st.v[i], st.sc[i], lo, hi);
                else dequant_unit_rne(st.v[i], __uint_as_float(st.sc[i]), lo, hi);
                *reinterpret_cast<i32x4*>(T + lds_unit(srow0 + r, 2 * u)) = lo;
                *reinterpret_cast<i32x4*>(T + lds_unit(srow0 + r, 2 * u + 1)) = hi;
            }
        }
    };

    // The chunk pipeline, run by both roles: chunk c lives in tile c % 4.
    // Chunk k is loaded into registers in iteration k-3 (k < 3: before the
    // first barrier) and stored into its tile in iteration k-1 (tile k % 4 was
    // last read by PV(k-4) in iteration k-2).  Iteration c (c = 0 .. nchunks,
    // after its barrier): chunk c is in LDS and P(c-2) is written; work(c) is
    // QK(c) with softmax(c-1) in the QK waves and PV(c-2) in the PV waves.
    // Both roles execute the same nchunks + 2 barriers; after the last one the
    // PV waves compute PV(nchunks-1) (tail()).
    auto pipeline = [&](auto&& work, auto&& tail) __attribute__((always_inline)) {
        if (nchunks == 0) return;
        Stage stA, stB;  // chunk k is staged in stA (k even) or stB (k odd)
        load_chunk(0, stA);
        if (nchunks > 1) load_chunk(1, stB);
        store_chunk(0, stA);
        if (nchunks > 2) load_chunk(2, stA);
        // st holds chunk c+1 and receives chunk c+3
        auto step = [&](int c, Stage& st) __attribute__((always_inline)) {
            sync_lds();  // barrier c
            if (c + 1 < nchunks) {
                store_chunk((c + 1) % kRing, st);
                if (c + 3 < nchunks) load_chunk(c + 3, st);
            }
            work(c);
        };
        step(0, stB);
        int c = 1;
        for (; c + 1 <= nchunks; c += 2) {
            step(c, stA);  // stores chunk c+1 (even), loads c+3 (even)
            step(c + 1, stB);
        }
        if (c <= nchunks) step(c, stA);
        sync_lds();  // barrier nchunks + 1
        tail();
    };

    // Softmax without rescaling.  Each head's probabilities are taken
    // relative to a reference: the first chunk's maximum.  The accumulators
    // never need rescaling as long as no later logit exceeds the reference by
    // more than 2^kSlack (probabilities, O and l stay far from fp32 and bf16
    // overflow); if one does, the whole work item is computed again with the
    // exact maximum, observed on the way, as the reference.  The result is the
    // same softmax either way (reference and denominator cancel).
    if (wave < kRoleWaves) {
        // ---------------------------------------------------------- QK role
        // heads hl0 .. hl0+15 of the half.  qf[ks] holds
        // q[hb + hl0 + j][32ks + 8g .. +8] (the B operand of S^T = K . Q^T).
        const int hl0 = kQkHeads * wave;
        bf16x8 qf[kDqk / 32];
        compact([&]() __attribute__((always_inline)) {
            const uint16_t* qrow = q + ((int64_t)row * kH + hb + hl0 + j) * kDqk + 8 * g;
#pragma unroll
            for (int ks = 0; ks < kDqk / 32; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
        });
        // per head hl0 + j: the reference (identical in the four lane groups),
        // and this lane's largest scaled logit seen and share of the
        // denominator (both reduced over the lane groups only at the end)
        float m_ref = -INFINITY, m_obs = -INFINITY, l_run = 0.f;
        bool exact = false;  // the reference is the exact maximum (second pass)

        // S for 16 heads x 32 positions: lane holds S[head hl0 + j][pos 16pt +
        // 4g + i] in s[pt][i].  K fragment (pt, ks): row 16pt + j, unit 4ks + g.
        // Reads run one batch of 6 fragments ahead of the MFMAs that consume
        // them.
        struct S2 { f32x4 v[2]; };
        auto qk = [&](const uint8_t* T) __attribute__((always_inline)) -> S2 {
            S2 s;
            s.v[0] = f32x4{0.f, 0.f, 0.f, 0.f};
            s.v[1] = f32x4{0.f, 0.f, 0.f, 0.f};
            constexpr int NB = 6, NBATCH = 2 * (kDqk / 32) / NB;  // 6 batches of 6 fragments
            // unit 4ks + g of row r sits at 16 * ((4(ks&1) + g) ^ swz(r)) + 128 (ks>>1);
            // rows j and 16 + j share swz, so two base addresses and immediate
            // offsets cover all 36 fragments.
            const uint8_t* base0 = T + j * kRowB + ((g ^ row_swz(j)) << 4);
            const uint8_t* base1 = T + j * kRowB + (((4 + g) ^ row_swz(j)) << 4);
            bf16x8 ka[2][NB];
            auto read_batch = [&](int bt, bf16x8 (&dst)[NB]) __attribute__((always_inline)) {
#pragma unroll
                for (int kk = 0; kk < NB; ++kk) {
                    const int f = bt * NB + kk, pt = f & 1, ks = f >> 1;
                    dst[kk] = *reinterpret_cast<const bf16x8*>(((ks & 1) ? base1 : base0) + 16 * pt * kRowB +
                                                               128 * (ks >> 1));
                }
            };
            read_batch(0, ka[0]);
#pragma unroll
            for (int bt = 0; bt < NBATCH; ++bt) {
                if (bt + 1 < NBATCH) read_batch(bt + 1, ka[(bt + 1) & 1]);
#pragma unroll
                for (int kk = 0; kk < NB; ++kk) {
                    const int f = bt * NB + kk, pt = f & 1, ks = f >> 1;
                    s.v[pt] = mfma_bf16(ka[bt & 1][kk], qf[ks], s.v[pt]);
                }
            }
            return s;
        };
        // softmax of the chunk for head hl0 + j, local to the wave.  Positions
        // past the valid ones are -inf; exp2 of -inf is 0.
        auto softmax = [&](const S2& s, int c) __attribute__((always_inline)) {
            const int lim = n_valid - c * kCh - 4 * g;  // position 16pt + 4g + i is valid iff 16pt + i < lim
            float sm[2][4];
            float cmax = -INFINITY;
#pragma unroll
            for (int pt = 0; pt < 2; ++pt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sm[pt][i] = 16 * pt + i < lim ? s.v[pt][i] : -INFINITY;
                    cmax = fmaxf(cmax, sm[pt][i]);
                }
            cmax *= scale_log2;  // scale_log2 > 0; this lane's positions only
            if (!exact && c == 0) m_ref = max_over_groups(cmax);
            m_obs = fmaxf(m_obs, cmax);
            const bool over = cmax > m_ref + kSlack;     // also a reference of -inf; any lane counts
            const float mneg = m_ref == -INFINITY ? 0.f : -m_ref;
            float psum = 0.f;
            const int hl = hl0 + j;
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) {
                float p[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[i] = __builtin_amdgcn_exp2f(fmaf(sm[pt][i], scale_log2, mneg));
                    psum += p[i];  // fp32 denominator
                }
                *reinterpret_cast<uint2*>(pbuf[c & 1] + hl * kPRow + 2 * (16 * pt + 4 * g)) =
                    make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
            }
            l_run += psum;
            if (ballot(over) != 0ull && lane == 0) overflow = 1;
        };

        for (;;) {
            S2 s_prev;  // S of the previous chunk, its softmax pending
            pipeline(
                [&](int c) __attribute__((always_inline)) {
                    if (c == 0) {
                        s_prev = qk(tile[0]);
                    } else if (c < nchunks) {
                        const S2 s_cur = qk(tile[c % kRing]);  // independent of the softmax below
                        softmax(s_prev, c - 1);
                        s_prev = s_cur;
                    } else {
                        softmax(s_prev, c - 1);
                    }
                },
                []() __attribute__((always_inline)) {});
            if (overflow == 0) break;  // read by every wave after the pipeline's last barrier
            __syncthreads();           // every wave has read the flag
            if (tid == 0) overflow = 0;
            exact = true;
            m_ref = max_over_groups(m_obs);
            l_run = 0.f;
        }
        l_run = sum_over_groups(l_run);
        if (g == 0) {
            l_s[hl0 + j] = l_run;
            m_s[hl0 + j] = m_ref;
        }
        __syncthreads();  // l and m are in LDS
        __syncthreads();  // the PV waves' results are in LDS
    } else {
        // ---------------------------------------------------------- PV role
        // value channels 128pw + 16dt + 4g + i for the half's 64 heads:
        // o[dt][ht] holds O^T[128pw + 16dt + 4g + i][head hb + 16ht + j].
        const int pw = wave - kRoleWaves;
        compact([]() __attribute__((always_inline)) {});
        f32x4 o[kDvPerPv / 16][kHalf / 16];
#pragma unroll
        for (int dt = 0; dt < kDvPerPv / 16; ++dt)
#pragma unroll
            for (int ht = 0; ht < kHalf / 16; ++ht) o[dt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};

        // V^T fragment (d-tile dt): lane j of group g addresses row 8g + 4h +
        // j/4, channels 128pw + 16dt + 4(j%4) (two transposing reads give
        // positions 8g .. 8g+7 in order); P^T fragment: lane reads P[head
        // 16ht + j][pos 8g .. 8g+7].  Channel 128pw + 16dt + 4(j%4) is unit
        // 16pw + 2dt + (j%4)/2, byte 8((j%4)&1); d-tiles 4 apart differ by one
        // 128-byte step, so four bases per row and immediates cover all 8.
        auto pv = [&](const uint8_t* T, int c) __attribute__((always_inline)) {
            bf16x8 pf[kHalf / 16];
#pragma unroll
            for (int ht = 0; ht < kHalf / 16; ++ht)
                pf[ht] = *reinterpret_cast<const bf16x8*>(pbuf[c & 1] + (16 * ht + j) * kPRow + 16 * g);
            // the V^T read places are rebuilt per chunk from a fresh lane index
            // rather than held in registers through the pipeline
            int lv = lane;
            asm volatile("" : "+v"(lv));
            const int jv = lv & 15, gv = lv >> 4;
            const int e_ = jv >> 2, q4 = jv & 3;
            const int r0 = 8 * gv + e_, r1 = 8 * gv + 4 + e_;
            auto vaddr = [&](int r_, int dd) __attribute__((always_inline)) -> const uint8_t* {
                const int unit = 16 * pw + 2 * dd + (q4 >> 1);
                return T + r_ * kRowB + ((unit ^ row_swz(r_)) << 4) + 8 * (q4 & 1);
            };
            constexpr int NBT = 2;  // d-tiles per batch
            auto read_v = [&](int bt, bf16x8 (&vf)[NBT]) __attribute__((always_inline)) {
#pragma unroll
                for (int dd = 0; dd < NBT; ++dd) {
                    const int dt = NBT * bt + dd;  // bases for dt % 4, one 128-byte step per 4 d-tiles
                    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (DSA_LDS v4i16*)(vaddr(r0, dt & 3) + 128 * (dt >> 2)));
                    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (DSA_LDS v4i16*)(vaddr(r1, dt & 3) + 128 * (dt >> 2)));
                    const v4i16 both[2] = {lo, hi};
                    vf[dd] = *reinterpret_cast<const bf16x8*>(both);
                }
            };
            bf16x8 vf[2][NBT];
            read_v(0, vf[0]);
#pragma unroll
            for (int bt = 0; bt < kDvPerPv / 16 / NBT; ++bt) {
                issue_fence();
                if (bt + 1 < kDvPerPv / 16 / NBT) read_v(bt + 1, vf[(bt + 1) & 1]);
#pragma unroll
                for (int dd = 0; dd < NBT; ++dd)
#pragma unroll
                    for (int ht = 0; ht < kHalf / 16; ++ht)
                        o[NBT * bt + dd][ht] = mfma_bf16(vf[bt & 1][dd], pf[ht], o[NBT * bt + dd][ht]);
            }
            issue_fence();
        };

        for (;;) {
            pipeline([&](int c) __attribute__((always_inline)) {
                         if (c >= 2) pv(tile[(c - 2) % kRing], c - 2);
                     },
                     [&]() __attribute__((always_inline)) { pv(tile[(nchunks - 1) % kRing], nchunks - 1); });
            if (overflow == 0) break;
            __syncthreads();  // every wave has read the flag; the work item is computed again
#pragma unroll
            for (int dt = 0; dt < kDvPerPv / 16; ++dt)
#pragma unroll
                for (int ht = 0; ht < kHalf / 16; ++ht) o[dt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

        // normalized bf16 rows into LDS (the tiles are free now)
        __syncthreads();  // l and m are in LDS
        constexpr int kORow = kDv * 2 + 16;  // padded LDS row of one head
        uint8_t* obuf = &tile[0][0];
#pragma unroll
        for (int ht = 0; ht < kHalf / 16; ++ht) {
            const float lsum = l_s[16 * ht + j];
            const float inv_l = lsum > 0.f ? 1.f / lsum : 0.f;
            uint8_t* orow = obuf + (16 * ht + j) * kORow + 2 * (pw * kDvPerPv + 4 * g);
#pragma unroll
            for (int dt = 0; dt < kDvPerPv / 16; ++dt) {
                const f32x4 v = o[dt][ht];
                *reinterpret_cast<uint2*>(orow + 32 * dt) =
                    make_uint2(pack_bf16x2(v[0] * inv_l, v[1] * inv_l), pack_bf16x2(v[2] * inv_l, v[3] * inv_l));
            }
        }
        __syncthreads();  // the results are in LDS
    }

    // 4. results: every store instruction writes one contiguous 1 KB head row,
    //    O[row][hb + h][:] (or the split's partial).
    constexpr int kORow = kDv * 2 + 16;
    const uint8_t* obuf = &tile[0][0];
    const int64_t part = (int64_t)row * splits + split;
    uint16_t* dst = splits == 1 ? out + ((int64_t)row * kH + hb) * kDv : ws_o + (part * kH + hb) * kDv;
    // the thread index, taken afresh: the addresses below are rebuilt here
    // rather than held in registers through the whole pipeline
    int t4 = (int)threadIdx.x;
    asm volatile("" : "+v"(t4));
    const int l4 = t4 & 63;
#pragma unroll
    for (int k = 0; k < kHalf / kWaves; ++k) {
        const int h = wave + kWaves * k;
        *reinterpret_cast<uint4*>(dst + (int64_t)h * kDv + 8 * l4) =
            *reinterpret_cast<const uint4*>(obuf + h * kORow + 16 * l4);
    }
    if (t4 < kHalf) {
        const float lsum = l_s[t4];
        const float hl_lse = lsum > 0.f ? (m_s[t4] + __log2f(lsum)) * kLn2 : -INFINITY;
        if (splits == 1) {
            if (lse != nullptr) lse[(int64_t)row * kH + hb + t4] = hl_lse;
        } else {
            ws_lse[part * kH + hb + t4] = hl_lse;
        }
    }
}

// Merge split partials: out = sum_s exp(lse_s - LSE) * O_s, LSE = log sum_s exp(lse_s).
// The partials O_s are bf16.  grid (rows, H/4), block 256: wave w -> head
// 4*blockIdx.y + w, lane -> 8 channels, so every load instruction of a wave
// reads 1 KB of contiguous partials.
__global__ __launch_bounds__(256) void sfa_combine_kernel(const uint16_t* __restrict__ ws_o,
                                                          const float* __restrict__ ws_lse, int splits,
                                                          int H, int Dv, uint16_t* __restrict__ out,
                                                          float* __restrict__ lse) {
    const int row = blockIdx.x;
    const int h = 4 * blockIdx.y + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (h >= H) return;
    // up to kBatch splits (the decode split count) in one round trip: their
    // LSEs and partial rows are all loaded before any is used; more splits
    // take further batches, merged in order with the running maximum fixed
    // by a first pass over the LSEs
    constexpr int kBatch = 4;
    float M = -INFINITY;
    if (splits > kBatch)
        for (int s = 0; s < splits; ++s) M = fmaxf(M, ws_lse[((int64_t)row * splits + s) * H + h]);
    for (int d = 8 * lane; d < Dv; d += 8 * 64) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        float W = 0.f;
        for (int s0 = 0; s0 < splits; s0 += kBatch) {
            uint4 v[kBatch];
            float ls[kBatch];
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                const int s = min(s0 + k, splits - 1);  // in range; weight 0 past the last split
                ls[k] = s0 + k < splits ? ws_lse[((int64_t)row * splits + s) * H + h] : -INFINITY;
                v[k] = *reinterpret_cast<const uint4*>(ws_o + (((int64_t)row * splits + s) * H + h) * Dv + d);
            }
            if (splits <= kBatch) {
#pragma unroll
                for (int k = 0; k < kBatch; ++k) M = fmaxf(M, ls[k]);
            }
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                const float wgt = (M == -INFINITY || ls[k] == -INFINITY) ? 0.f : expf(ls[k] - M);
                W += wgt;
                const uint32_t w4[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] = fmaf(wgt, __uint_as_float(w4[i] << 16), acc[2 * i]);
                    acc[2 * i + 1] = fmaf(wgt, __uint_as_float(w4[i] & 0xffff0000u), acc[2 * i + 1]);
                }
            }
        }
        const float inv = W > 0.f ? 1.f / W : 0.f;
        uint16_t* o = out + ((int64_t)row * H + h) * Dv + d;
        uint32_t w4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w4[i] = pack_bf16x2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
        *reinterpret_cast<uint4*>(o) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
        if (lse != nullptr && lane == 0 && d == 0) lse[(int64_t)row * H + h] = W > 0.f ? M + logf(W) : -INFINITY;
    }
}

// fp32 attention for small shapes: one wave per (head, row); logits of the
// row's valid positions in LDS, two-pass softmax, lanes over value channels.
__global__ __launch_bounds__(64) void sfa_f32_kernel(
    const float* __restrict__ q, const uint8_t* __restrict__ kv, PoolLayout kvl, const int32_t* __restrict__ seq_lens,
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
        const float* k = reinterpret_cast<const float*>(kv + (int64_t)(pr[t] >> 6) * kvl.bs + (pr[t] & 63) * kvl.rs);
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
        for (int t = 0; t < n; ++t)
            acc = fmaf(z[t], reinterpret_cast<const float*>(kv + (int64_t)(pr[t] >> 6) * kvl.bs +
                                                            (pr[t] & 63) * kvl.rs)[d], acc);
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

// The latent pool (and its scales) in the dense layout of its format, in
// bytes: rows, blocks, scale rows, scale blocks.
static bool dense_pool(const AttnLaunch& a) {
    const int64_t drow = a.kv_kind == 1 ? kRowB : kDqk;
    const int64_t dsrow = a.kv_kind == 2 ? kDqk / 32 : a.kv_kind == 3 ? 5 * 4 : 0;
    return a.kvl.rs == drow && a.kvl.bs == 64 * drow &&
           (a.kv_kind == 1 || (a.kvl.srs == dsrow && a.kvl.sbs == 64 * dsrow));
}

int attn_per_split(int top_k, int splits) {
    const int nchunks = (top_k + kCh - 1) / kCh;
    return ((nchunks + splits - 1) / splits) * kCh;
}

// Whether the attention selects its rows' Top-K itself (a.scores set): the
// MLA kernel with a dense pool, rows up to 8192 positions (16 keys per
// thread), and few enough rows that the Top-K kernel, one workgroup per row,
// would leave most compute units idle.  Measured on the decode workloads:
// 8192-position rows save 0.8-2.9 us of a 65-67 us step; 16384-position rows
// (32 keys per thread) save nothing, the longer selection outweighing the
// launch it replaces.
bool attn_fuses_topk(const AttnLaunch& a) {
    if (a.q_dtype == 0 || a.Dqk != kDqk || a.H != kH || a.Dv != kDv) return false;
    if (a.max_seq_len > kThreads * kFusedTopkKpt || (int64_t)a.batch * a.n_q > 256) return false;
    return dense_pool(a);
}

hipError_t launch_sparse_attn(const AttnLaunch& a, hipStream_t st) {
    const int rows = a.batch * a.n_q;
    if (rows == 0) return hipSuccess;
    if (a.q_dtype == 0) {
        const size_t sh = (size_t)a.top_k * (sizeof(float) + sizeof(int));
        hipLaunchKernelGGL(sfa_f32_kernel, dim3(a.H, rows), dim3(64), sh, st, (const float*)a.q,
                           (const uint8_t*)a.kv, a.kvl, a.seq_lens, a.table, a.max_blocks, a.num_blocks, a.n_q,
                           a.max_seq_len, a.indices, a.top_k, a.H, a.Dqk, a.Dv, a.sm_scale, (float*)a.out,
                           a.lse);
        return hipGetLastError();
    }
    const int splits = a.splits;
    const int per = splits == 1 ? a.top_k : attn_per_split(a.top_k, splits);
    const int grid = ((rows + 7) / 8) * 8 * 2 * splits;   // (row, head half, split)
    const float scale_log2 = a.sm_scale * kLog2e;
    uint16_t* ws_o = (uint16_t*)a.ws;
    float* ws_lse = splits == 1 ? nullptr : (float*)(ws_o + (size_t)rows * splits * kH * kDv);
    const bool dense = dense_pool(a);
#define DSA_SFA(KV, D, TK)                                                                                      \
    hipLaunchKernelGGL((sfa_mla_kernel<KV, D, TK>), dim3(grid), dim3(kThreads), 0, st, (const uint16_t*)a.q,    \
                       (const uint8_t*)a.kv, a.kvscale, a.kvl, a.seq_lens, a.table, a.max_blocks, a.num_blocks, \
                       a.n_q, a.max_seq_len, rows, a.indices, a.top_k, per, splits, scale_log2,              \
                       (uint16_t*)a.out, a.lse, ws_o, ws_lse, a.scores, a.ld)
    if (a.scores != nullptr) {  // fused Top-K (attn_fuses_topk holds)
        if (a.kv_kind == 3) DSA_SFA(3, true, kFusedTopkKpt);
        else if (a.kv_kind == 2) DSA_SFA(2, true, kFusedTopkKpt);
        else DSA_SFA(1, true, kFusedTopkKpt);
    } else if (a.kv_kind == 3) {
        if (dense) DSA_SFA(3, true, 0); else DSA_SFA(3, false, 0);
    } else if (a.kv_kind == 2) {
        if (dense) DSA_SFA(2, true, 0); else DSA_SFA(2, false, 0);
    } else {
        if (dense) DSA_SFA(1, true, 0); else DSA_SFA(1, false, 0);
    }
#undef DSA_SFA
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    hipLaunchKernelGGL(sfa_combine_kernel, dim3(rows, kH / 4), dim3(256), 0, st, ws_o, ws_lse, splits, kH, kDv,
                       (uint16_t*)a.out, a.lse);
    return hipGetLastError();
}

size_t attn_ws_bytes(int rows, int top_k, int Dqk, int H, int Dv) {
    const int s = attn_splits(rows, top_k, Dqk);
    if (s == 1) return 0;
    // bf16 partial outputs, then fp32 partial LSEs
    return (size_t)rows * s * H * (sizeof(uint16_t) * (size_t)Dv + sizeof(float));
}

}  // namespace dsa
