// indexer.hip -- Lightning Indexer scoring for gfx950.
//
//   I[r][s] = sum_j w[r][j] * max(0, q[r][j][:] . k[s][:]),  s < L_r
//
// Relevance scoring and the per-head weighted aggregation of the indexer
// ("Day0 Inference Adaptation and Performance Optimization for
// New-Architecture LLMs", §4.1 Indexer Fusion; the ReLU is the per-head
// nonlinearity), reading the paged index-K cache directly through the block
// table ("Day0 Inference Optimization for New Architecture LLMs Based on
// CANN", §2.1).  The quantized path keeps one fp32 scale per 128 elements of
// q and k; scales are positive, so they are taken out of the ReLU:
//   I = s_k[s] * sum_j (w_j * s_q[j]) * max(0, q8_j . k8_s).
//
// The contraction q.K^T runs on MFMA with heads as M, positions as N and the
// index dimension as K; the ReLU-weighted sum over the 64 heads is a
// register epilogue plus two cross-lane swaps.
#include "common.hpp"
#include "kernels.hpp"

namespace dsa {

// --------------------------------------------------------------- fp32 path
// Small fp32 shapes: one thread per (row, position); q and w of the row in LDS.
__global__ __launch_bounds__(64) void indexer_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ w, const uint8_t* __restrict__ kpool, PoolLayout kl,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ table, int max_blocks,
    int64_t num_blocks, int n_q, int max_seq_len, int H, int D, float* __restrict__ scores,
    int64_t ld) {
    extern __shared__ float sh[];  // [H*D] q, then [H] w
    const int r = blockIdx.y, b = r / n_q, i = r % n_q;
    const int L = history_len(clamp_len(seq_lens, b, max_seq_len), n_q, i);
    if ((int)blockIdx.x * 64 >= L) return;  // block-uniform
    for (int t = threadIdx.x; t < H * D; t += 64) sh[t] = q[(int64_t)r * H * D + t];
    for (int t = threadIdx.x; t < H; t += 64) sh[H * D + t] = w[(int64_t)r * H + t];
    __syncthreads();
    const int s = blockIdx.x * 64 + threadIdx.x;
    if (s >= L) return;
    const int64_t p = phys_block(table, max_blocks, b, s / kBlock, num_blocks);
    if (p < 0) {
        scores[(int64_t)r * ld + s] = -INFINITY;
        return;
    }
    const float* k = reinterpret_cast<const float*>(kpool + p * kl.bs + (s % kBlock) * kl.rs);
    float acc = 0.f;
    for (int j = 0; j < H; ++j) {
        float d = 0.f;
        for (int c = 0; c < D; ++c) d = fmaf(sh[j * D + c], k[c], d);
        acc = fmaf(sh[H * D + j], fmaxf(d, 0.f), acc);
    }
    scores[(int64_t)r * ld + s] = acc;
}

// ------------------------------------------------------------- MFMA paths
// Element traits: per-lane operand fragment of one MFMA and the k-steps that
// cover the 128-wide index vector.
struct IdxBf16 {
    using frag = bf16x8;
    static constexpr int KSTEPS = 4;      // 4 x K=32
    static constexpr int FB = 16;         // fragment bytes per lane
    static constexpr int ROW = 256;       // bytes per 128-wide vector
    static constexpr bool SCALED = false;
    static constexpr bool MX = false;
};
struct IdxFp8 {  // e4m3 with one fp32 scale per 128-element vector, applied after the MFMA
    using frag = i32x8;
    static constexpr int KSTEPS = 1;      // 1 x K=128
    static constexpr int FB = 32;
    static constexpr int ROW = 128;
    static constexpr bool SCALED = true;
    static constexpr bool MX = false;
};
struct IdxMx {   // MXFP8: e4m3 with one E8M0 scale per 32 elements, applied inside the MFMA
    using frag = i32x8;
    static constexpr int KSTEPS = 1;
    static constexpr int FB = 32;
    static constexpr int ROW = 128;
    static constexpr bool SCALED = false;
    static constexpr bool MX = true;
};

// sa, sb: this lane's E8M0 block scales of A and B (MXFP8 only).
template <class T>
__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c, int, int) { return mfma_bf16(a, b, c); }
template <class T>
__device__ __forceinline__ f32x4 mma(i32x8 a, i32x8 b, f32x4 c, int sa, int sb) {
    if constexpr (T::MX) return mfma_mx_k128(a, b, c, sa, sb);
    else return mfma_fp8_k128(a, b, c);
}

constexpr int kIdxHeads = 64;  // 4 M-tiles of 16 heads

// Lane's fragment of vector `vec` (ROW bytes each) for k-step ks.  bf16: 16
// bytes at 64ks + 16g, elements [32ks + 8g, +8).  fp8: elements [16g, +16) and
// [64 + 16g, +16), the operand order of the scaled 16x16x128 MFMA.
template <class T>
__device__ __forceinline__ typename T::frag load_frag(const uint8_t* vec, int ks, int g) {
    if constexpr (T::FB == 16) {
        return *reinterpret_cast<const typename T::frag*>(vec + ks * 4 * T::FB + g * T::FB);
    } else {
        const i32x4 lo = *reinterpret_cast<const i32x4*>(vec + 16 * g);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(vec + 64 + 16 * g);
        return typename T::frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
}

// Query fragments and head weights of one row.  Loads are unconditional
// (a row past the end reads row 0 and is zeroed afterwards), so they issue
// back to back.
// MXFP8: qs[mt] is this lane's E8M0 scale of head 16mt + j, k-block g.
template <class T>
__device__ __forceinline__ void load_row_query(const uint8_t* q, const void* q_scale, const float* w,
                                               int64_t row, bool valid, int g, int j,
                                               typename T::frag (&qa)[4][T::KSTEPS], float (&wr)[4][4],
                                               int (&qs)[4]) {
    const int64_t rr = valid ? row : 0;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const uint8_t* v = q + ((rr * kIdxHeads) + 16 * mt + j) * (int64_t)T::ROW;
#pragma unroll
        for (int ks = 0; ks < T::KSTEPS; ++ks) qa[mt][ks] = load_frag<T>(v, ks, g);
        qs[mt] = T::MX ? (int)static_cast<const uint8_t*>(q_scale)[(rr * kIdxHeads + 16 * mt + j) * 4 + g] : 127;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = 16 * mt + 4 * g + i;
            float x = w[rr * kIdxHeads + h];
            if constexpr (T::SCALED) x *= static_cast<const float*>(q_scale)[rr * kIdxHeads + h];
            wr[mt][i] = valid ? x : 0.f;
        }
    }
    if (!valid) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int ks = 0; ks < T::KSTEPS; ++ks) qa[mt][ks] = typename T::frag{};
    }
}

// ReLU-weighted sum over the 64 heads of a 16-position N-tile, where lane
// 16g + j holds D[head 16*mt + 4g + i][pos j].
// max(x, 0) as one signed-integer max on the bits: negative floats (and -0)
// are negative integers.  A float max would also quiet NaNs first (two
// instructions); here a NaN with the sign bit clear passes through.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// This lane's share of the sum: its 16 heads, as four independent partial
// sums (one per M-tile) and a tree.
__device__ __forceinline__ float head_weighted_relu_part(const f32x4 (&acc)[4], const float (&wr)[4][4]) {
    float v[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        v[mt] = wr[mt][0] * relu(acc[mt][0]);
#pragma unroll
        for (int i = 1; i < 4; ++i) v[mt] = fmaf(wr[mt][i], relu(acc[mt][i]), v[mt]);
    }
    return (v[0] + v[1]) + (v[2] + v[3]);
}

// The sums over the four lane groups of four N-tiles' shares at once, each
// group keeping its own N-tile's: lane 16g + j returns N-tile g's sum for
// position j.  Pairs of N-tiles meet in one permlane16 swap (row r keeps
// N-tile r&1 of the pair, the sum of its row pair), then the pairs in one
// permlane32 swap; the additions are those of sum_over_groups, in its order.
__device__ __forceinline__ float pair_sum16(float p0, float p1) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}
__device__ __forceinline__ float pair_sum32(float u01, float u23) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(u01), __float_as_uint(u23), false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// Decode: a sequence's n_q <= NQ rows share every K tile.  Each wave owns TPW
// consecutive 64-position tiles of one sequence and streams them through two
// LDS slots of its own, two tiles in flight while the previous one is scored.
// Everything the kernel reads from global memory beyond the block table
// arrives by DMA (global_load_lds), each instruction one contiguous 1 KB of
// K (or of the queries): fragment loads straight from HBM touch half of 16
// cache lines per instruction, and a plain read in that pattern stays near
// 4 TB/s where contiguous 1 KB reads reach 5.5.  Being invisible to the
// compiler's wait bookkeeping, the DMAs are waited for with hand-counted
// waits; there are no compiler-visible vector loads, whose waits would also
// drain the tiles in flight.  grid (ceil(tiles / (NW*TPW)), batch), block
// 64*NW.
template <class T, int NQ, int TPW, int NW>
__global__ __launch_bounds__(64 * NW) void indexer_decode_kernel(
    const uint8_t* __restrict__ q, const void* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ kpool, const void* __restrict__ kscale, PoolLayout kl,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ table, int max_blocks,
    int64_t num_blocks, int n_q, int max_seq_len, float* __restrict__ scores, int64_t ld) {
    static_assert(NQ <= 2 && NQ <= NW, "decode rows per sequence");
    constexpr int UNITS = T::ROW / 16;                  // 16-byte units per 128-element vector
    constexpr int TILE_BYTES = kBlock * T::ROW;
    constexpr int TILE_K = TILE_BYTES / (16 * kWave);   // 1 KB gathers per K tile (16 or 8)
    constexpr int Q_K = NQ * kIdxHeads * T::ROW / (16 * kWave);  // 1 KB gathers of the queries
    constexpr bool kScaleLine = T::SCALED || T::MX;
    // Unit c of vector v (a query head row or a K position) sits at column
    // c ^ (v % UNITS), an XOR swizzle that keeps the fragment reads free of
    // bank conflicts.
    __shared__ __attribute__((aligned(16))) uint8_t q_s[NQ * kIdxHeads * T::ROW];
    __shared__ __attribute__((aligned(16))) float w_s[NQ][kIdxHeads];
    // fp8: the query scale of each head; MXFP8: its four E8M0 bytes
    __shared__ __attribute__((aligned(16))) float qsc_s[NQ][kIdxHeads];
    __shared__ __attribute__((aligned(16))) uint8_t ktile[NW][2][TILE_BYTES];
    // fp8: the scale of each position of the tile; MXFP8: its four E8M0 bytes
    __shared__ __attribute__((aligned(16))) float kst[NW][2][kBlock];

    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: the table reads are scalar
    const int g = lane >> 4, j = lane & 15;
    const int Lb = clamp_len(seq_lens, b, max_seq_len);
    if ((int)blockIdx.x * NW * TPW * kBlock >= Lb) return;  // block-uniform
    const int tile0 = (blockIdx.x * NW + wave) * TPW;

    // Round trips before the first K tile: the block-table entries (scalar
    // loads; the K addresses depend on them) and, at the same time, the
    // queries, head weights and query scales (DMA, shared by the waves).
    int32_t traw[TPW];  // raw table entries; checked once they have arrived
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int t = tile0 + u;
        traw[u] = table[(int64_t)b * max_blocks + (t < max_blocks ? t : 0)];  // unconditional read
    }
    __builtin_amdgcn_sched_barrier(0);  // the table reads issue first
    int issued = 0;  // vector-memory operations this wave has issued (uniform)
    for (int k = wave; k < Q_K; k += NW) {
        const int U = k * kWave + lane;
        const int v = U / UNITS, col = (U % UNITS) ^ (v % UNITS);
        const int qi = v / kIdxHeads;
        const int64_t rr = (int64_t)b * n_q + (qi < n_q ? qi : 0);
        lds_gather16(q + (rr * kIdxHeads + v % kIdxHeads) * (int64_t)T::ROW + col * 16, lds_addr(q_s) + k * kWave * 16);
        ++issued;
    }
    if (wave < NQ) {  // wave qi brings row qi's head weights and query scales
        const int64_t rr = (int64_t)b * n_q + (wave < n_q ? wave : 0);
        lds_gather4(w + rr * kIdxHeads + lane, lds_addr(&w_s[wave][0]));
        ++issued;
        if constexpr (kScaleLine) {
            lds_gather4(static_cast<const uint8_t*>(q_scale) + (rr * kIdxHeads + lane) * 4, lds_addr(&qsc_s[wave][0]));
            ++issued;
        }
    }
    const int markQ = issued;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < TPW; ++u) asm volatile("" ::"s"(traw[u]));  // all entries arrive in one round trip
    int64_t pt[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int t = tile0 + u;
        const int64_t p = traw[u];
        pt[u] = (t * kBlock < Lb && t < max_blocks && p >= 0 && p < num_blocks) ? p : -1;
    }

    auto gather = [&](int u, int slot) __attribute__((always_inline)) {
        const int64_t p = pt[u] < 0 ? 0 : pt[u];  // an absent block reads block 0 (its scores are -inf)
        const uint8_t* base = kpool + p * kl.bs;
        const uint32_t dst = lds_addr(&ktile[wave][slot][0]);
#pragma unroll
        for (int k = 0; k < TILE_K; ++k) {
            const int U = k * kWave + lane;
            const int row = U / UNITS, col = (U % UNITS) ^ (row % UNITS);
            lds_gather16(base + row * kl.rs + col * 16, dst + k * kWave * 16);
        }
        if constexpr (kScaleLine)  // one dword per position: the fp32 scale or the four E8M0 bytes
            lds_gather4(static_cast<const uint8_t*>(kscale) + p * kl.sbs + lane * kl.srs,
                        lds_addr(&kst[wave][slot][0]));
        issued += TILE_K + (kScaleLine ? 1 : 0);
    };
    // markA, markB: `issued` right after the gathers of tiles u and u+1
    gather(0, 0);
    int markA = issued, markB = issued;
    if (TPW > 1) {
        gather(1, 1);
        markB = issued;
    }

    wait_vmcnt(issued - markQ);  // this wave's query parts have landed (operations complete in order)
    sync_lds();                  // ... and every wave's
    typename T::frag qa[NQ][4][T::KSTEPS];
    float wr[NQ][4][4];
    int qsx[NQ][4];  // MXFP8: E8M0 scale of head 16mt + j, k-block g
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
        const bool valid = qi < n_q;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int v = qi * kIdxHeads + 16 * mt + j;
            const uint8_t* rowp = q_s + v * T::ROW;
#pragma unroll
            for (int ks = 0; ks < T::KSTEPS; ++ks) {
                if constexpr (T::FB == 16) {
                    qa[qi][mt][ks] = *reinterpret_cast<const bf16x8*>(rowp + ((4 * ks + g) ^ (v % UNITS)) * 16);
                } else {  // elements [16g, +16) and [64 + 16g, +16) (the MFMA's operand order)
                    const i32x4 lo = *reinterpret_cast<const i32x4*>(rowp + (g ^ (v % UNITS)) * 16);
                    const i32x4 hi = *reinterpret_cast<const i32x4*>(rowp + ((4 + g) ^ (v % UNITS)) * 16);
                    qa[qi][mt][ks] = typename T::frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                }
            }
            qsx[qi][mt] = T::MX ? (int)reinterpret_cast<const uint8_t*>(&qsc_s[qi][0])[(16 * mt + j) * 4 + g] : 127;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int h = 16 * mt + 4 * g + i;
                float x = w_s[qi][h];
                if constexpr (T::SCALED) x *= qsc_s[qi][h];
                wr[qi][mt][i] = valid ? x : 0.f;
            }
        }
    }

#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int slot = u & 1;
        const int s0 = (tile0 + u) * kBlock;
        wait_vmcnt(issued - markA);  // tile u is in this wave's slot (operations complete in order)
        if (s0 < Lb) {
            // each N-tile leaves this lane's share per row; after N-tiles 1
            // and 3 the shares of two N-tiles are reduced across the lane
            // groups, and lane 16g + j keeps N-tile g's sum, which is
            // position 16g + j
            float sel[NQ], shr[NQ][2], u01[NQ];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int prow = 16 * nt + j;
                const uint8_t* rowp = &ktile[wave][slot][prow * T::ROW];
                const int kx = T::MX ? (int)reinterpret_cast<const uint8_t*>(&kst[wave][slot][0])[prow * 4 + g] : 127;
                typename T::frag kf[T::KSTEPS];
#pragma unroll
                for (int ks = 0; ks < T::KSTEPS; ++ks) {
                    if constexpr (T::FB == 16) {
                        kf[ks] = *reinterpret_cast<const bf16x8*>(rowp + ((4 * ks + g) ^ (prow % UNITS)) * 16);
                    } else {
                        const i32x4 lo = *reinterpret_cast<const i32x4*>(rowp + (g ^ (prow % UNITS)) * 16);
                        const i32x4 hi = *reinterpret_cast<const i32x4*>(rowp + ((4 + g) ^ (prow % UNITS)) * 16);
                        kf[ks] = typename T::frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    }
                }
#pragma unroll
                for (int qi = 0; qi < NQ; ++qi) {
                    f32x4 acc[4];
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {
                        acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < T::KSTEPS; ++ks)
                            acc[mt] = mma<T>(qa[qi][mt][ks], kf[ks], acc[mt], qsx[qi][mt], kx);
                    }
                    shr[qi][nt & 1] = head_weighted_relu_part(acc, wr[qi]);
                    if (nt == 1) u01[qi] = pair_sum16(shr[qi][0], shr[qi][1]);
                    if (nt == 3) sel[qi] = pair_sum32(u01[qi], pair_sum16(shr[qi][0], shr[qi][1]));
                }
            }
            // one 256-byte store per row: lane l scores position s0 + l
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi) {
                if (qi >= n_q) continue;  // uniform
                const int Lr = history_len(Lb, n_q, qi);
                float v = sel[qi];
                if constexpr (T::SCALED) v *= kst[wave][slot][lane];
                if (pt[u] < 0) v = -INFINITY;  // absent block: every position scores -inf
                if (s0 + lane < Lr) scores[((int64_t)b * n_q + qi) * ld + s0 + lane] = v;
                issued += s0 < Lr;  // the store issues when lane 0 is active
            }
        }
        if (u + 2 < TPW) {
            // the slot's fragment reads have returned before it is refilled
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            gather(u + 2, slot);
        }
        markA = markB;
        markB = issued;
    }
}

// Prefill (many query rows per sequence): 8 waves x 2 rows = 16 rows per row
// block; the block's K tiles are gathered straight into a 6-tile LDS ring and
// shared by all 16 rows, scored two tiles per barrier.  Causal load skew is balanced by pairing row block x
// with row block NB-1-x in one workgroup, the head-tail pairing the pages use
// across devices ("Day0 Inference Adaptation and Performance Optimization for
// New-Architecture LLMs", §6.2 Zigzag Layout), applied here across the GPU's
// compute units.  grid (ceil(NB/2), batch), block 512.
constexpr int kIdxRing = 6;

template <class T>
__global__ __launch_bounds__(512) void indexer_prefill_kernel(
    const uint8_t* __restrict__ q, const void* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ kpool, const void* __restrict__ kscale, PoolLayout kl,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ table, int max_blocks,
    int64_t num_blocks, int n_q, int max_seq_len, float* __restrict__ scores, int64_t ld) {
    constexpr int UNITS = T::ROW / 16;              // 16-byte units per K row
    constexpr int TILE_BYTES = kBlock * T::ROW;
    constexpr int TILE_K = TILE_BYTES / (16 * kWave);  // wave-instructions per tile (16 or 8)
    __shared__ __attribute__((aligned(16))) uint8_t ktile[kIdxRing][TILE_BYTES];
    // fp8: the scale of each position of the tile; MXFP8: its four E8M0 bytes (k-blocks 0..3)
    __shared__ __attribute__((aligned(16))) float kst[kIdxRing][kBlock];

    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, j = lane & 15;
    const int Lb = clamp_len(seq_lens, b, max_seq_len);
    const int NB = (n_q + 15) / 16;
    const int rbs[2] = {(int)blockIdx.x, NB - 1 - (int)blockIdx.x};
    const int npass = (rbs[1] > rbs[0]) ? 2 : 1;
    // gathers issued per tile by this wave: K units (+ the scale line, wave 0, fp8)
    constexpr bool kScaleLine = T::SCALED || T::MX;  // the tile's scales are gathered too
    const int per_tile = (TILE_K - wave + 7) / 8 + ((kScaleLine && wave == 0) ? 1 : 0);

    // Vector-memory operations this wave has issued (uniform), so that the wait
    // for a tile counts exactly the operations issued after its gathers.
    int issued = 0;
    // Raw block-table entries of tiles 64m .. 64m+63, gathered by each wave
    // into its own LDS window (clamped columns; validated when used).  Window
    // m+1 is gathered when tile 64m is staged, 64 tiles before it is needed;
    // the tile waits cover it, since operations complete in order.  When tile
    // 64m is staged the wave also reads window m into a register (lane l holds
    // tile 64m + l), so each later tile's entry is one lane read.
    __shared__ int tabw[8][2][kWave];
    auto tab_fetch = [&](int m) __attribute__((always_inline)) {
        const int j_ = min(kWave * m + lane, max_blocks - 1);
        lds_gather4(table + (int64_t)b * max_blocks + j_, lds_addr(&tabw[wave][m & 1][0]));
        ++issued;
    };

    // Gather tile t into ring slot `buf`: unit U of the tile (row U/UNITS, column
    // U%UNITS) receives global column (U%UNITS) ^ (row % UNITS), an XOR swizzle
    // that keeps the column reads below bank-conflict free.  The wave gathers
    // units U = 64k + lane for k = wave, wave + 8, at the same offsets in every
    // tile.  Absent blocks read block 0 and are flagged in a bit mask that
    // every wave keeps alike (each stages every tile); their scores are -inf.
    constexpr int KPW = (TILE_K + 7) / 8;
    int64_t goff[KPW];
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
        const int U = (wave + 8 * i) * kWave + lane;
        const int row = U / UNITS, col = (U % UNITS) ^ (row % UNITS);
        goff[i] = row * kl.rs + col * 16;
    }
    int win = 0;        // the table window of the tiles being staged
    uint32_t okm = 0u;  // bit s: ring slot s holds a present block
    auto stage = [&](int t, int buf) __attribute__((always_inline)) {
        if ((t & 63) == 0) {
            tab_fetch((t >> 6) + 1);
            win = tabw[wave][(t >> 6) & 1][lane];
        }
        int64_t p = __builtin_amdgcn_readlane(win, t & 63);
        if (t >= max_blocks || p < 0 || p >= num_blocks) p = -1;  // absent block
        okm = (okm & ~(1u << buf)) | ((p >= 0 ? 1u : 0u) << buf);
        if (p < 0) p = 0;
        const uint8_t* base = kpool + p * kl.bs;
        const uint32_t dst = lds_addr(&ktile[buf][0]);
#pragma unroll
        for (int i = 0; i < KPW; ++i) {
            const int k = wave + 8 * i;
            if (k < TILE_K) lds_gather16(base + goff[i], dst + k * kWave * 16);
        }
        if constexpr (kScaleLine) {  // one dword per position: the fp32 scale or the four E8M0 bytes
            if (wave == 0)
                lds_gather4(static_cast<const uint8_t*>(kscale) + p * kl.sbs + lane * kl.srs,
                            lds_addr(&kst[buf][0]));
        }
        issued += per_tile;
    };

    for (int pass = 0; pass < npass; ++pass) {
        const int rb = rbs[pass];
        typename T::frag qa[2][4][T::KSTEPS];
        float wr[2][4][4];
        int qsx[2][4];
        int Lr[2];
        for (int qi = 0; qi < 2; ++qi) {
            const int i = rb * 16 + wave * 2 + qi;
            const bool valid = i < n_q;
            Lr[qi] = valid ? history_len(Lb, n_q, i) : 0;
            load_row_query<T>(q, q_scale, w, (int64_t)b * n_q + i, valid, g, j, qa[qi], wr[qi], qsx[qi]);
        }
        const int last = (rb * 16 + 15 < n_q - 1) ? rb * 16 + 15 : n_q - 1;
        const int Lmax = history_len(Lb, n_q, last);
        const int ntiles = (Lmax + kBlock - 1) / kBlock;
        // retire the query loads before the ring starts (known to the compiler, so
        // it places no wait for them inside the tile loop)
        __builtin_amdgcn_s_waitcnt(0x0f70);

        if (ntiles > 0) {
            tab_fetch(0);
            wait_vmcnt<0>();
        }
        // Tiles are scored in pairs (t, t+1), t even, with one wait and one
        // barrier per pair; the two pairs after it are in flight meanwhile.
        // markA: `issued` right after the gathers of the pair scored next;
        // markB: of the pair after it.
        static_assert(kIdxRing == 6, "two pairs of tiles are in flight ahead of the pair scored");
        if (ntiles > 0) stage(0, 0);
        if (ntiles > 1) stage(1, 1);
        int markA = issued;
        if (ntiles > 2) stage(2, 2);
        if (ntiles > 3) stage(3, 3);
        int markB = issued;
        for (int t = 0; t < ntiles; t += 2) {
            wait_vmcnt(issued - markA);  // tiles t and t+1 have landed (operations complete in order)
            sync_lds();  // ... for every wave; the slots of tiles t-2 and t-1 are free
            if (t + 4 < ntiles) stage(t + 4, (t + 4) % kIdxRing);
            if (t + 5 < ntiles) stage(t + 5, (t + 5) % kIdxRing);
            markA = markB;
            markB = issued;
            // tiles of the pair that this wave scores: none, t, or t and t+1
            const int Lw = max(Lr[0], Lr[1]);
            const int ntw = t * kBlock >= Lw ? 0 : (t + 1 < ntiles && (t + 1) * kBlock < Lw ? 2 : 1);
            if (ntw > 0) {
                // per tile eight steps k = (N-tile k/2, row k%2): 16 MFMAs, then the
                // ReLU-weighted head sum (VALU).  A wave's own MFMAs and VALU
                // work do not overlap; waves w and w+4 share a SIMD, and waves
                // 4..7 run each step's sum one step late (across the two tiles
                // of the pair), so that one wave's sum runs under the other's
                // MFMAs.  MFMA steps run at raised wave priority, so the matrix
                // core is fed first.
                typename T::frag kf[2][T::KSTEPS];
                int ksx[2];  // MXFP8: E8M0 scale of position 16nt + j, k-block g
                auto read_k = [&](int buf, int nt, typename T::frag (&f)[T::KSTEPS], int& kx) __attribute__((always_inline)) {
                    const int prow = 16 * nt + j;
                    const uint8_t* rowp = &ktile[buf][prow * T::ROW];
                    kx = T::MX ? (int)reinterpret_cast<const uint8_t*>(&kst[buf][0])[prow * 4 + g] : 127;
#pragma unroll
                    for (int ks = 0; ks < T::KSTEPS; ++ks) {
                        if constexpr (T::FB == 16) {
                            const int u = (4 * ks + g) ^ (prow % UNITS);
                            f[ks] = *reinterpret_cast<const bf16x8*>(rowp + u * 16);
                        } else {  // elements [16g, +16) and [64 + 16g, +16) (the MFMA's operand order)
                            const int u0 = g ^ (prow % UNITS), u1 = (4 + g) ^ (prow % UNITS);
                            const i32x4 lo = *reinterpret_cast<const i32x4*>(rowp + u0 * 16);
                            const i32x4 hi = *reinterpret_cast<const i32x4*>(rowp + u1 * 16);
                            f[ks] = typename T::frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        }
                    }
                };
                auto mfma_step = [&](int u, int k, f32x4 (&acc)[4]) __attribute__((always_inline)) {
                    __builtin_amdgcn_sched_barrier(0);
                    __builtin_amdgcn_s_setprio(2);
                    __builtin_amdgcn_sched_barrier(0);
                    const int nt = k >> 1, qi = k & 1;
                    if (qi == 0) read_k((t + u) % kIdxRing, nt, kf[nt & 1], ksx[nt & 1]);
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {
                        acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < T::KSTEPS; ++ks)
                            acc[mt] = mma<T>(qa[qi][mt][ks], kf[nt & 1][ks], acc[mt], qsx[qi][mt], ksx[nt & 1]);
                    }
                };
                // step k leaves this lane's share of row k%2, N-tile k/2; after
                // N-tiles 1 and 3 the shares of two N-tiles are reduced across
                // the lane groups, and lane 16g + j keeps N-tile g's sum, which
                // is position 16g + j
                float sel0 = 0.f, sel1 = 0.f;
                float sh[2][2], u01[2];  // shares of the pending N-tile pair; pair sums of N-tiles 0, 1
                auto sum_step = [&](int k, const f32x4 (&acc)[4]) __attribute__((always_inline)) {
                    __builtin_amdgcn_sched_barrier(0);
                    __builtin_amdgcn_s_setprio(0);
                    __builtin_amdgcn_sched_barrier(0);
                    const int nt = k >> 1, qi = k & 1;
                    sh[qi][nt & 1] = head_weighted_relu_part(acc, wr[qi]);
                    if (nt == 1) u01[qi] = pair_sum16(sh[qi][0], sh[qi][1]);
                    if (nt == 3) {
                        const float v = pair_sum32(u01[qi], pair_sum16(sh[qi][0], sh[qi][1]));
                        if (qi) sel1 = v; else sel0 = v;
                    }
                };
                // one 256-byte store per row: lane l scores position s0 + l
                auto store = [&](int u) __attribute__((always_inline)) {
                    const int tt = t + u, buf = tt % kIdxRing, s0 = tt * kBlock;
                    const bool ok = (okm >> buf) & 1u;
#pragma unroll
                    for (int qi = 0; qi < 2; ++qi) {
                        float v = qi ? sel1 : sel0;
                        if constexpr (T::SCALED) v *= kst[buf][lane];
                        if (!ok) v = -INFINITY;
                        const int64_t row = (int64_t)b * n_q + rb * 16 + wave * 2 + qi;
                        if (s0 + lane < Lr[qi]) scores[row * ld + s0 + lane] = v;
                        issued += s0 < Lr[qi];  // the store issues when lane 0 is active
                    }
                };
                f32x4 acc[2][4];
                if (wave < 4) {
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        if (u < ntw) {
#pragma unroll
                            for (int k = 0; k < 8; ++k) {
                                mfma_step(u, k, acc[0]);
                                sum_step(k, acc[0]);
                            }
                            store(u);
                        }
                    }
                } else {
                    // the first tile's stores wait for the second tile's
                    // second MFMA step, where no K fragments are held
                    mfma_step(0, 0, acc[0]);
#pragma unroll
                    for (int k = 1; k < 8; ++k) {
                        mfma_step(0, k, acc[k & 1]);
                        sum_step(k - 1, acc[(k - 1) & 1]);
                    }
                    if (ntw == 2) {
                        mfma_step(1, 0, acc[0]);
                        sum_step(7, acc[1]);
                        mfma_step(1, 1, acc[1]);
                        store(0);
                        sum_step(0, acc[0]);
#pragma unroll
                        for (int k = 2; k < 8; ++k) {
                            mfma_step(1, k, acc[k & 1]);
                            sum_step(k - 1, acc[(k - 1) & 1]);
                        }
                        sum_step(7, acc[1]);
                        store(1);
                    } else {
                        sum_step(7, acc[1]);
                        store(0);
                    }
                }
            }
        }
        sync_lds();  // ring slots are reused by the next pass
    }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_indexer(const IndexerLaunch& a, hipStream_t st) {
    const int rows = a.batch * a.n_q;
    if (rows == 0 || a.max_seq_len == 0) return hipSuccess;
    if (a.dtype == 0) {  // f32
        dim3 grid((a.max_seq_len + 63) / 64, rows);
        size_t sh = sizeof(float) * (size_t)(a.H * a.D + a.H);
        hipLaunchKernelGGL(indexer_f32_kernel, grid, dim3(64), sh, st, (const float*)a.q, a.w,
                           (const uint8_t*)a.kpool, a.kl, a.seq_lens, a.table, a.max_blocks, a.num_blocks,
                           a.n_q, a.max_seq_len, a.H, a.D, a.scores, a.ld);
        return hipGetLastError();
    }
    if (a.n_q <= 2) {
        // Each wave streams TPW consecutive tiles with two in flight.  One
        // row: 4 waves per workgroup and the longest run that still gives 256
        // workgroups, up to 8 tiles of fp8 keys (8 KB each) or 4 of bf16 (16
        // KB).  Two rows: 3 waves of 4 tiles (the second row's queries take
        // LDS that a fourth wave's slots would need).
        const int tiles = (a.max_seq_len + kBlock - 1) / kBlock;
        int tpw = 4;
        if (a.n_q == 1) {
            tpw = a.dtype == 1 ? 4 : 8;
            while (tpw > 2 && (int64_t)((tiles + 4 * tpw - 1) / (4 * tpw)) * a.batch < 256) tpw /= 2;
        }
#define DSA_DEC(T, NQ, TPW, NW)                                                                  \
    hipLaunchKernelGGL((indexer_decode_kernel<T, NQ, TPW, NW>),                                  \
                       dim3((tiles + NW * TPW - 1) / (NW * TPW), a.batch), dim3(64 * NW), 0, st, \
                       (const uint8_t*)a.q, a.q_scale, a.w, (const uint8_t*)a.kpool, a.kscale,   \
                       a.kl, a.seq_lens, a.table, a.max_blocks, a.num_blocks, a.n_q, a.max_seq_len, \
                       a.scores, a.ld)
#define DSA_DEC1(T)                               \
    if (tpw == 8) DSA_DEC(T, 1, 8, 4);            \
    else if (tpw == 4) DSA_DEC(T, 1, 4, 4);       \
    else DSA_DEC(T, 1, 2, 4);
        if (a.dtype == 2) {
            if (a.n_q == 1) { DSA_DEC1(IdxFp8) } else DSA_DEC(IdxFp8, 2, 4, 3);
        } else if (a.dtype == 3) {
            if (a.n_q == 1) { DSA_DEC1(IdxMx) } else DSA_DEC(IdxMx, 2, 4, 3);
        } else {
            if (a.n_q == 1) { DSA_DEC1(IdxBf16) } else DSA_DEC(IdxBf16, 2, 4, 3);
        }
#undef DSA_DEC1
#undef DSA_DEC
        return hipGetLastError();
    }
    const int NB = (a.n_q + 15) / 16;
    dim3 grid((NB + 1) / 2, a.batch);
#define DSA_PRE(T)                                                                                   \
    hipLaunchKernelGGL((indexer_prefill_kernel<T>), grid, dim3(512), 0, st, (const uint8_t*)a.q,    \
                       a.q_scale, a.w, (const uint8_t*)a.kpool, a.kscale, a.kl, a.seq_lens, a.table, \
                       a.max_blocks, a.num_blocks, a.n_q, a.max_seq_len, a.scores, a.ld)
    if (a.dtype == 2) DSA_PRE(IdxFp8);
    else if (a.dtype == 3) DSA_PRE(IdxMx);
    else DSA_PRE(IdxBf16);
#undef DSA_PRE
    return hipGetLastError();
}

}  // namespace dsa
