// topk.hip -- exact per-row Top-K selection for gfx950.
//
// Keeps the k_r = min(top_k, L_r) highest-scoring history positions of each
// row ("Day0 Inference Adaptation and Performance Optimization for
// New-Architecture LLMs", §4.1, the top-k step of the indexer; only the set
// matters downstream, §5.1).  Ties go to the lowest position and the output
// is ascending, padded with -1.
//
// Method: scores map to order-preserving 32-bit keys (-0.0 folded into
// +0.0; key 0 marks an empty slot, see score_key); an MSB-first radix select
// with LDS histograms finds the k-th largest key T and how many keys equal to
// T are needed; every key > T and the first needed keys == T are kept, in
// position order.  One workgroup per
// row at a time, the rows taken from the last (in a causal prefill, the
// longest) down.
// Three forms:
//   * rows up to 32768 positions: the keys stay in registers (8, 16 or 32
//     per thread of a 1024-thread workgroup), three digit passes;
//   * longer rows: a top_k per 16384-position segment into a candidate
//     workspace, then the same register-resident selection over the
//     candidates;
//   * otherwise (no workspace): the keys are re-read from memory in four
//     8-bit passes.
#include "common.hpp"
#include "kernels.hpp"

namespace dsa {

// Order-preserving key of a score, never 0: the one float that would map to 0
// (the NaN with every bit set; NaN has no specified order) shares key 1 with
// its neighbour, so 0 is free to mark an empty slot.  An empty slot's key is
// below every score's, so as long as a row has top_k real keys, empty slots
// never reach the k-th largest key and can sit in the histograms unnoticed.
__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u << 1) == 0u) u = 0u;  // -0.0 == +0.0
    const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return k > 1u ? k : 1u;
}

template <int NT, bool CACHE>
__global__ __launch_bounds__(NT) void topk_kernel(const float* __restrict__ scores, int64_t ld,
                                                  const int32_t* __restrict__ seq_lens, int n_q,
                                                  int max_seq_len, int rows, int top_k,
                                                  int32_t* __restrict__ indices) {
    constexpr int NW = NT / kWave;
    extern __shared__ uint32_t keys[];  // [max_seq_len] when CACHE
    __shared__ uint32_t hist[256];
    __shared__ uint32_t cut_digit, cut_above;
    __shared__ int wave_cnt[2][NW];

    const int r = rows - 1 - (int)blockIdx.x;
    const int b = r / n_q, i = r % n_q;
    const int L = history_len(clamp_len(seq_lens, b, max_seq_len), n_q, i);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int32_t* out = indices + (int64_t)r * top_k;
    const float* row = scores + (int64_t)r * ld;

    if (L <= top_k) {  // keep the whole history
        for (int t = tid; t < top_k; t += NT) out[t] = t < L ? t : -1;
        return;
    }

    auto key_at = [&](int s) -> uint32_t {
        if constexpr (CACHE) return keys[s];
        else return score_key(row[s]);
    };

    uint32_t prefix = 0u, mask = 0u, krem = (uint32_t)top_k;
    if constexpr (CACHE) {
        // stage the row's keys in LDS; the unrolled loop issues its loads back to back
#pragma unroll 8
        for (int s = tid; s < L; s += NT) keys[s] = score_key(row[s]);
    }
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int t = tid; t < 256; t += NT) hist[t] = 0u;
        __syncthreads();
#pragma unroll 8
        for (int s = tid; s < L; s += NT) {
            const uint32_t k = key_at(s);
            if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (wave == 0) {
            // suffix counts S(d) = #keys with digit >= d; the cut digit D has
            // S(D) >= krem > S(D+1).
            const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1];
            const uint32_t h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
            const uint32_t tot = h0 + h1 + h2 + h3;
            uint32_t T = tot;
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t o = __shfl_down(T, off, 64);
                if (lane + off < 64) T += o;
            }
            const uint32_t above = T - tot;
            const uint32_t S3 = above + h3, S2 = S3 + h2, S1 = S2 + h1, S0 = S1 + h0;
            if (S3 >= krem && above < krem) { cut_digit = 4 * lane + 3; cut_above = above; }
            if (S2 >= krem && S3 < krem) { cut_digit = 4 * lane + 2; cut_above = S3; }
            if (S1 >= krem && S2 < krem) { cut_digit = 4 * lane + 1; cut_above = S2; }
            if (S0 >= krem && S1 < krem) { cut_digit = 4 * lane; cut_above = S1; }
        }
        __syncthreads();
        prefix |= cut_digit << shift;
        mask |= 255u << shift;
        krem -= cut_above;
    }
    // prefix is the k-th largest key; krem keys equal to it are taken, lowest first.
    const uint32_t T = prefix;
    int n_sel = 0, n_eq = 0, par = 0;
    for (int base = 0; base < L && n_sel < top_k; base += NT, par ^= 1) {
        const int s = base + tid;
        const uint32_t k = s < L ? key_at(s) : 0u;
        const bool gt = s < L && k > T, eq = s < L && k == T;
        const uint64_t meq = ballot(eq);
        if (lane == 0) wave_cnt[par][wave] = __popcll(meq);
        __syncthreads();
        int eq_before = 0, eq_tot = 0;
        for (int w = 0; w < NW; ++w) {
            const int c = wave_cnt[par][w];
            eq_before += w < wave ? c : 0;
            eq_tot += c;
        }
        const int eq_rank = n_eq + eq_before + lanes_below(meq);
        const bool sel = gt || (eq && eq_rank < (int)krem);
        const uint64_t msel = ballot(sel);
        __syncthreads();  // all reads of wave_cnt[par] done
        if (lane == 0) wave_cnt[par][wave] = __popcll(msel);
        __syncthreads();
        int sel_before = 0, sel_tot = 0;
        for (int w = 0; w < NW; ++w) {
            const int c = wave_cnt[par][w];
            sel_before += w < wave ? c : 0;
            sel_tot += c;
        }
        const int slot = n_sel + sel_before + lanes_below(msel);
        if (sel && slot < top_k) out[slot] = s;
        n_sel += sel_tot;
        n_eq += eq_tot;
    }
}

// Register-resident selection by one 1024-thread workgroup over up to
// 1024 * KPT slots: thread t holds the keys of slots KPT*t .. KPT*t + KPT - 1
// (key 0 for an empty slot), so the keys are read from memory once.  The MSB-first radix select uses digits of 12, 10 and
// 10 bits (one LDS histogram per pass, bins owned by threads for the suffix
// scan); the k-th largest key T and the number of ties to keep follow, and one
// block scan of the per-thread counts gives every kept slot its output place,
// lowest slot first among equal keys.  emit(place, q) writes kept slot
// KPT*t + q.  Exactly `top_k` slots are kept (callers guarantee that at least
// top_k slots are not empty).  Empty slots are left out of the first
// histogram only to spare one bin the atomic traffic; the later passes and
// the final comparisons need no test, since key 0 lies below the cut.
constexpr int kSelThreads = 1024;
struct SelectShared {
    uint32_t hist[4096];
    uint32_t wsum[kSelThreads / 64] __attribute__((aligned(16)));
    uint32_t cut_digit, cut_above;
};

// emit(place, q) takes a run-time q: a thread walks its kept slots as the set
// bits of a mask, as many steps as it keeps.
template <int KPT, class Emit>
__device__ __forceinline__ void block_select(SelectShared& sh, const uint32_t (&key)[KPT], int top_k,
                                             Emit&& emit) {
    constexpr int NT = kSelThreads, NW = NT / kWave;
    // the wave index is uniform across the wave; saying so keeps the per-wave
    // comparisons below scalar instead of 64-bit lane masks held in registers
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    auto wsum_where = [&](auto pick) -> uint32_t {  // sum of the per-wave totals of the waves w with pick(w)
        uint32_t t = 0u;
#pragma unroll
        for (int q = 0; q < NW / 4; ++q) {
            const uint4 v = reinterpret_cast<const uint4*>(sh.wsum)[q];
            t += (pick(4 * q) ? v.x : 0u) + (pick(4 * q + 1) ? v.y : 0u) + (pick(4 * q + 2) ? v.z : 0u) +
                 (pick(4 * q + 3) ? v.w : 0u);
        }
        return t;
    };
    for (int t = tid; t < 4096; t += NT) sh.hist[t] = 0u;
    __syncthreads();

    uint32_t prefix = 0u, mask = 0u, krem = (uint32_t)top_k;
    auto pass = [&](int shift, int bits, bool first) {
        const uint32_t nb = 1u << bits, dm = nb - 1u;
#pragma unroll
        for (int q = 0; q < KPT; ++q)
            if (first ? key[q] != 0u : (key[q] & mask) == prefix) atomicAdd(&sh.hist[(key[q] >> shift) & dm], 1u);
        __syncthreads();
        // thread t owns bins [per*t, per*t + per); its counts are read, cleared
        // for the next pass, and scanned from the top digit down.
        const int per = (int)nb / NT;  // 4 or 1
        uint32_t cnt[4] = {0u, 0u, 0u, 0u}, own = 0u;
        for (int k = 0; k < per; ++k) {
            cnt[k] = sh.hist[per * tid + k];
            sh.hist[per * tid + k] = 0u;
            own += cnt[k];
        }
        const uint32_t P = wave_scan_incl(own);                    // lanes <= this one
        const uint32_t wtot = __builtin_amdgcn_readlane(P, kWave - 1);
        if (lane == 0) sh.wsum[wave] = wtot;
        __syncthreads();
        // keys in higher bins: later lanes of this wave, then later waves
        const uint32_t above = (wtot - P) + wsum_where([&](int w) { return w > wave; });
        // S(d) = keys with digit >= d; the cut digit D has S(D) >= krem > S(D+1)
        if (above < krem && above + own >= krem) {
            uint32_t sfx = above;
            for (int k = per - 1; k >= 0; --k) {
                if (sfx + cnt[k] >= krem) {
                    sh.cut_digit = (uint32_t)(per * tid + k);
                    sh.cut_above = sfx;
                    break;
                }
                sfx += cnt[k];
            }
        }
        __syncthreads();
        prefix |= sh.cut_digit << shift;
        mask |= dm << shift;
        krem -= sh.cut_above;
    };
    pass(20, 12, true);
    pass(10, 10, false);
    pass(0, 10, false);

    // prefix is the k-th largest key; krem keys equal to it are taken, lowest first.
    const uint32_t T = prefix;
    // this thread's slots above and at T, as bit masks (each comparison is
    // made once: held as lane masks, they would not fit the scalar registers)
    uint32_t gtm = 0u, eqm = 0u;
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
        gtm |= key[q] > T ? (1u << q) : 0u;
        eqm |= key[q] == T ? (1u << q) : 0u;
    }
    const uint32_t gt = (uint32_t)__builtin_popcount(gtm), eq = (uint32_t)__builtin_popcount(eqm);
    const uint32_t packed = (gt << 16) | eq;  // both totals stay below 2^16
    const uint32_t incl = wave_scan_incl(packed);
    if (lane == kWave - 1) sh.wsum[wave] = incl;
    __syncthreads();
    const uint32_t excl = (incl - packed) + wsum_where([&](int w) { return w < wave; });
    const uint32_t gt_before = excl >> 16, eq_before = excl & 0xffffu;
    int place = (int)(gt_before + min(eq_before, krem));
    // the lowest krem - eq_before of this thread's keys equal to T are kept
    uint32_t take = eq_before < krem ? krem - eq_before : 0u;
    uint32_t sel = gtm;
    while (take > 0u && eqm != 0u) {
        sel |= eqm & (0u - eqm);
        eqm &= eqm - 1u;
        --take;
    }
    while (sel != 0u) {  // ascending slot order
        emit(place++, __builtin_ctz(sel));
        sel &= sel - 1u;
    }
}

// Keys of `n` consecutive scores starting at row[base] (n <= KPT; the slots
// from n on are empty), vector loads when the whole run is present and aligned.
template <int KPT>
__device__ __forceinline__ void load_keys(const float* row, int base, int n, bool vec, uint32_t (&key)[KPT]) {
    if (vec && n == KPT) {
#pragma unroll
        for (int q = 0; q < KPT / 4; ++q) {
            const float4 v = *reinterpret_cast<const float4*>(row + base + 4 * q);
            key[4 * q] = score_key(v.x);
            key[4 * q + 1] = score_key(v.y);
            key[4 * q + 2] = score_key(v.z);
            key[4 * q + 3] = score_key(v.w);
        }
    } else {
#pragma unroll
        for (int q = 0; q < KPT; ++q) key[q] = q < n ? score_key(row[base + q]) : 0u;
    }
}

// Rows up to 1024 * KPT positions.  Workgroups are persistent: workgroup b
// takes rows b, b + G, b + 2G, ... counted from the last (longest) row.
template <int KPT>
__global__ __launch_bounds__(kSelThreads) void topk_reg_kernel(const float* __restrict__ scores, int64_t ld,
                                                               const int32_t* __restrict__ seq_lens, int n_q,
                                                               int max_seq_len, int rows, int top_k, bool vec,
                                                               int32_t* __restrict__ indices) {
    __shared__ SelectShared sh;
    const int tid = threadIdx.x;
    const int base = KPT * tid;
    for (int i = (int)blockIdx.x; i < rows; i += (int)gridDim.x) {
        const int r = rows - 1 - i;
        const int L = history_len(clamp_len(seq_lens, r / n_q, max_seq_len), n_q, r % n_q);
        int32_t* out = indices + (int64_t)r * top_k;
        if (L <= top_k) {  // keep the whole history
            for (int t = tid; t < top_k; t += kSelThreads) out[t] = t < L ? t : -1;
            continue;  // workgroup-uniform; no shared memory was touched
        }
        const int nv = min(max(L - base, 0), KPT);  // valid keys of this thread (a prefix)
        uint32_t key[KPT];
        load_keys<KPT>(scores + (int64_t)r * ld, base, nv, vec, key);
        block_select<KPT>(sh, key, top_k, [&](int place, int q) { out[place] = base + q; });
        __syncthreads();  // the shared histogram and scan words are reused by the next row
    }
}

// Rows longer than the register-resident kernel takes: stage 1 keeps the top_k
// of every 16384-position segment (all of a shorter segment) as ascending
// positions in cand[row][segment][top_k] (-1 padded); the row's top_k is
// contained in the union.  Stage 2 selects from those candidates, which are
// in ascending position order, so the lowest-position rule for equal scores
// carries over.  grid (segments, rows) and (rows).
constexpr int kSegLen = kSelThreads * 16;

__global__ __launch_bounds__(kSelThreads) void topk_segment_kernel(const float* __restrict__ scores, int64_t ld,
                                                                   const int32_t* __restrict__ seq_lens, int n_q,
                                                                   int max_seq_len, int rows, int top_k, bool vec,
                                                                   int nseg, int32_t* __restrict__ cand) {
    __shared__ SelectShared sh;
    const int seg = blockIdx.x, r = rows - 1 - (int)blockIdx.y;
    const int b = r / n_q, i0 = r % n_q;
    const int L = history_len(clamp_len(seq_lens, b, max_seq_len), n_q, i0);
    const int tid = threadIdx.x;
    if (L <= top_k) return;  // stage 2 writes such rows itself
    int32_t* out = cand + ((int64_t)r * nseg + seg) * top_k;
    const int s0 = seg * kSegLen;
    const int Ls = min(max(L - s0, 0), kSegLen);  // positions of this segment in the history
    if (Ls <= top_k) {
        for (int t = tid; t < top_k; t += kSelThreads) out[t] = t < Ls ? s0 + t : -1;
        return;
    }
    const int base = 16 * tid;
    const int nv = min(max(Ls - base, 0), 16);
    uint32_t key[16];
    load_keys<16>(scores + (int64_t)r * ld + s0, base, nv, vec, key);
    block_select<16>(sh, key, top_k, [&](int place, int q) { out[place] = s0 + base + q; });
}

template <int KPT>
__global__ __launch_bounds__(kSelThreads) void topk_merge_kernel(const float* __restrict__ scores, int64_t ld,
                                                                 const int32_t* __restrict__ seq_lens, int n_q,
                                                                 int max_seq_len, int rows, int top_k, int nseg,
                                                                 const int32_t* __restrict__ cand,
                                                                 int32_t* __restrict__ indices) {
    __shared__ SelectShared sh;
    const int r = rows - 1 - (int)blockIdx.x;
    const int b = r / n_q, i0 = r % n_q;
    const int L = history_len(clamp_len(seq_lens, b, max_seq_len), n_q, i0);
    const int tid = threadIdx.x;
    int32_t* out = indices + (int64_t)r * top_k;
    if (L <= top_k) {
        for (int t = tid; t < top_k; t += kSelThreads) out[t] = t < L ? t : -1;
        return;
    }
    const int n = nseg * top_k;  // candidate slots of the row
    const int32_t* cr = cand + (int64_t)r * n;
    const float* row = scores + (int64_t)r * ld;
    const int base = KPT * tid;
    int pos[KPT];
    uint32_t key[KPT];
#pragma unroll
    for (int q = 0; q < KPT; ++q) pos[q] = base + q < n ? cr[base + q] : -1;
#pragma unroll
    for (int q = 0; q < KPT; ++q) key[q] = pos[q] < 0 ? 0u : score_key(row[pos[q]]);
    // a kept slot's position is read again from the candidate list (a cached
    // line) rather than held in registers through the selection
    block_select<KPT>(sh, key, top_k, [&](int place, int q) { out[place] = cr[base + q]; });
}

int topk_segments(int max_seq_len) { return (max_seq_len + kSegLen - 1) / kSegLen; }

size_t topk_ws_bytes(int rows, int max_seq_len, int top_k) {
    if (max_seq_len <= 32 * 1024) return 0;
    const int64_t n = (int64_t)topk_segments(max_seq_len) * top_k;
    if (n > 32 * 1024) return 0;  // beyond the merge kernel: the global-memory kernel, no workspace
    return sizeof(int32_t) * (size_t)rows * (size_t)n;
}

hipError_t launch_topk(const TopkLaunch& a, hipStream_t st) {
    const int rows = a.batch * a.n_q;
    if (rows == 0) return hipSuccess;
    const bool vec = (a.ld % 4) == 0 && ((uintptr_t)a.scores % 16) == 0;
    // persistent workgroups for the register-resident kernel: at most two per
    // compute unit
    int cus = 0;
    hipError_t e0 = compute_units(&cus);
    if (e0 != hipSuccess) return e0;
    const int reg_grid = rows < 2 * cus ? rows : 2 * cus;
#define DSA_REG(K)                                                                                           \
    hipLaunchKernelGGL((topk_reg_kernel<K>), dim3(reg_grid), dim3(kSelThreads), 0, st, a.scores, a.ld,      \
                       a.seq_lens, a.n_q, a.max_seq_len, rows, a.top_k, vec, a.indices)
    if (a.max_seq_len <= 8 * 1024) DSA_REG(8);
    else if (a.max_seq_len <= 16 * 1024) DSA_REG(16);
    else if (a.max_seq_len <= 32 * 1024) DSA_REG(32);
#undef DSA_REG
    else if (topk_ws_bytes(rows, a.max_seq_len, a.top_k) > 0) {
        const int nseg = topk_segments(a.max_seq_len);
        hipLaunchKernelGGL(topk_segment_kernel, dim3(nseg, rows), dim3(kSelThreads), 0, st, a.scores, a.ld,
                           a.seq_lens, a.n_q, a.max_seq_len, rows, a.top_k, vec, nseg, a.ws);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int n = nseg * a.top_k;
#define DSA_MERGE(K)                                                                                         \
    hipLaunchKernelGGL((topk_merge_kernel<K>), dim3(rows), dim3(kSelThreads), 0, st, a.scores, a.ld, a.seq_lens, \
                       a.n_q, a.max_seq_len, rows, a.top_k, nseg, a.ws, a.indices)
        if (n <= 8 * 1024) DSA_MERGE(8);
        else if (n <= 16 * 1024) DSA_MERGE(16);
        else DSA_MERGE(32);
#undef DSA_MERGE
    } else {
        hipLaunchKernelGGL((topk_kernel<1024, false>), dim3(rows), dim3(1024), 0, st, a.scores, a.ld,
                           a.seq_lens, a.n_q, a.max_seq_len, rows, a.top_k, a.indices);
    }
    return hipGetLastError();
}

}  // namespace dsa
