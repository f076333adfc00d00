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
//     per thread of a 1024-thread workgroup), up to three digit passes;
//   * longer rows: a top_k per 16384-position segment into a candidate
//     workspace, then the same register-resident selection over the
//     candidates;
//   * otherwise (no workspace): the keys are re-read from memory in four
//     8-bit passes.
#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace dsa {


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

constexpr int kSelThreads = 1024;

// Rows up to 1024 * KPT positions.  Workgroups are persistent: workgroup b
// takes rows b, b + G, b + 2G, ... counted from the last (longest) row.
template <int KPT>
__global__ __launch_bounds__(kSelThreads) void topk_reg_kernel(const float* __restrict__ scores, int64_t ld,
                                                               const int32_t* __restrict__ seq_lens, int n_q,
                                                               int max_seq_len, int rows, int top_k,
                                                               int32_t* __restrict__ indices) {
    __shared__ SelectShared<kSelThreads> sh;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wb = KPT * kWave * __builtin_amdgcn_readfirstlane(tid >> 6);  // the wave's first slot
    clear_hist(sh);
    for (int i = (int)blockIdx.x; i < rows; i += (int)gridDim.x) {
        const int r = rows - 1 - i;
        const int L = history_len(clamp_len(seq_lens, r / n_q, max_seq_len), n_q, r % n_q);
        int32_t* out = indices + (int64_t)r * top_k;
        if (L <= top_k) {  // keep the whole history
            for (int t = tid; t < top_k; t += kSelThreads) out[t] = t < L ? t : -1;
            continue;  // workgroup-uniform; no shared memory was touched
        }
        uint32_t key[KPT];
        load_keys<KPT>(scores + (int64_t)r * ld, wb, L, lane, key);
        block_select<kSelThreads, KPT>(sh, key, top_k, [&](int place, int, int slot) { out[place] = slot; });
        __syncthreads();  // the scan words and column masks are reused by the next row
    }
}

// Rows longer than the register-resident kernel takes: stage 1 keeps the top_k
// of every 16384-position segment (all of a shorter segment) as ascending
// positions in cand[row][segment][top_k] (-1 padded), with their keys in
// ckey[row][segment][top_k] (0 for padding); the row's top_k is contained in
// the union.  Stage 2 selects from those candidates, which are in ascending
// position order, so the lowest-position rule for equal scores carries over.
// grid (segments, rows) and (rows).  The workspace holds cand, then ckey.
constexpr int kSegKpt = 16;
constexpr int kSegLen = kSelThreads * kSegKpt;

__global__ __launch_bounds__(kSelThreads) void topk_segment_kernel(const float* __restrict__ scores, int64_t ld,
                                                                   const int32_t* __restrict__ seq_lens, int n_q,
                                                                   int max_seq_len, int rows, int top_k, int nseg,
                                                                   int32_t* __restrict__ cand,
                                                                   uint32_t* __restrict__ ckey) {
    __shared__ SelectShared<kSelThreads> sh;
    const int seg = blockIdx.x, r = rows - 1 - (int)blockIdx.y;
    const int b = r / n_q, i0 = r % n_q;
    const int L = history_len(clamp_len(seq_lens, b, max_seq_len), n_q, i0);
    const int tid = threadIdx.x, lane = tid & 63;
    if (L <= top_k) return;  // stage 2 writes such rows itself
    const int64_t o = ((int64_t)r * nseg + seg) * top_k;
    int32_t* outp = cand + o;
    uint32_t* outk = ckey + o;
    const int s0 = seg * kSegLen;
    const int Ls = min(max(L - s0, 0), kSegLen);  // positions of this segment in the history
    const float* row = scores + (int64_t)r * ld + s0;
    if (Ls <= top_k) {
        for (int t = tid; t < top_k; t += kSelThreads) {
            outp[t] = t < Ls ? s0 + t : -1;
            outk[t] = t < Ls ? score_key(row[t]) : 0u;
        }
        return;
    }
    const int wb = kSegKpt * kWave * __builtin_amdgcn_readfirstlane(tid >> 6);
    uint32_t key[kSegKpt];
    load_keys<kSegKpt>(row, wb, Ls, lane, key);
    clear_hist(sh);
    block_select<kSelThreads, kSegKpt>(sh, key, top_k, [&](int place, int q, int slot) {
        outp[place] = s0 + slot;
        outk[place] = key[q];
    });
}

template <int KPT>
__global__ __launch_bounds__(kSelThreads) void topk_merge_kernel(const int32_t* __restrict__ seq_lens, int n_q,
                                                                 int max_seq_len, int rows, int top_k, int nseg,
                                                                 const int32_t* __restrict__ cand,
                                                                 const uint32_t* __restrict__ ckey,
                                                                 int32_t* __restrict__ indices) {
    __shared__ SelectShared<kSelThreads> sh;
    const int r = rows - 1 - (int)blockIdx.x;
    const int b = r / n_q, i0 = r % n_q;
    const int L = history_len(clamp_len(seq_lens, b, max_seq_len), n_q, i0);
    const int tid = threadIdx.x, lane = tid & 63;
    int32_t* out = indices + (int64_t)r * top_k;
    if (L <= top_k) {
        for (int t = tid; t < top_k; t += kSelThreads) out[t] = t < L ? t : -1;
        return;
    }
    const int n = nseg * top_k;  // candidate slots of the row
    const int32_t* cr = cand + (int64_t)r * n;
    const uint32_t* ck = ckey + (int64_t)r * n;
    const int wb = KPT * kWave * __builtin_amdgcn_readfirstlane(tid >> 6);
    // unconditional loads (clamped to the last slot): one batch in flight
    int32_t pos[KPT];
    uint32_t key[KPT];
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
        const int sl = min(wb + kWave * q + lane, n - 1);
        pos[q] = cr[sl];
        key[q] = ck[sl];
    }
    // slots past the list (n <= KPT * 1024) and -1 padding are empty
#pragma unroll
    for (int q = 0; q < KPT; ++q)
        if (wb + kWave * q + lane >= n || pos[q] < 0) key[q] = 0u;
    clear_hist(sh);
    block_select<kSelThreads, KPT>(sh, key, top_k, [&](int place, int q, int) { out[place] = pos[q]; });
}

int topk_segments(int max_seq_len) { return (max_seq_len + kSegLen - 1) / kSegLen; }

size_t topk_ws_bytes(int rows, int max_seq_len, int top_k) {
    if (max_seq_len <= 32 * 1024) return 0;
    const int64_t n = (int64_t)topk_segments(max_seq_len) * top_k;
    if (n > 32 * 1024) return 0;  // beyond the merge kernel: the global-memory kernel, no workspace
    return 2 * sizeof(int32_t) * (size_t)rows * (size_t)n;  // positions, then their keys
}

hipError_t launch_topk(const TopkLaunch& a, hipStream_t st) {
    const int rows = a.batch * a.n_q;
    if (rows == 0) return hipSuccess;
    // persistent workgroups for the register-resident kernel: at most two per
    // compute unit
    int cus = 0;
    hipError_t e0 = compute_units(&cus);
    if (e0 != hipSuccess) return e0;
    const int reg_grid = rows < 2 * cus ? rows : 2 * cus;
#define DSA_REG(K)                                                                                           \
    hipLaunchKernelGGL((topk_reg_kernel<K>), dim3(reg_grid), dim3(kSelThreads), 0, st, a.scores, a.ld,      \
                       a.seq_lens, a.n_q, a.max_seq_len, rows, a.top_k, a.indices)
    if (a.max_seq_len <= 8 * 1024) DSA_REG(8);
    else if (a.max_seq_len <= 16 * 1024) DSA_REG(16);
    else if (a.max_seq_len <= 32 * 1024) DSA_REG(32);
#undef DSA_REG
    else if (topk_ws_bytes(rows, a.max_seq_len, a.top_k) > 0) {
        const int nseg = topk_segments(a.max_seq_len);
        const int n = nseg * a.top_k;
        int32_t* cand = a.ws;
        uint32_t* ckey = reinterpret_cast<uint32_t*>(a.ws + (size_t)rows * n);
        hipLaunchKernelGGL(topk_segment_kernel, dim3(nseg, rows), dim3(kSelThreads), 0, st, a.scores, a.ld,
                           a.seq_lens, a.n_q, a.max_seq_len, rows, a.top_k, nseg, cand, ckey);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
#define DSA_MERGE(K)                                                                                         \
    hipLaunchKernelGGL((topk_merge_kernel<K>), dim3(rows), dim3(kSelThreads), 0, st, a.seq_lens, a.n_q,       \
                       a.max_seq_len, rows, a.top_k, nseg, cand, ckey, a.indices)
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
