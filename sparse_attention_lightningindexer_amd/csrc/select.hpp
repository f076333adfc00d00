// select.hpp -- the exact Top-K selection of one row by one workgroup, shared
// by the Top-K kernels and the attention kernel's fused form: order-preserving
// score keys and a register-resident MSB-first radix select with an ordered
// emit ("Day0 Inference Adaptation and Performance Optimization for
// New-Architecture LLMs", §4.1, the top-k step of the indexer).
#pragma once

#include "common.hpp"

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

// Register-resident selection by one NT-thread workgroup over up to
// NT * KPT slots.  Slots are wave-strided: lane l of wave w holds in key[q]
// slot 64 * (KPT * w + q) + l, so a column q of a wave is 64 consecutive
// slots -- one coalesced load, and one ballot is the column's bit mask.  Key 0
// marks an empty slot.  The MSB-first radix select uses digits of 12, 10 and
// 10 bits (one LDS histogram per pass, bins owned by threads for the suffix
// scan; the later passes are skipped once a cut bin holds exactly the keys
// still needed) and finds the cut key T and the number of keys equal to T to
// keep.  The histogram is all zero on entry (clear_hist, once per workgroup)
// and is left so.  The emit goes column by column: a kept slot's place is the
// number of kept slots before it, the keys > T before it plus min(keys == T
// before it, the number to keep), so the lowest slots come first among equal
// keys; the waves' totals go through one block scan and a column's lanes
// count with mbcnt.  emit(place, q, slot) writes a kept slot.  Exactly top_k
// slots are kept (callers guarantee that at least top_k slots are not empty).
// Empty slots are left out of the first histogram only to spare one bin the
// atomic traffic; the later passes and the final comparisons need no test,
// since key 0 lies below the cut.
template <int NT>
struct SelectShared {
    uint32_t hist[4096];
    uint32_t wsum[NT / kWave] __attribute__((aligned(16)));
    uint32_t cut_digit, cut_above, cut_count;
};

// Workgroup barrier of the select.  LDSB: wait for LDS operations only, so
// that unrelated global loads (a caller's prefetch) stay in flight.
template <bool LDSB>
__device__ __forceinline__ void select_barrier() {
    if constexpr (LDSB) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else __syncthreads();
}

template <int NT, bool LDSB = false>
__device__ __forceinline__ void clear_hist(SelectShared<NT>& sh) {
    for (int t = threadIdx.x; t < 4096; t += NT) sh.hist[t] = 0u;
    select_barrier<LDSB>();
}

template <int NT, int KPT, bool LDSB = false, class Emit>
__device__ __forceinline__ void block_select(SelectShared<NT>& sh, const uint32_t (&key)[KPT], int top_k,
                                             Emit&& emit) {
    static_assert(KPT <= 32, "registers per thread");
    static_assert(NT == 512 || NT == 1024, "bins per thread");
    constexpr int NW = NT / kWave;
    // the wave index is uniform across the wave; saying so keeps the per-wave
    // comparisons below scalar instead of 64-bit lane masks held in registers
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // sums of the per-wave totals in sh.wsum over the waves before this one
    // and after it: lane w < NW reads wave w's total, one wave scan, two
    // lane reads (no per-wave comparisons held in registers)
    auto wsum_around = [&](uint32_t& before, uint32_t& after) {
        const uint32_t v = lane < NW ? sh.wsum[lane] : 0u;
        const uint32_t incl = wave_scan_incl(v);
        const uint32_t upto = __builtin_amdgcn_readlane(incl, wave);
        before = upto - __builtin_amdgcn_readlane(v, wave);
        after = __builtin_amdgcn_readlane(incl, NW - 1) - upto;
    };
    uint32_t prefix = 0u, mask = 0u, krem = (uint32_t)top_k;  // uniform
    auto pass = [&](int shift, int bits, bool first) {
        const uint32_t nb = 1u << bits, dm = nb - 1u;
#pragma unroll
        for (int q = 0; q < KPT; ++q)
            if (first ? key[q] != 0u : (key[q] & mask) == prefix) atomicAdd(&sh.hist[(key[q] >> shift) & dm], 1u);
        select_barrier<LDSB>();
        // thread t owns bins [per*t, per*t + per); its counts are read, cleared
        // for the next pass, and scanned from the top digit down.
        const int per = (int)nb / NT;  // bins per thread
        uint32_t cnt[4096 / NT] = {}, own = 0u;
        for (int k = 0; k < per; ++k) {
            cnt[k] = sh.hist[per * tid + k];
            sh.hist[per * tid + k] = 0u;
            own += cnt[k];
        }
        const uint32_t P = wave_scan_incl(own);                    // lanes <= this one
        const uint32_t wtot = __builtin_amdgcn_readlane(P, kWave - 1);
        if (lane == 0) sh.wsum[wave] = wtot;
        select_barrier<LDSB>();
        // keys in higher bins: later lanes of this wave, then later waves
        uint32_t wb_, wa_;
        wsum_around(wb_, wa_);
        const uint32_t above = (wtot - P) + wa_;
        // S(d) = keys with digit >= d; the cut digit D has S(D) >= krem > S(D+1)
        if (above < krem && above + own >= krem) {
            uint32_t sfx = above;
            for (int k = per - 1; k >= 0; --k) {
                if (sfx + cnt[k] >= krem) {
                    sh.cut_digit = (uint32_t)(per * tid + k);
                    sh.cut_above = sfx;
                    sh.cut_count = cnt[k];
                    break;
                }
                sfx += cnt[k];
            }
        }
        select_barrier<LDSB>();
        prefix |= __builtin_amdgcn_readfirstlane(sh.cut_digit) << shift;
        mask |= dm << shift;
        krem -= __builtin_amdgcn_readfirstlane(sh.cut_above);
    };
    // When the cut bin holds exactly the krem keys still needed, every key from
    // that bin's lowest value up is kept and the remaining passes are skipped:
    // the cut becomes the value just below the bin (T = prefix - 1, no keys
    // equal to T taken).  A bin starting at 0 goes on to the next pass.
    bool whole_bin = false;
    auto take_whole_bin = [&]() {
        whole_bin = __builtin_amdgcn_readfirstlane(sh.cut_count) == krem && prefix != 0u;
    };
    pass(20, 12, true);
    take_whole_bin();
    if (!whole_bin) {
        pass(10, 10, false);
        take_whole_bin();
        if (!whole_bin) pass(0, 10, false);
    }
    if (whole_bin) krem = 0u;

    // T is the k-th largest key, or the value just below its whole cut bin;
    // krem keys equal to it are taken, lowest first.
    const uint32_t T = whole_bin ? prefix - 1u : prefix;
    // Ordered emit, column by column.  A kept slot's place is the number of
    // kept slots before it: the keys > T before it plus min(keys == T before
    // it, krem).  The waves' totals go through one block scan; within a wave
    // the running counts of the earlier columns are scalar and a column's own
    // lanes count with mbcnt.  The comparisons are made again in the second
    // loop (T passes through an opaque copy) rather than held as lane masks.
    uint32_t wgt = 0u, weq = 0u;  // this wave's keys > T and == T (uniform)
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
        wgt += (uint32_t)__popcll(ballot(key[q] > T));
        weq += (uint32_t)__popcll(ballot(key[q] == T));
        asm volatile("" : "+s"(wgt), "+s"(weq));  // summed column by column, one column's masks live
    }
    if (lane == 0) sh.wsum[wave] = (wgt << 16) | weq;  // both totals stay below 2^16
    select_barrier<LDSB>();
    uint32_t before, after_;
    wsum_around(before, after_);
    uint32_t gtb = before >> 16, eqb = before & 0xffffu;  // keys > T and == T in earlier columns
    uint32_t Tq = T;
    asm volatile("" : "+s"(Tq));
    const int wslot = KPT * kWave * wave + lane;
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
        const bool gt = key[q] > Tq, eq = key[q] == Tq;
        const uint64_t mg = ballot(gt), me = ballot(eq);
        const uint32_t eq_before = eqb + (uint32_t)lanes_below(me);
        if (gt || (eq && eq_before < krem))
            emit((int)(gtb + (uint32_t)lanes_below(mg) + min(eq_before, krem)), q, wslot + kWave * q);
        gtb += (uint32_t)__popcll(mg);
        eqb += (uint32_t)__popcll(me);
        asm volatile("" : "+s"(gtb), "+s"(eqb));  // one column's masks live at a time
    }
}

// Keys of the wave's slots wb + 64q + lane (q < KPT) of a run of n scores
// (slots from n on are empty).  Loads are unconditional (a slot past the run
// reads the last score) so that each column is one coalesced load and all of
// them are in flight at once.
template <int KPT>
__device__ __forceinline__ void load_keys(const float* row, int wb, int n, int lane, uint32_t (&key)[KPT]) {
    if (wb + kWave * KPT <= n) {  // wave-uniform
#pragma unroll
        for (int q = 0; q < KPT; ++q) key[q] = score_key(row[wb + kWave * q + lane]);
    } else if (wb < n) {
        float v[KPT];
#pragma unroll
        for (int q = 0; q < KPT; ++q) v[q] = row[min(wb + kWave * q + lane, n - 1)];
#pragma unroll
        for (int q = 0; q < KPT; ++q) key[q] = wb + kWave * q + lane < n ? score_key(v[q]) : 0u;
    } else {
#pragma unroll
        for (int q = 0; q < KPT; ++q) key[q] = 0u;
    }
}

}  // namespace dsa
