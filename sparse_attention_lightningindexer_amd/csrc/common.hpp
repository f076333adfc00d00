// common.hpp -- device helpers shared by the gfx950 kernels of libdsa.
//
// Lane layouts of the matrix instructions used here (64-lane wave, l = lane,
// g = l / 16, j = l % 16), checked on gfx950 hardware:
//   v_mfma_f32_16x16x32_bf16   A: lane holds A[j][8g + 0..7], B: B[8g + 0..7][j],
//                              D: lane holds D[4g + 0..3][j]
//   v_mfma_f32_16x16x32_fp8    same as bf16 with 8 e4m3 bytes per lane (OCP e4m3)
//   v_mfma_scale_f32_16x16x128_f8f6f4 (fp8 operands): bytes 0..15 of a lane are
//                              A[j][16g + 0..15] / B[16g + 0..15][j], bytes 16..31
//                              A[j][64 + 16g + 0..15] / B[64 + 16g + 0..15][j]; the
//                              E8M0 scale byte of lane 16b + j applies to k-block b
//                              (k = 32b .. 32b+31) of row j of A / column j of B
//   ds_read_b64_tr_b16         in each 16-lane group, lane j's element e is the
//                              16-bit word (j % 4) at the address given by lane
//                              4e + j/4 of that group.
//   v_permlane16_swap / v_permlane32_swap with both operands x give the pair
//                              (x[l], x[l ^ 16]) / (x[l], x[l ^ 32]) in some order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef short v4i16 __attribute__((ext_vector_type(4)));

#define DSA_LDS __attribute__((address_space(3)))

constexpr int kWave = 64;
constexpr int kBlock = 64;  // tokens per cache block

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}

// float -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Sum of x over lanes l, l^16, l^32, l^48 (every lane gets the total).
__device__ __forceinline__ float sum_over_groups(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Max of x over lanes l, l^16, l^32, l^48.
__device__ __forceinline__ float max_over_groups(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Inclusive prefix sum over the 64 lanes of a wave (sum over lanes <= this
// one) with DPP moves: shifts within rows of 16 lanes, then row broadcasts.
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t x) {
    x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
    x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
    return x;
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16x16x128 e4m3 x e4m3 with unit (E8M0 = 127) block scales.
__device__ __forceinline__ f32x4 mfma_fp8_k128(i32x8 a, i32x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// The same with this lane's E8M0 block scales for A and B (layout above).
__device__ __forceinline__ f32x4 mfma_mx_k128(i32x8 a, i32x8 b, f32x4 c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// Number of lanes below this one whose bit is set in `mask`.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
    uint32_t lo = (uint32_t)mask, hi = (uint32_t)(mask >> 32);
    return (int)__builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) {
    return __builtin_amdgcn_ballot_w64(p);
}

// ---- asynchronous gathers into LDS, outside the compiler's wait-count tracking
//
// global_load_lds writes each lane's bytes to LDS at M0 + lane * size.  Issued
// through the builtin, the compiler cannot tell which LDS buffer such a load
// targets and waits for it (vmcnt(0)) before any later LDS read or barrier,
// which serializes a multi-stage gather pipeline.  Issued here, the loads are
// invisible to its bookkeeping: the caller waits on them with wait_vmcnt(n)
// (n = this wave's vector-memory operations issued after the ones needed; they
// complete in order) and then sync_lds().  Extra outstanding loads only make
// the compiler's own waits stricter, never incorrect.  `lds` must be uniform.
__device__ __forceinline__ void lds_gather16(const void* src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void lds_gather4(const void* src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// wave-uniform n in [0, 63] (the counter's range; a larger n waits for 63)
__device__ __forceinline__ void wait_vmcnt(int n) {
    switch (n) {
#define DSA_W(N) case N: wait_vmcnt<N>(); break;
    DSA_W(0) DSA_W(1) DSA_W(2) DSA_W(3) DSA_W(4) DSA_W(5) DSA_W(6) DSA_W(7)
    DSA_W(8) DSA_W(9) DSA_W(10) DSA_W(11) DSA_W(12) DSA_W(13) DSA_W(14) DSA_W(15)
    DSA_W(16) DSA_W(17) DSA_W(18) DSA_W(19) DSA_W(20) DSA_W(21) DSA_W(22) DSA_W(23)
    DSA_W(24) DSA_W(25) DSA_W(26) DSA_W(27) DSA_W(28) DSA_W(29) DSA_W(30) DSA_W(31)
    DSA_W(32) DSA_W(33) DSA_W(34) DSA_W(35) DSA_W(36) DSA_W(37) DSA_W(38) DSA_W(39)
    DSA_W(40) DSA_W(41) DSA_W(42) DSA_W(43) DSA_W(44) DSA_W(45) DSA_W(46) DSA_W(47)
    DSA_W(48) DSA_W(49) DSA_W(50) DSA_W(51) DSA_W(52) DSA_W(53) DSA_W(54) DSA_W(55)
    DSA_W(56) DSA_W(57) DSA_W(58) DSA_W(59) DSA_W(60) DSA_W(61) DSA_W(62)
#undef DSA_W
    default: wait_vmcnt<63>(); break;
    }
}
// Workgroup barrier for LDS data only (no wait on outstanding global loads).
__device__ __forceinline__ void sync_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The value of x, hidden from the optimizer so that address arithmetic derived
// from it is recomputed where it is used instead of being hoisted out of a loop
// (and kept live, or spilled) for the whole kernel.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Scheduling fence: no instruction is moved across it, so a block of LDS
// reads written before it is issued as a block (their latencies overlap)
// instead of being interleaved one by one with the MFMAs that consume them.
__device__ __forceinline__ void issue_fence() { __builtin_amdgcn_sched_barrier(0); }

// LDS byte address of a __shared__ object (generic pointer cast to the LDS address space).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const DSA_LDS void*)p;
}

// Causal history of row r = b*n_q + i with the clamped sequence length Lb.
__device__ __forceinline__ int history_len(int Lb, int n_q, int i) {
    int L = Lb - n_q + i + 1;
    return L < 0 ? 0 : L;
}

__device__ __forceinline__ int clamp_len(const int32_t* seq_lens, int b, int max_seq_len) {
    int L = seq_lens[b];
    L = L < 0 ? 0 : L;
    return L > max_seq_len ? max_seq_len : L;
}

// Physical block of logical block j of sequence b, or -1 when absent.  The
// table entry is read unconditionally (from a clamped, in-range column), so
// that several lookups issue back to back instead of each behind a branch.
__device__ __forceinline__ int64_t phys_block(const int32_t* table, int max_blocks, int b, int j,
                                              int64_t num_blocks) {
    const bool in = j >= 0 && j < max_blocks;
    const int64_t p = table[(int64_t)b * max_blocks + (in ? j : 0)];
    return (!in || p < 0 || p >= num_blocks) ? -1 : p;
}

}  // namespace dsa
