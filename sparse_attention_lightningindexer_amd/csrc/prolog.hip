// prolog.hip -- the indexer prolog for gfx950: the index query and head weights
// projected from the hidden state, the index query quantized, and the new index
// key RMS-normalized, in one launch.
//
// The pages run these preparation steps on three streams so that the
// independent ones overlap ("Day0 Inference Adaptation and Performance
// Optimization for New-Architecture LLMs", §4.2 Three-Stream Coordination for
// Indexer Preprocessing; "Day0 Inference Adaptation and Performance
// Optimization for a New Architecture Domestic Large Language Model on
// Ascend", §4).  Here the branches are workgroup roles of one grid, so they
// run side by side on the compute units with no cross-stream events:
//   role N (one workgroup per row tile): k_norm = k * gain / sqrt(mean k^2 + eps)
//   role H (ceil(H_I/32) workgroups):    head_w = W_h x, fp32
//   role Q (H_I*d_I/32 workgroups):      q = W_q x, stored as bf16 or as MXFP8
//                                         (e4m3 codes, one E8M0 scale per 32),
//                                         quantized in the epilogue
// Projections take bf16 operands with fp32 accumulation on MFMA; the pages keep
// projections in BF16 and the index query in MXFP8 (the first page above, §5
// Layered Quantization).
//
// A Q or H workgroup owns 32 output columns (one MXFP8 group of one head) and a
// tile of 16*MT rows.  Its eight waves split the hidden width: wave w takes the
// 128-wide k chunks w, w+8, ...; in a chunk, lane (g = lane/16, j = lane%16)
// loads 32 consecutive k (64 B) of weight row j and of hidden-state row j, so
// one wave load covers 256 contiguous bytes of 16 rows.  The four bf16x8 pieces
// of a lane feed four 16x16x32 MFMAs; since A and B pieces of a lane cover the
// same k, the sum over k is unchanged.  The weights are read once from HBM (the
// bound at decode sizes); the hidden state is re-read by every workgroup from
// L2.  The waves' partial sums meet in LDS, added in wave order.
#include "common.hpp"
#include "kernels.hpp"

namespace dsa {

namespace {

constexpr int kPWaves = 8;
constexpr int kPThreads = kPWaves * kWave;
constexpr int kPCols = 32;     // output columns per workgroup: one MXFP8 group
constexpr int kPChunk = 128;   // k per wave step: 4 lane groups x 32 consecutive k
constexpr int kPPad = 65;      // LDS row of one partial register (64 lanes + 1)

__device__ __forceinline__ void load64(const uint16_t* p, bool ok, bf16x8 (&f)[4]) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint4 u = ok ? q[s] : make_uint4(0u, 0u, 0u, 0u);
        f[s] = __builtin_bit_cast(bf16x8, u);
    }
}

__device__ __forceinline__ float clamp448p(float v) { return fminf(fmaxf(v, -448.f), 448.f); }

// k_norm rows row0 .. row0 + nrows - 1: one wave per row, lane c holds
// channels c, c + 64, ... (head_dim <= 256).
__device__ void rms_norm_rows(const PrologLaunch& a, int row0, int nrows) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int rr = w; rr < nrows; rr += kPWaves) {
        const int r = row0 + rr;
        if (r >= a.rows) break;
        float v[4];
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = lane + 64 * e;
            v[e] = c < a.d_I ? bf16_bits_to_f32(a.k[(int64_t)r * a.d_I + c]) : 0.f;
            ss += v[e] * v[e];
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, kWave);
        const float inv = 1.0f / sqrtf(ss / (float)a.d_I + a.eps);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = lane + 64 * e;
            if (c < a.d_I) a.k_norm[(int64_t)r * a.d_I + c] = f32_to_bf16_bits(v[e] * inv * a.gain[c]);
        }
    }
}

template <int MT>
__global__ __launch_bounds__(kPThreads, MT == 4 ? 1 : 2) void indexer_prolog_kernel(PrologLaunch a) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int row0 = blockIdx.y * (16 * MT);
    if (blockIdx.x == 0) {
        rms_norm_rows(a, row0, 16 * MT);
        return;
    }
    const int nq = a.H_I * a.d_I;
    const int n_ht = (a.H_I + kPCols - 1) / kPCols;
    const int bx = blockIdx.x - 1;
    const bool head = bx < n_ht;
    const int col0 = (head ? bx : bx - n_ht) * kPCols;
    const int ncols = head ? a.H_I : nq;
    const uint16_t* W = head ? a.w_h : a.w_q;
    const int j = lane & 15, g = lane >> 4;

    const uint16_t* brow[2];
    bool bok[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int n = col0 + nt * 16 + j;
        bok[nt] = n < ncols;
        brow[nt] = W + (int64_t)(bok[nt] ? n : 0) * a.d_x + 32 * g;
    }
    const uint16_t* arow[MT];
    bool aok[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = row0 + mt * 16 + j;
        aok[mt] = m < a.rows;
        arow[mt] = a.x + (int64_t)(aok[mt] ? m : 0) * a.d_x + 32 * g;
    }

    f32x4 acc[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nchunks = a.d_x / kPChunk;
    for (int c = w; c < nchunks; c += kPWaves) {
        const int k0 = c * kPChunk;
        bf16x8 A[MT][4], B[2][4];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) load64(brow[nt] + k0, bok[nt], B[nt]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) load64(arow[mt] + k0, aok[mt], A[mt]);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mfma_bf16(A[mt][s], B[nt][s], acc[mt][nt]);
    }

    // Partial sums of the eight waves: element (row 4g + i of tile mt, column
    // j of tile nt) sits in register i of lane 16g + j.
    __shared__ float red[kPWaves * MT * 2 * 4 * kPPad];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[(((w * MT + mt) * 2 + nt) * 4 + i) * kPPad + lane] = acc[mt][nt][i];
    __syncthreads();

    // Thread t finishes MT consecutive columns of one row: row t / TPR of the
    // tile, columns (t % TPR) * MT ...; a row's 32 columns are TPR adjacent lanes.
    constexpr int TPR = kPCols / MT;
    const int t = threadIdx.x;
    const int rho = t / TPR, cb = (t % TPR) * MT;
    const int mt = rho / 16, gg = (rho % 16) / 4, ii = rho % 4;
    float v[MT];
#pragma unroll
    for (int e = 0; e < MT; ++e) {
        const int col = cb + e, nt = col / 16, src = 16 * gg + col % 16;
        float s = 0.f;
#pragma unroll
        for (int ww = 0; ww < kPWaves; ++ww) s += red[(((ww * MT + mt) * 2 + nt) * 4 + ii) * kPPad + src];
        v[e] = s;
    }
    const int r = row0 + rho;
    const bool live_row = r < a.rows;

    if (head) {
#pragma unroll
        for (int e = 0; e < MT; ++e)
            if (live_row && col0 + cb + e < ncols) a.head_w[(int64_t)r * a.H_I + col0 + cb + e] = v[e];
        return;
    }
    const int64_t o = (int64_t)r * nq + col0 + cb;
    if (!a.q_mx) {
        if (!live_row) return;
        uint16_t* q = static_cast<uint16_t*>(a.q_out) + o;
        if constexpr (MT == 1) {
            q[0] = f32_to_bf16_bits(v[0]);
        } else if constexpr (MT == 2) {
            *reinterpret_cast<uint32_t*>(q) = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
        } else {
            const uint32_t lo = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
            const uint32_t hi = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
            *reinterpret_cast<uint2*>(q) = make_uint2(lo, hi);
        }
        return;
    }
    // MXFP8: e = floor(log2 amax) - 8 (-127 when amax = 0), clamped to
    // [-127, 127]; code = e4m3(clamp(x * 2^-e, +-448)); scale byte e + 127.
    float am = 0.f;
#pragma unroll
    for (int e = 0; e < MT; ++e) am = fmaxf(am, fabsf(v[e]));
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1) am = fmaxf(am, __shfl_xor(am, m, kWave));
    int e2 = 0;
    (void)frexpf(am, &e2);
    int ex = am > 0.f ? e2 - 1 - 8 : -127;
    ex = min(max(ex, -127), 127);
    if (!live_row) return;
    uint8_t* q = static_cast<uint8_t*>(a.q_out) + o;
    if constexpr (MT == 1) {
        q[0] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(clamp448p(ldexpf(v[0], -ex)), 0.f, 0, false) & 0xff);
    } else if constexpr (MT == 2) {
        const int p = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448p(ldexpf(v[0], -ex)), clamp448p(ldexpf(v[1], -ex)), 0,
                                                      false);
        *reinterpret_cast<uint16_t*>(q) = (uint16_t)(p & 0xffff);
    } else {
        int p = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448p(ldexpf(v[0], -ex)), clamp448p(ldexpf(v[1], -ex)), 0, false);
        p = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448p(ldexpf(v[2], -ex)), clamp448p(ldexpf(v[3], -ex)), p, true);
        *reinterpret_cast<uint32_t*>(q) = (uint32_t)p;
    }
    if (cb == 0) a.q_scale[(int64_t)r * (nq / 32) + col0 / 32] = (uint8_t)(ex + 127);
}

}  // namespace

hipError_t launch_indexer_prolog(const PrologLaunch& a, hipStream_t st) {
    if (a.rows == 0) return hipSuccess;
    const int MT = a.rows <= 16 ? 1 : (a.rows <= 32 ? 2 : 4);
    const int n_tiles = 1 + (a.H_I + kPCols - 1) / kPCols + a.H_I * a.d_I / kPCols;
    const dim3 grid(n_tiles, (a.rows + 16 * MT - 1) / (16 * MT));
    if (MT == 1)
        hipLaunchKernelGGL(indexer_prolog_kernel<1>, grid, dim3(kPThreads), 0, st, a);
    else if (MT == 2)
        hipLaunchKernelGGL(indexer_prolog_kernel<2>, grid, dim3(kPThreads), 0, st, a);
    else
        hipLaunchKernelGGL(indexer_prolog_kernel<4>, grid, dim3(kPThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace dsa
