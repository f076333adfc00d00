// prolog.hip -- the indexer prolog for gfx950: the index query and head weights
// projected from the hidden state, the index query quantized, and the new index
// key RMS-normalized, in one launch.
//
// The pages run these preparation steps on three streams so that the
// independent ones overlap ("Day0 Inference Adaptation and Performance
// Optimization for New-Architecture LLMs", §4.2 Three-Stream Coordination for
// Indexer Preprocessing; "Day0 Inference Adaptation and Performance
// Optimization for a New Architecture Domestic Large Language Model on
// Ascend", §4).  Here the branches share one grid with no cross-stream events:
//   q = W_q x       every workgroup: 32 columns of q (one MXFP8 group of one
//                   head) for a tile of 16*MT rows, stored as bf16 or MXFP8
//                   (e4m3 codes, one E8M0 scale per 32) by its epilogue
//   head_w = W_h x  the workgroup holding channels 0..31 of head h also streams
//                   row h of W_h and computes head h's weight on a third MFMA
//                   column tile (fp32)
//   k_norm          k * gain / sqrt(mean k^2 + eps): the rows of a row tile are
//                   shared out over that tile's workgroups
// so a decode step with 64 heads of 128 channels is exactly 256 workgroups, one
// per compute unit.  Projections take bf16 operands with fp32 accumulation on
// MFMA; the pages keep projections in BF16 and the index query in MXFP8 (the
// first page above, §5 Layered Quantization).
//
// Data movement.  The weights are read once from HBM, which bounds the kernel
// at decode sizes.  A workgroup's operands for 256 consecutive k (a stage: its
// 32 weight rows, its 16*MT hidden-state rows and the head row, 512 B each) go
// into LDS with global_load_lds: each wave instruction moves 1 KB, two whole
// 512 B row segments, so HBM sees long contiguous reads rather than 16 rows
// 14 KB apart per instruction.  Within a row, 16-byte piece q is stored at slot
// q ^ (row % 16), so the 16 rows an MFMA operand read touches fall in distinct
// bank groups.  A ring of S stages keeps S-1 stages in flight.  Wave w takes k
// slice 32w .. 32w+31 of each stage for its MFMAs; the waves' partial sums
// meet in LDS at the end, added in wave order.
#include "common.hpp"
#include "kernels.hpp"

namespace dsa {

namespace {

constexpr int kPWaves = 8;
constexpr int kPThreads = kPWaves * kWave;
constexpr int kPCols = 32;        // output columns per workgroup: one MXFP8 group
constexpr int kPStage = 256;      // k per LDS stage (32 per wave)
constexpr int kPRowB = kPStage * 2;  // bytes of one row segment in a stage
constexpr int kPPad = 65;         // LDS row of one partial register (64 lanes + 1)

template <int MT>
struct PCfg {
    static constexpr int XR = 16 * MT;            // hidden-state rows per tile
    static constexpr int ROWS = kPCols + XR + 2;  // + the head row (and an unused twin)
    static constexpr int STAGE = ROWS * kPRowB;   // bytes per stage
    static constexpr int S = MT == 4 ? 3 : 4;     // ring depth
    static constexpr int INS = ROWS / 2;          // 1 KB DMA instructions per stage
    static constexpr int RED = (kPWaves * MT * 2 * 4 * kPPad + kPWaves * XR) * 4;  // reduction bytes
    static constexpr int LDS = S * STAGE > RED ? S * STAGE : RED;
};

__device__ __forceinline__ float clamp448p(float v) { return fminf(fmaxf(v, -448.f), 448.f); }

// One row of k_norm: a wave, lane c holding channels c, c + 64, ... (d_I <= 256).
__device__ void rms_norm_row(const PrologLaunch& a, int r, int lane) {
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

template <int MT>
__global__ __launch_bounds__(kPThreads, 2) void indexer_prolog_kernel(PrologLaunch a) {
    using C = PCfg<MT>;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[C::LDS];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int nq = a.H_I * a.d_I;
    const int n_qt = nq / kPCols;
    const int row0 = blockIdx.y * C::XR;
    const int col0 = blockIdx.x * kPCols;
    const bool head = col0 % a.d_I == 0;   // this workgroup also computes head col0 / d_I
    const int hidx = col0 / a.d_I;
    const int j = lane & 15, g = lane >> 4;

    // normalized keys: rows row0 + i, i = blockIdx.x, blockIdx.x + n_qt, ...
    for (int i = blockIdx.x + n_qt * w; i < C::XR; i += n_qt * kPWaves)
        if (row0 + i < a.rows) rms_norm_row(a, row0 + i, lane);

    // This wave's DMA instructions: numbers w, w+8, ... of the stage's INS (the
    // head row's instruction, number INS-1, only in head workgroups).  Stage
    // row r is weight row col0 + r (r < 32), hidden-state row row0 + r - 32,
    // or head row; rows past the end load row 0 and are never stored.
    constexpr int MAXI = (C::INS + kPWaves - 1) / kPWaves;
    const uint16_t* src[MAXI];
    int n_ins = 0;
#pragma unroll
    for (int t = 0; t < MAXI; ++t) {
        const int ins = w + kPWaves * t;
        const int r = 2 * ins + (lane >> 5);
        const int q = (lane & 31) ^ (r & 15);
        const uint16_t* row;
        if (r < kPCols) {
            const int n = col0 + r;
            row = a.w_q + (int64_t)n * a.d_x;
        } else if (r < kPCols + C::XR) {
            const int m = row0 + r - kPCols;
            row = a.x + (int64_t)(m < a.rows ? m : 0) * a.d_x;
        } else {
            row = a.w_h + (int64_t)(hidx < a.H_I ? hidx : 0) * a.d_x;
        }
        src[t] = row + 8 * q;
        const bool use = ins < C::INS - 1 || (ins == C::INS - 1 && head);
        n_ins += use ? 1 : 0;
    }
    const uint32_t base = lds_addr(lds);
    auto issue = [&](int st, int slot) {
        const int kb = st * kPStage;
#pragma unroll
        for (int t = 0; t < MAXI; ++t)
            if (t < n_ins)
                lds_gather16(src[t] + kb, (uint32_t)__builtin_amdgcn_readfirstlane(
                                              (int)(base + slot * C::STAGE + (w + kPWaves * t) * 1024)));
    };

    f32x4 acc[MT][3];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 3; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // operand reads of lane (g, j) for slice w: piece 4w + g of row j of a tile
    const int piece = (4 * w + g) ^ j;
    const int nst = a.d_x / kPStage;
#pragma unroll
    for (int s = 0; s < C::S - 1; ++s)
        if (s < nst) issue(s, s);
    for (int st = 0; st < nst; ++st) {
        const int after = min(C::S - 2, nst - 1 - st);  // stages issued after st
        wait_vmcnt(after * n_ins);
        sync_lds();
        if (st + C::S - 1 < nst) issue(st + C::S - 1, (st + C::S - 1) % C::S);
        const unsigned char* sb = lds + (st % C::S) * C::STAGE;
        bf16x8 B[3], A[MT];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
            B[nt] = *reinterpret_cast<const bf16x8*>(sb + (nt * 16 + j) * kPRowB + piece * 16);
        B[2] = *reinterpret_cast<const bf16x8*>(sb + (kPCols + C::XR) * kPRowB + (4 * w + g) * 16);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            A[mt] = *reinterpret_cast<const bf16x8*>(sb + (kPCols + mt * 16 + j) * kPRowB + piece * 16);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            acc[mt][0] = mfma_bf16(A[mt], B[0], acc[mt][0]);
            acc[mt][1] = mfma_bf16(A[mt], B[1], acc[mt][1]);
            if (head) acc[mt][2] = mfma_bf16(A[mt], B[2], acc[mt][2]);
        }
    }
    sync_lds();  // every wave is done with the ring before it becomes the reduction buffer

    // Partial sums of the eight waves: element (row 4g + i of tile mt, column
    // j of tile nt) sits in register i of lane 16g + j.
    float* red = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[(((w * MT + mt) * 2 + nt) * 4 + i) * kPPad + lane] = acc[mt][nt][i];
    // head weights: column 0 of the third tile (lanes j == 0), after the q partials
    float* redh = red + kPWaves * MT * 2 * 4 * kPPad;
    if (head && j == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) redh[w * C::XR + mt * 16 + 4 * g + i] = acc[mt][2][i];
    }
    __syncthreads();
    if (head && threadIdx.x < C::XR && row0 + (int)threadIdx.x < a.rows) {
        float s = 0.f;
#pragma unroll
        for (int ww = 0; ww < kPWaves; ++ww) s += redh[ww * C::XR + threadIdx.x];
        a.head_w[(int64_t)(row0 + threadIdx.x) * a.H_I + hidx] = s;
    }

    // Thread t finishes MT consecutive columns of one row: row t / TPR of the
    // tile, columns (t % TPR) * MT ...; a row's 32 columns are TPR adjacent lanes.
    constexpr int TPR = kPCols / MT;
    const int t = threadIdx.x;
    const int rho = t / TPR, cb = (t % TPR) * MT;
    const int mt = rho / 16, gg = (rho % 16) / 4, ii = rho % 4;
    float v[MT];
#pragma unroll
    for (int e = 0; e < MT; ++e) {
        const int col = cb + e, nt = col / 16, srcl = 16 * gg + col % 16;
        float s = 0.f;
#pragma unroll
        for (int ww = 0; ww < kPWaves; ++ww) s += red[(((ww * MT + mt) * 2 + nt) * 4 + ii) * kPPad + srcl];
        v[e] = s;
    }
    const int r = row0 + rho;
    const bool live_row = r < a.rows;
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
    const dim3 grid(a.H_I * a.d_I / kPCols, (a.rows + 16 * MT - 1) / (16 * MT));
    if (MT == 1)
        hipLaunchKernelGGL(indexer_prolog_kernel<1>, grid, dim3(kPThreads), 0, st, a);
    else if (MT == 2)
        hipLaunchKernelGGL(indexer_prolog_kernel<2>, grid, dim3(kPThreads), 0, st, a);
    else
        hipLaunchKernelGGL(indexer_prolog_kernel<4>, grid, dim3(kPThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace dsa
