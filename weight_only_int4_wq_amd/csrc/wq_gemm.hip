// Prefill GEMM: y[M][N] = x[M][K] . dequant(Wq)^T on fp16 matrix cores.
//
// Batched inference is the one place the layer is a dense contraction, so
// the weight tiles are dequantized to fp16 and fed to MFMA instructions
// with fp32 accumulators ("AutoAWQ vs The Stack v2" and "AutoAWQ vs Unsloth",
// WQLinear_* paragraphs: a GEMM kernel for batches, dequantizing on the fly
// without materializing fp16 weights in memory).
//
// Tiling: a 256-thread block owns a BM x BN output tile, split over a
// WAVES_M x WAVES_N grid of wavefronts; K advances in stages of 128.
//  - A (activations): each stage's BM x 128 fp16 tile goes through LDS,
//    written in the decoder's pair order, and is read back as
//    v_mfma_f32_16x16x32_f16 A fragments (16 rows x 32 k).  A is double
//    buffered in LDS (one barrier per stage) and the next stage's global
//    loads of A and B are issued before this stage's MFMAs.
//  - B (weights): for v_mfma_f32_16x16x32_f16 a lane holds 8 consecutive k
//    of one output column, which is exactly one 8-code block of the packed
//    row.  Each lane therefore loads its own packed chunk (32 codes: 4
//    blocks = the 4 MFMA k-steps of the stage), dequantizes it in registers
//    with the exact (q - z) * s arithmetic, and uses the result directly as B
//    fragments: the dequantized tile lives in registers rather than LDS.
//    Lane group g (lanes 16g..16g+15) takes chunk g of the stage, and the A
//    fragments are read with the same k mapping, so the k sum is unchanged.
#include "wq_common.h"

namespace {

using namespace wq;

template <int BITS>
__device__ __forceinline__ void load_chunk_b(const uint32_t* p, uint32_t* w) {
    if constexpr (BITS == 4) {
        const u4 v = *reinterpret_cast<const u4*>(p);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else if constexpr (BITS == 8) {
        const u4 a = reinterpret_cast<const u4*>(p)[0];
        const u4 b = reinterpret_cast<const u4*>(p)[1];
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else if constexpr (BITS == 2) {
        typedef uint32_t u2 __attribute__((ext_vector_type(2)));
        const u2 v = *reinterpret_cast<const u2*>(p);
        w[0] = v.x; w[1] = v.y;
    } else {
        w[0] = p[0]; w[1] = p[1]; w[2] = p[2];
    }
}

// B operand of one stage for this lane: the raw packed chunk of each of its
// TN columns plus the group's zero byte and scale bits.  Loads are
// unconditional (out-of-range columns and chunks read row 0, chunk 0) and
// are converted only at use, so the compiler never waits on them early.
template <int BITS, int TN>
struct BStage {
    uint32_t w[TN][BITS];
    uint32_t z[TN], s[TN];
    bool ok[TN];
};

template <int BITS, int TN, bool HAS_Z>
__device__ __forceinline__ void load_b_stage(BStage<BITS, TN>& b, const uint32_t* __restrict__ packed,
                                             const uint16_t* __restrict__ scales,
                                             const uint8_t* __restrict__ zeros, int n_lane0, int N,
                                             size_t row_words, int G, GroupDiv gd, int cg, bool kval) {
    const int cgc = kval ? cg : 0;
    const int g = chunk_group(cgc, gd);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int n = n_lane0 + j * 16;
        const bool ok = kval && n < N;
        const size_t nn = ok ? size_t(n) : 0;
        b.ok[j] = ok;
        load_chunk_b<BITS>(packed + nn * row_words + (size_t)cgc * BITS, b.w[j]);
        b.s[j] = scales[nn * G + g];
        if constexpr (HAS_Z)
            b.z[j] = zeros[nn * G + g];
        else
            b.z[j] = 1u << (BITS - 1);
    }
}

// Activation tile of one stage: A_ITERS 16-byte pieces per thread, loaded
// from clamped addresses; pieces outside the matrix are zeroed when written.
template <int BM, int BK, int A_ITERS>
__device__ __forceinline__ void load_a_stage(u4 (&av)[A_ITERS], uint32_t& amask, const uint16_t* __restrict__ x,
                                             int tid, int m0, int k0, int M, int K) {
    amask = 0;
#pragma unroll
    for (int i = 0; i < A_ITERS; ++i) {
        const int t = tid + 256 * i;
        const int row = t / (BK / 8), blk = t % (BK / 8);
        const int gm = m0 + row, gk = k0 + 8 * blk;
        const bool ok = gm < M && gk < K;
        amask |= ok ? (1u << i) : 0u;
        const size_t off = ok ? (size_t)gm * K + gk : 0;
        av[i] = *reinterpret_cast<const u4*>(x + off);
    }
}

template <int BITS, int BM, int BN, int WAVES_M, bool HAS_Z>
__global__ void __launch_bounds__(256) gemm_kernel(const uint16_t* __restrict__ x,
                                                   const uint32_t* __restrict__ packed,
                                                   const uint16_t* __restrict__ scales,
                                                   const uint8_t* __restrict__ zeros, uint16_t* __restrict__ y,
                                                   int M, int N, int K, int gs, GroupDiv gd) {
    constexpr int WAVES_N = 4 / WAVES_M;
    constexpr int BK = 128;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int LDA = BK + 8;              // halves per LDS row: 16-byte pad
    constexpr int A_ITERS = BM * (BK / 8) / 256;
    static_assert(TM >= 1 && TN >= 1 && A_ITERS >= 1, "tile shape");

    // Two A buffers: stage s is written to buffer s & 1 while the other one
    // may still be read by slower wavefronts of stage s - 1.
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDA];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int li = lane & 15, lg = lane >> 4;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int G = K / gs;
    const int chunks = K / 32;
    const size_t row_words = (size_t)chunks * BITS;
    const int n_lane0 = n0 + wn * WN + li;
    const int stages = (K + BK - 1) / BK;

    f4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

    u4 av[A_ITERS];
    uint32_t amask;
    BStage<BITS, TN> bnext;
    load_a_stage<BM, BK, A_ITERS>(av, amask, x, tid, m0, 0, M, K);
    load_b_stage<BITS, TN, HAS_Z>(bnext, packed, scales, zeros, n_lane0, N, row_words, G, gd, lg, lg < chunks);

    for (int st = 0; st < stages; ++st) {
        uint16_t* Ab = As[st & 1];
        // ---- activations of this stage: registers -> LDS, in pair order
#pragma unroll
        for (int i = 0; i < A_ITERS; ++i) {
            const int t = tid + 256 * i;
            const int row = t / (BK / 8), blk = t % (BK / 8);
            const u4 v = ((amask >> i) & 1u) ? av[i] : u4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u4*>(Ab + row * LDA + 8 * blk) = stage_block(v);
        }
        const BStage<BITS, TN> bcur = bnext;
        // ---- next stage's global loads stay in flight during this stage's MFMAs
        if (st + 1 < stages) {
            const int k1 = (st + 1) * BK;
            load_a_stage<BM, BK, A_ITERS>(av, amask, x, tid, m0, k1, M, K);
            const int cg = k1 / 32 + lg;
            load_b_stage<BITS, TN, HAS_Z>(bnext, packed, scales, zeros, n_lane0, N, row_words, G, gd, cg,
                                          cg < chunks);
        }
        __syncthreads();

        uint32_t h[TN][16], zz[TN], ss[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            decode_chunk<BITS>(bcur.w[j], h[j]);
            zz[j] = zero_pair(bcur.z[j]);
            ss[j] = bcur.ok[j] ? scale_pair(uint16_t(bcur.s[j])) : 0u;  // zero weight outside the matrix
        }
        // ---- 4 k-steps of 32: dequantize block s of every chunk, then MFMA
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            h8 bf[TN];
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                uint32_t f[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) f[i] = as_u32(dequant_pair(h[j][4 * s + i], zz[j], ss[j]));
                const u4 fv = {f[0], f[1], f[2], f[3]};
                bf[j] = __builtin_bit_cast(h8, fv);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wm * WM + i * 16 + li;
                const h8 a = *reinterpret_cast<const h8*>(Ab + row * LDA + 32 * lg + 8 * s);
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bf[j], acc[i][j], 0, 0, 0);
            }
        }
    }

    // ---- epilogue: lane holds rows 4*lg + r of column li of each 16x16 tile
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = n0 + wn * WN + j * 16 + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm * WM + i * 16 + 4 * lg + r;
                if (row < M && col < N)
                    y[(size_t)row * N + col] = __builtin_bit_cast(uint16_t, (_Float16)acc[i][j][r]);
            }
        }
}

// x_out[m][k'] = x[m][perm[k']]: activations in packed column order.
__global__ void __launch_bounds__(256) gather_act_kernel(const uint16_t* __restrict__ x,
                                                         const int32_t* __restrict__ perm, int M, int K,
                                                         uint16_t* __restrict__ x_out) {
    const long long total = (long long)M * K;
    for (long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (long long)gridDim.x * blockDim.x) {
        const long long m = t / K;
        const int kp = int(t - m * K);
        x_out[t] = x[m * K + perm[kp]];
    }
}

template <int BITS, int BM, int BN, int WAVES_M>
wq_status launch_tile(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                      uint16_t* y, int M, int N, int K, int gs, hipStream_t s) {
    const dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
    const GroupDiv gd = wqh::group_magic(gs);
    if (zeros)
        hipLaunchKernelGGL((gemm_kernel<BITS, BM, BN, WAVES_M, true>), grid, dim3(256), 0, s, x, packed, scales, zeros,
                           y, M, N, K, gs, gd);
    else
        hipLaunchKernelGGL((gemm_kernel<BITS, BM, BN, WAVES_M, false>), grid, dim3(256), 0, s, x, packed, scales,
                           zeros, y, M, N, K, gs, gd);
    return wqh::launch_status();
}

template <int BITS>
wq_status launch_bits(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                      uint16_t* y, int M, int N, int K, int gs, hipStream_t s) {
    if (M <= 32) return launch_tile<BITS, 32, 128, 2>(x, packed, scales, zeros, y, M, N, K, gs, s);
    if (M <= 64) return launch_tile<BITS, 64, 128, 2>(x, packed, scales, zeros, y, M, N, K, gs, s);
    if (M <= 128) return launch_tile<BITS, 128, 128, 2>(x, packed, scales, zeros, y, M, N, K, gs, s);
    return launch_tile<BITS, 256, 128, 2>(x, packed, scales, zeros, y, M, N, K, gs, s);
}

}  // namespace

namespace wqh {
wq_status check_linear_args(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint16_t* y,
                            int M, int N, int K, int bits, int group_size, int* gs_out);
}

extern "C" size_t wq_workspace_size(int32_t M, int32_t K, int32_t has_perm) {
    if (!has_perm || M <= 0 || K <= 0) return 0;
    return size_t(M) * size_t(K) * 2;
}

extern "C" wq_status wq_gemm(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                             const int32_t* perm, uint16_t* y, int32_t M, int32_t N, int32_t K, int32_t bits,
                             int32_t group_size, void* workspace, size_t workspace_bytes, void* stream) {
    int gs = 0;
    const wq_status st = wqh::check_linear_args(x, packed, scales, y, M, N, K, bits, group_size, &gs);
    if (st != WQ_OK) return st;
    if (M == 0 || N == 0) return WQ_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint16_t* xa = x;
    if (perm) {
        const size_t need = wq_workspace_size(M, K, 1);
        if (!workspace || workspace_bytes < need || !wqh::aligned16(workspace)) return WQ_ERR_ARG;
        uint16_t* xg = static_cast<uint16_t*>(workspace);
        long long total = (long long)M * K;
        long long blocks = (total + 255) / 256;
        if (blocks > 65536) blocks = 65536;
        hipLaunchKernelGGL(gather_act_kernel, dim3(int(blocks)), dim3(256), 0, s, x, perm, int(M), int(K), xg);
        const wq_status ls = wqh::launch_status();
        if (ls != WQ_OK) return ls;
        xa = xg;
    }
    switch (bits) {
        case 2: return launch_bits<2>(xa, packed, scales, zeros, y, M, N, K, gs, s);
        case 3: return launch_bits<3>(xa, packed, scales, zeros, y, M, N, K, gs, s);
        case 4: return launch_bits<4>(xa, packed, scales, zeros, y, M, N, K, gs, s);
        default: return launch_bits<8>(xa, packed, scales, zeros, y, M, N, K, gs, s);
    }
}
