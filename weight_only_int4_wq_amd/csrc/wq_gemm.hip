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
//    v_mfma_f32_16x16x32_f16 A fragments (16 rows x 32 k).
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

template <int BITS, int BM, int BN, int WAVES_M>
__global__ void __launch_bounds__(256) gemm_kernel(const uint16_t* __restrict__ x,
                                                   const uint32_t* __restrict__ packed,
                                                   const uint16_t* __restrict__ scales,
                                                   const uint8_t* __restrict__ zeros, uint16_t* __restrict__ y,
                                                   int M, int N, int K, int gs) {
    constexpr int WAVES_N = 4 / WAVES_M;
    constexpr int BK = 128;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int LDA = BK + 8;              // halves per LDS row: 16-byte pad
    constexpr int A_ITERS = BM * (BK / 8) / 256;
    static_assert(TM >= 1 && TN >= 1 && A_ITERS >= 1, "tile shape");

    __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDA];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int li = lane & 15, lg = lane >> 4;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int G = K / gs;
    const int chunks = K / 32;
    const size_t row_words = (size_t)chunks * BITS;

    f4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < K; k0 += BK) {
        // ---- B: this lane's packed chunk of each of its TN columns
        const int cg = k0 / 32 + lg;
        const bool kval = cg < chunks;
        uint32_t bw[TN][BITS];
        uint32_t zz[TN], ss[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = n0 + wn * WN + j * 16 + li;
            if (kval && n < N) {
                load_chunk_b<BITS>(packed + (size_t)n * row_words + (size_t)cg * BITS, bw[j]);
                const int g = (cg * 32) / gs;
                const uint32_t z = zeros ? uint32_t(zeros[(size_t)n * G + g]) : (1u << (BITS - 1));
                zz[j] = zero_pair(z);
                ss[j] = scale_pair(scales[(size_t)n * G + g]);
            } else {
#pragma unroll
                for (int i = 0; i < BITS; ++i) bw[j][i] = 0u;
                zz[j] = zero_pair(0);
                ss[j] = 0u;  // zero weight outside the matrix
            }
        }
        // ---- A: global -> registers
        u4 av[A_ITERS];
#pragma unroll
        for (int i = 0; i < A_ITERS; ++i) {
            const int t = tid + 256 * i;
            const int row = t / (BK / 8), blk = t % (BK / 8);
            const int gm = m0 + row, gk = k0 + 8 * blk;
            if (gm < M && gk < K)
                av[i] = *reinterpret_cast<const u4*>(x + (size_t)gm * K + gk);
            else
                av[i] = u4{0u, 0u, 0u, 0u};
        }
        __syncthreads();  // previous stage's fragments have been read
#pragma unroll
        for (int i = 0; i < A_ITERS; ++i) {
            const int t = tid + 256 * i;
            const int row = t / (BK / 8), blk = t % (BK / 8);
            *reinterpret_cast<u4*>(As + row * LDA + 8 * blk) = stage_block(av[i]);
        }
        __syncthreads();

        // ---- dequantize B fragments: bf[j][s] = 8 fp16 of k-step s
        h8 bf[TN][4];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            uint32_t h[16];
            decode_chunk<BITS>(bw[j], h);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                uint32_t f[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) f[i] = as_u32(dequant_pair(h[4 * s + i], zz[j], ss[j]));
                u4 fv = {f[0], f[1], f[2], f[3]};
                bf[j][s] = __builtin_bit_cast(h8, fv);
            }
        }
        // ---- MFMA over the 4 k-steps of the stage
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wm * WM + i * 16 + li;
                const h8 a = *reinterpret_cast<const h8*>(As + row * LDA + 32 * lg + 8 * s);
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bf[j][s], acc[i][j], 0, 0, 0);
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
    hipLaunchKernelGGL((gemm_kernel<BITS, BM, BN, WAVES_M>), grid, dim3(256), 0, s, x, packed, scales, zeros, y, M,
                       N, K, gs);
    return wqh::launch_status();
}

template <int BITS>
wq_status launch_bits(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                      uint16_t* y, int M, int N, int K, int gs, hipStream_t s) {
    if (M <= 32) return launch_tile<BITS, 32, 128, 2>(x, packed, scales, zeros, y, M, N, K, gs, s);
    return launch_tile<BITS, 128, 128, 2>(x, packed, scales, zeros, y, M, N, K, gs, s);
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
