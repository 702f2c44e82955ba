// GPTQ ("GPTQ, AWQ and the rules of post-training quantization", section
// "GPTQ: pay for the error with the other weights"): the columns of W are
// quantized one at a time in a fixed order (index order), and each column's
// rounding error is compensated on the columns not yet quantized through
// the inverse Hessian of the layer's reconstruction loss, written with a
// Cholesky factor; the compensation is applied lazily, a block of 64
// columns at a time, so most of the work is a matrix product.
//
//   H = x^T x (float32 sums of fp16 products on the matrix cores); a
//   channel with H[k][k] = 0 gets
//   H[k][k] = 1 and a zero weight column; H += damp * mean(diag H) * I.
//   U = the upper Cholesky factor of H^-1 (H^-1 = U^T U), computed as
//   U = P L^-1 P with L L^T = P H P and P the index reversal, the factor
//   and its inverse together, right-looking in blocks of 64 (fp32 matrix-core
//   products for everything but the 64 x 64 diagonal blocks).
//   For each block of 64 columns, one thread per weight row walks the
//   block's columns in order: at the first column of a group, the RTN scale
//   and zero from the group's running weights; the column's code and
//   dequantized weight; err = (w - w_hat) / U[i][i]; the block's later
//   columns -= err * U[i][j].  Then the columns after the block receive all
//   of the block's errors at once: W[:, after] -= Err . U[block, after].
//
// Everything runs in float32 on the GPU; the oracle follows the same steps
// in float64 (unblocked), so the two agree in distribution, not bit for bit.
#include <math.h>

#include "wq_gemm_common.h"

namespace {

using namespace wq;

__device__ __forceinline__ float h2f(uint16_t h) { return float(__builtin_bit_cast(_Float16, h)); }
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

constexpr int kGptqB = 64;   // columns walked by one launch
constexpr int kGptqOuter = 256;  // outer lazy-update block

// ------------------------------------------------------------ helpers ----

// xt[k][m] = x[m][k] (fp16), 32 x 32 tiles through LDS.
__global__ void __launch_bounds__(256) transpose_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                        uint16_t* __restrict__ xt) {
    __shared__ uint16_t t[32][33];
    const int m0 = blockIdx.y * 32, k0 = blockIdx.x * 32;
    for (int e = threadIdx.x; e < 1024; e += 256) {
        const int r = e / 32, c = e % 32;
        const int m = m0 + r, k = k0 + c;
        t[r][c] = (m < M && k < K) ? x[(size_t)m * K + k] : uint16_t(0);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 1024; e += 256) {
        const int r = e / 32, c = e % 32;
        const int k = k0 + r, m = m0 + c;
        if (k < K && m < M) xt[(size_t)k * M + m] = t[c][r];
    }
}

// Dead channels and damping, one block, fixed order: dead[k] = (H[k][k] == 0),
// those diagonals become 1 (copied to diag, the act-order key), then every
// diagonal gains damp * mean(diag).
__global__ void __launch_bounds__(1024) damp_kernel(float* __restrict__ H, int K, float damp,
                                                    uint8_t* __restrict__ dead, float* __restrict__ diag) {
    __shared__ float part[1024];
    float acc = 0.f;
    for (int k = threadIdx.x; k < K; k += 1024) {
        float d = H[(size_t)k * K + k];
        const bool z = d == 0.f;
        dead[k] = z ? 1 : 0;
        if (z) d = 1.f;
        H[(size_t)k * K + k] = d;
        diag[k] = d;
        acc += d;
    }
    part[threadIdx.x] = acc;
    __syncthreads();
    for (int h = 512; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) part[threadIdx.x] += part[threadIdx.x + h];
        __syncthreads();
    }
    const float lambda = damp * (part[0] / float(K));
    for (int k = threadIdx.x; k < K; k += 1024) H[(size_t)k * K + k] += lambda;
}

// dst[i][j] = src[K-1-i][K-1-j] for j >= i, 0 below the diagonal (both
// K x K float32; only src's lower triangle is read).
__global__ void __launch_bounds__(256) upper_reverse_kernel(const float* __restrict__ src, int K,
                                                            float* __restrict__ dst) {
    const long long total = (long long)K * K;
    for (long long t = (long long)blockIdx.x * 256 + threadIdx.x; t < total; t += (long long)gridDim.x * 256) {
        const int i = int(t / K), j = int(t % K);
        dst[t] = j >= i ? src[(size_t)(K - 1 - i) * K + (K - 1 - j)] : 0.f;
    }
}

// Sort key of a float under a total order: the bit pattern mapped so that
// unsigned comparison follows the float order (-inf < ... < -0 < +0 < ...
// < +inf), with every NaN below all numbers.
__device__ __forceinline__ uint32_t order_key(float v) {
    const uint32_t b = __builtin_bit_cast(uint32_t, v);
    if (v != v) return 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Processing order: perm[i] = the channel of rank i.  With act-order the
// rank is the position in descending diag order, ties by channel index (a
// stable sort); otherwise the identity.  The comparison is a strict total
// order on (key, index), so the ranks are a permutation of 0..K-1 even when
// the diagonal holds NaN (from non-finite calibration data): every perm slot
// is written exactly once.
__global__ void __launch_bounds__(256) rank_kernel(const float* __restrict__ diag, int K, int act_order,
                                                   int32_t* __restrict__ perm) {
    const int k = blockIdx.x * 256 + threadIdx.x;
    if (k >= K) return;
    if (!act_order) {
        perm[k] = k;
        return;
    }
    const uint32_t d = order_key(diag[k]);
    int rank = 0;
    for (int j = 0; j < K; ++j) {
        const uint32_t e = order_key(diag[j]);
        rank += (e > d || (e == d && j < k)) ? 1 : 0;
    }
    perm[rank] = k;
}

// dst[i][j] = H[perm[K-1-i]][perm[K-1-j]]: the Hessian in processing order,
// index-reversed.
__global__ void __launch_bounds__(256) permute_reverse_kernel(const float* __restrict__ H,
                                                              const int32_t* __restrict__ perm, int K,
                                                              float* __restrict__ dst) {
    const long long total = (long long)K * K;
    for (long long t = (long long)blockIdx.x * 256 + threadIdx.x; t < total; t += (long long)gridDim.x * 256) {
        const int i = int(t / K), j = int(t % K);
        dst[t] = H[(size_t)perm[K - 1 - i] * K + perm[K - 1 - j]];
    }
}

// W32[n][i] = fp32(w[n][perm[i]]), 0 on dead channels (columns in
// processing order).
__global__ void __launch_bounds__(256) init_w_kernel(const uint16_t* __restrict__ w, const uint8_t* __restrict__ dead,
                                                     const int32_t* __restrict__ perm, long long total, int K,
                                                     float* __restrict__ W32) {
    for (long long t = (long long)blockIdx.x * 256 + threadIdx.x; t < total; t += (long long)gridDim.x * 256) {
        const long long n = t / K;
        const int k = perm[int(t % K)];
        W32[t] = dead[k] ? 0.f : h2f(w[n * K + k]);
    }
}

// The same without act-order (processing order = channel order): eight
// columns per thread, 16-byte loads and stores (K a multiple of 8, w
// 16-byte aligned).
__global__ void __launch_bounds__(256) init_w_vec_kernel(const uint16_t* __restrict__ w,
                                                         const uint8_t* __restrict__ dead, long long total8, int K,
                                                         float* __restrict__ W32) {
    for (long long t = (long long)blockIdx.x * 256 + threadIdx.x; t < total8; t += (long long)gridDim.x * 256) {
        const long long e = 8 * t;
        const int k0 = int(e % K);
        const u4 v = *reinterpret_cast<const u4*>(w + e);
        const uint32_t in[4] = {v.x, v.y, v.z, v.w};
        float o[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = dead[k0 + 2 * i] ? 0.f : h2f(uint16_t(in[i]));
            o[2 * i + 1] = dead[k0 + 2 * i + 1] ? 0.f : h2f(uint16_t(in[i] >> 16));
        }
        *reinterpret_cast<f4*>(W32 + e) = f4{o[0], o[1], o[2], o[3]};
        *reinterpret_cast<f4*>(W32 + e + 4) = f4{o[4], o[5], o[6], o[7]};
    }
}

// codes[n][perm[i]] = cp[n][i] and g_idx[perm[i]] = i / gs (act-order).
__global__ void __launch_bounds__(256) unpermute_kernel(const uint8_t* __restrict__ cp, const int32_t* __restrict__ perm,
                                                        long long total, int K, int gs, uint8_t* __restrict__ codes,
                                                        int32_t* __restrict__ g_idx) {
    for (long long t = (long long)blockIdx.x * 256 + threadIdx.x; t < total; t += (long long)gridDim.x * 256) {
        const long long n = t / K;
        const int i = int(t % K);
        codes[n * K + perm[i]] = cp[t];
        if (n == 0) g_idx[perm[i]] = i / gs;
    }
}

// acc = A . opB for one 64 x 64 tile in float32 on the matrix cores
// (v_mfma_f32_16x16x4f32), opB(k, j) = TB ? B[j][k] : B[k][j]; A points at
// the tile's first row, B at its first column (TB: first row); mlim and nlim
// are the rows and columns of the tile that exist, Kd (a multiple of 4) the
// depth.  256 threads, each wavefront a 32 x 32 quarter (2 x 2
// instructions); k in steps of 32 through LDS, A as As[m][k] and opB as
// Bs[n][k] so that a lane reads four consecutive k of its row with one
// 16-byte load.  The four instructions of one such load take
// k = 4 * (lane / 16) + t for t = 0..3 in A and B alike: a permutation of
// the sum's terms.
constexpr int kTileLd = 36;  // LDS row stride in floats: 16-byte aligned, spreads banks

template <bool TB>
__device__ __forceinline__ void tile_acc(f4 (&acc)[2][2], const float* __restrict__ A, int lda,
                                         const float* __restrict__ B, int ldb, int mlim, int nlim, int Kd,
                                         float* __restrict__ As, float* __restrict__ Bs) {
    constexpr int LD = kTileLd;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < Kd; k0 += 32) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int e = tid + 256 * q;
            {
                const int r = e >> 5, k = e & 31;  // A: consecutive k per row
                const int gk = k0 + k;
                As[r * LD + k] = (r < mlim && gk < Kd) ? A[(size_t)r * lda + gk] : 0.f;
            }
            if (TB) {
                const int n = e >> 5, k = e & 31;  // B[n][k]: consecutive k
                const int gk = k0 + k;
                Bs[n * LD + k] = (n < nlim && gk < Kd) ? B[(size_t)n * ldb + gk] : 0.f;
            } else {
                const int k = e >> 6, n = e & 63;  // B[k][n]: consecutive n
                const int gk = k0 + k;
                Bs[n * LD + k] = (n < nlim && gk < Kd) ? B[(size_t)gk * ldb + n] : 0.f;
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 32; kk += 16) {
            f4 a[2], b[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                a[t] = *reinterpret_cast<const f4*>(&As[(wm + 16 * t + li) * LD + kk + 4 * lg]);
                b[t] = *reinterpret_cast<const f4*>(&Bs[(wn + 16 * t + li) * LD + kk + 4 * lg]);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][t], b[j][t], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }
}

// C = beta * C + alpha * acc on the tile at C (beta = 0: C is not read;
// beta = 1: an atomic add in L2, one per element, the same rounded sum
// without a read).  A lane holds rows 4 * (lane / 16) + r of column
// lane % 16 of each 16 x 16 block.
__device__ __forceinline__ void tile_store(const f4 (&acc)[2][2], float* __restrict__ C, int ldc, int mlim, int nlim,
                                           float alpha, float beta) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = wn + 16 * j + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = wm + 16 * i + 4 * lg + r;
                if (m < mlim && n < nlim) {
                    float* p = C + (size_t)m * ldc + n;
                    if (beta == 1.f)
                        unsafeAtomicAdd(p, alpha * acc[i][j][r]);
                    else
                        *p = (beta == 0.f ? 0.f : beta * *p) + alpha * acc[i][j][r];
                }
            }
        }
}

// C = beta * C + alpha * A . opB for one 64 x 64 tile of depth Kd <= 64
// (a multiple of 4) in one shot: the tile's A, opB and C are requested with
// 16-byte loads before anything waits (lda, ldb, ldc, nlim multiples of 4,
// pointers 16-byte aligned), both operands go to LDS whole (A as As[m][k],
// opB as Bs[n][k]), v_mfma_f32_16x16x4f32 as in tile_acc, and the result
// returns through LDS so that C is written with 16-byte stores too.  256
// threads; smem: 2 * 64 * 68 floats.  Thread t moves the four 16-byte
// pieces (row t / 16 + 16 q, columns 4 (t % 16) ..).
constexpr int kShotLd = 68;
constexpr int kShotSmem = 2 * 64 * kShotLd;

template <bool TB>
__device__ __forceinline__ void tile_shot(const float* __restrict__ A, int lda, const float* __restrict__ B, int ldb,
                                          float* __restrict__ C, int ldc, int mlim, int nlim, int Kd, float alpha,
                                          float beta, float* __restrict__ smem) {
    constexpr int LD = kShotLd;
    float* As = smem;
    float* Bs = smem + 64 * LD;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int pr = tid >> 4, p4 = 4 * (tid & 15);
    const f4 zero = {0.f, 0.f, 0.f, 0.f};
    f4 ra[4], rb[4], rc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = pr + 16 * q;
        ra[q] = (r < mlim && p4 < Kd) ? *reinterpret_cast<const f4*>(A + (size_t)r * lda + p4) : zero;
        if (TB)  // B[n][k]: row n = r, k = p4
            rb[q] = (r < nlim && p4 < Kd) ? *reinterpret_cast<const f4*>(B + (size_t)r * ldb + p4) : zero;
        else     // B[k][n]: row k = r, n = p4
            rb[q] = (r < Kd && p4 < nlim) ? *reinterpret_cast<const f4*>(B + (size_t)r * ldb + p4) : zero;
        rc[q] = (beta != 0.f && r < mlim && p4 < nlim) ? *reinterpret_cast<const f4*>(C + (size_t)r * ldc + p4)
                                                       : zero;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = pr + 16 * q;
        *reinterpret_cast<f4*>(&As[r * LD + p4]) = ra[q];
        if (TB) {
            *reinterpret_cast<f4*>(&Bs[r * LD + p4]) = rb[q];
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) Bs[(p4 + t) * LD + r] = rb[q][t];
        }
    }
    __syncthreads();
    const int li = lane & 15, lg = lane >> 4;
    const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
    f4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = zero;
    for (int kk = 0; kk < Kd; kk += 16) {
        f4 a[2], b[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            a[t] = *reinterpret_cast<const f4*>(&As[(wm + 16 * t + li) * LD + kk + 4 * lg]);
            b[t] = *reinterpret_cast<const f4*>(&Bs[(wn + 16 * t + li) * LD + kk + 4 * lg]);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][t], b[j][t], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
    // lane holds rows 4 * lg + r of column li of each 16 x 16 block
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) As[(wm + 16 * i + 4 * lg + r) * LD + wn + 16 * j + li] = acc[i][j][r];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = pr + 16 * q;
        if (r < mlim && p4 < nlim) {
            const f4 v = *reinterpret_cast<const f4*>(&As[r * LD + p4]);
            f4 o;
#pragma unroll
            for (int t = 0; t < 4; ++t) o[t] = (beta == 0.f ? 0.f : beta * rc[q][t]) + alpha * v[t];
            *reinterpret_cast<f4*>(C + (size_t)r * ldc + p4) = o;
        }
    }
}

// C = beta * C + alpha * A . B (NN), depth Kd <= 64, one shot per 64 x 64
// tile (the column walk's updates inside an outer block).
__global__ void __launch_bounds__(256) sgemm_shot_kernel(int M, int N, int Kd, float alpha, const float* __restrict__ A,
                                                         int lda, const float* __restrict__ B, int ldb, float beta,
                                                         float* __restrict__ C, int ldc) {
    __shared__ __align__(16) float smem[kShotSmem];
    const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
    tile_shot<false>(A + (size_t)i0 * lda, lda, B + j0, ldb, C + (size_t)i0 * ldc + j0, ldc, M - i0, N - j0, Kd, alpha,
                     beta, smem);
}

// C = beta * C + alpha * A . opB (leading dimensions lda, ldb, ldc), a
// 64 x 64 output tile per 256-thread block.
template <bool TB>
__global__ void __launch_bounds__(256) sgemm_kernel(int M, int N, int Kd, float alpha, const float* __restrict__ A,
                                                    int lda, const float* __restrict__ B, int ldb, float beta,
                                                    float* __restrict__ C, int ldc) {
    __shared__ float As[64 * kTileLd];
    __shared__ float Bs[64 * kTileLd];
    const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
    f4 acc[2][2];
    tile_acc<TB>(acc, A + (size_t)i0 * lda, lda, TB ? B + (size_t)j0 * ldb : B + j0, ldb, M - i0, N - j0, Kd, As, Bs);
    tile_store(acc, C + (size_t)i0 * ldc + j0, ldc, M - i0, N - j0, alpha, beta);
}

template <bool TB>
wq_status sgemm(int M, int N, int Kd, float alpha, const float* A, int lda, const float* B, int ldb, float beta,
                float* C, int ldc, hipStream_t s) {
    if (M <= 0 || N <= 0) return WQ_OK;
    if (Kd % 4 != 0) return WQ_ERR_ARG;
    hipLaunchKernelGGL((sgemm_kernel<TB>), dim3((N + 63) / 64, (M + 63) / 64), dim3(256), 0, s, M, N, Kd, alpha, A,
                       lda, B, ldb, beta, C, ldc);
    return wqh::launch_status();
}

// C = beta * C + alpha * A . B (B as B[k][n]) for the column walk's large
// products: 128 x 128 output tiles per 256-thread block, each wavefront a
// 64 x 64 quarter of 2 x 2 v_mfma_f32_32x32x2f32 blocks.  k in stages of
// 32 through LDS (A as As[m][k], B as Bs[k][n], both written with 16-byte
// stores); the next stage's 16-byte global loads are issued into registers
// before the current stage's products.  A lane reads four consecutive k of
// its A row with one 16-byte load; instruction t of such a load takes
// k = 4 * (lane / 32) + t in A and B alike (a permutation of the sum's
// terms).  Needs N, lda, ldb and Kd multiples of 4 and A, B 16-byte
// aligned.  With beta = 1 the result goes to C by atomic adds (one per
// element and launch, so the sum is the same; C is not read).
typedef float f16v __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(256) sgemm128_kernel(int M, int N, int Kd, float alpha, const float* __restrict__ A,
                                                       int lda, const float* __restrict__ B, int ldb, float beta,
                                                       float* __restrict__ C, int ldc) {
    constexpr int LDA = 36, LDB = 132;
    __shared__ __align__(16) float As[128 * LDA];
    __shared__ __align__(16) float Bs[32 * LDB];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, h = lane >> 5;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    const int i0 = blockIdx.y * 128, j0 = blockIdx.x * 128;
    f16v acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    f4 ra[4], rb[4];
    auto gload = [&](int k0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = tid + 256 * q;
            const int r = e >> 3, ka = k0 + 4 * (e & 7);
            ra[q] = (i0 + r < M && ka < Kd) ? *reinterpret_cast<const f4*>(A + (size_t)(i0 + r) * lda + ka)
                                            : f4{0.f, 0.f, 0.f, 0.f};
            const int kb = k0 + (e >> 5), n = j0 + 4 * (e & 31);
            rb[q] = (kb < Kd && n < N) ? *reinterpret_cast<const f4*>(B + (size_t)kb * ldb + n)
                                       : f4{0.f, 0.f, 0.f, 0.f};
        }
    };
    gload(0);
    for (int k0 = 0; k0 < Kd; k0 += 32) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = tid + 256 * q;
            *reinterpret_cast<f4*>(&As[(e >> 3) * LDA + 4 * (e & 7)]) = ra[q];
            *reinterpret_cast<f4*>(&Bs[(e >> 5) * LDB + 4 * (e & 31)]) = rb[q];
        }
        __syncthreads();
        if (k0 + 32 < Kd) gload(k0 + 32);
#pragma unroll
        for (int kk = 0; kk < 32; kk += 8) {
            f4 a[2];
            float b[2][4];
#pragma unroll
            for (int i = 0; i < 2; ++i) a[i] = *reinterpret_cast<const f4*>(&As[(wm + 32 * i + l32) * LDA + kk + 4 * h]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int t = 0; t < 4; ++t) b[j][t] = Bs[(kk + 4 * h + t) * LDB + wn + 32 * j + l32];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][t], b[j][t], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }
    // lane holds rows 8 * (r / 4) + 4 * (lane / 32) + r % 4 of column
    // lane % 32 of each 32 x 32 block
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int gj = j0 + wn + 32 * j + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gi = i0 + wm + 32 * i + 8 * (r / 4) + 4 * h + (r % 4);
                if (gi < M && gj < N) {
                    float* p = C + (size_t)gi * ldc + gj;
                    // one addition per element and launch: an atomic add
                    // in L2 gives the same rounded sum without a read
                    if (beta == 1.f)
                        unsafeAtomicAdd(p, alpha * acc[i][j][r]);
                    else
                        *p = (beta == 0.f ? 0.f : beta * *p) + alpha * acc[i][j][r];
                }
            }
        }
}

// NN product: the 128-tile kernel when its alignment holds and it makes at
// least 256 tiles, else the 64-tile one.
wq_status sgemm_nn(int M, int N, int Kd, float alpha, const float* A, int lda, const float* B, int ldb, float beta,
                   float* C, int ldc, hipStream_t s) {
    if (M <= 0 || N <= 0) return WQ_OK;
    if (Kd % 4 != 0) return WQ_ERR_ARG;
    const long long tiles = (long long)((M + 127) / 128) * ((N + 127) / 128);
    if (tiles >= 256 && N % 4 == 0 && lda % 4 == 0 && ldb % 4 == 0 && wqh::aligned16(A) && wqh::aligned16(B)) {
        hipLaunchKernelGGL(sgemm128_kernel, dim3((N + 127) / 128, (M + 127) / 128), dim3(256), 0, s, M, N, Kd, alpha,
                           A, lda, B, ldb, beta, C, ldc);
        return wqh::launch_status();
    }
    return sgemm<false>(M, N, Kd, alpha, A, lda, B, ldb, beta, C, ldc, s);
}

// NN product of depth <= 64 in one shot per tile when the 16-byte rules
// hold, else the staged 64-tile kernel.
wq_status sgemm_shot(int M, int N, int Kd, float alpha, const float* A, int lda, const float* B, int ldb, float beta,
                     float* C, int ldc, hipStream_t s) {
    if (M <= 0 || N <= 0) return WQ_OK;
    if (Kd % 4 != 0) return WQ_ERR_ARG;
    if (Kd <= 64 && N % 4 == 0 && lda % 4 == 0 && ldb % 4 == 0 && ldc % 4 == 0 && wqh::aligned16(A) &&
        wqh::aligned16(B) && wqh::aligned16(C)) {
        hipLaunchKernelGGL(sgemm_shot_kernel, dim3((N + 63) / 64, (M + 63) / 64), dim3(256), 0, s, M, N, Kd, alpha, A,
                           lda, B, ldb, beta, C, ldc);
        return wqh::launch_status();
    }
    return sgemm<false>(M, N, Kd, alpha, A, lda, B, ldb, beta, C, ldc, s);
}

// ------------------------------------------- Cholesky with its inverse ----
//
// Right-looking and blocked by 64 on the K x K matrix A (lower triangle
// valid on entry), with L^-1 built alongside by forward substitution on
// the identity.  Block row / column t covers [64 t, 64 t + 64).  Before
// step j, A's tiles (r, c) with r >= j hold: for c >= j the Schur
// complement of the leading j blocks (lower part), for c < j the partial
// sums B[r][c] = -sum_{k<j} L[r][k] . Li[k][c] of the substitution.  Step j:
//   block:  L_jj = chol(A_jj), Li[j][j] = L_jj^-1;
//   panel:  Li[j][c] = Li_jj . B[j][c] (c < j), L[r][j] = A[r][j] . Li_jj^T
//           (r > j);
//   update: for r > j and c <= r, A[r][c] = (c == j ? 0 : A[r][c]) -
//           L[r][j] . R[c], R[c] = Li[j][c] for c <= j and L[c][j]^T after.
// After the last step Li's lower triangle (diagonal blocks included) is
// L^-1; its upper triangle is never written.  The block step of j + 1 runs
// inside the update launch of step j, in the block of tile (j + 1, j + 1).

// The diagonal block: nb x nb (nb <= 64) at A[j0][j0], lower triangle read
// and mirrored, padded with the identity; writes Li's diagonal block (zeros
// above its diagonal included).  Four wavefronts; lane c of wave w holds
// rows [16 w, 16 w + 16) of column c of the Schur complement (a) and of the
// identity under the same row operations (t).  Step j publishes row j (a's
// entries past j, zeros before; t's in full) and the pivot p = a[j][j]
// (clamped to 1e-30 against rounding), and every row r > j takes
// a[r] -= a[j][r] * (a[j][c] * rcp(p)) and t[r] -= a[j][r] * (t[j][c] *
// rcp(p)), rcp the hardware reciprocal (v_rcp_f32, about 1 ulp): the
// pivot's division sits on the steps' serial chain.  The
// steps go in runs of 16, the pivot rows of one wavefront: that wavefront
// walks the run alone, updating its own rows at each step, and then the
// wavefronts holding later rows apply the run's 16 updates in step order
// (the same operations in the same order per element).  At the end t is
// the inverse of the unit factor and Li[r][c] = t[r][c] / sqrt(p_r); square
// roots are taken only at the end.
// smem: 64 * 65 + 2 * 16 * 64 + 64 floats, 16-byte aligned.  256 threads.
constexpr int kFactorSmem = 64 * 65 + 2 * 16 * 64 + 64;

__device__ __forceinline__ void chol_factor(const float* __restrict__ A, int K, int j0, int nb, float* __restrict__ Li,
                                            float* __restrict__ smem) {
    float* S = smem;
    float(*hA)[64] = reinterpret_cast<float(*)[64]>(smem + 64 * 65);
    float(*hT)[64] = reinterpret_cast<float(*)[64]>(smem + 64 * 65 + 16 * 64);
    float* pd = smem + 64 * 65 + 2 * 16 * 64;
    const int c = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll 4
    for (int q = 0; q < 16; ++q) {
        const int r = w + 4 * q;
        S[r * 65 + c] = (r < nb && c < nb) ? A[(size_t)(j0 + r) * K + j0 + c] : (r == c ? 1.f : 0.f);
    }
    __syncthreads();
    float a[16], t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = 16 * w + i;
        a[i] = r >= c ? S[r * 65 + c] : S[c * 65 + r];
        t[i] = r == c ? 1.f : 0.f;
    }
    for (int jb = 0; jb < 4; ++jb) {
        if (w == jb) {
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const int j = 16 * jb + jj;
                hA[jj][c] = c > j ? a[jj] : 0.f;
                hT[jj][c] = t[jj];
                if (c == j) pd[j] = fmaxf(a[jj], 1e-30f);
                // LDS writes and reads of one wavefront stay in order
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                const float ip = __builtin_amdgcn_rcpf(pd[j]);
                const float fa = hA[jj][c] * ip, ft = hT[jj][c] * ip;
#pragma unroll
                for (int i = jj + 1; i < 16; ++i) {
                    const float m = hA[jj][16 * jb + i];
                    a[i] = fmaf(-m, fa, a[i]);
                    t[i] = fmaf(-m, ft, t[i]);
                }
            }
        }
        __syncthreads();
        if (w > jb) {
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const float ip = __builtin_amdgcn_rcpf(pd[16 * jb + jj]);
                const float fa = hA[jj][c] * ip, ft = hT[jj][c] * ip;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float m = hA[jj][16 * w + i];
                    a[i] = fmaf(-m, fa, a[i]);
                    t[i] = fmaf(-m, ft, t[i]);
                }
            }
        }
        __syncthreads();  // the run's rows are rewritten by the next run
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = 16 * w + i;
        if (r < nb && c < nb) Li[(size_t)(j0 + r) * K + j0 + c] = t[i] * (1.f / sqrtf(pd[r]));
    }
}

// The first diagonal block on its own; every later one is factored by the
// previous step's update (chol_update_kernel).
__global__ void __launch_bounds__(256) chol_block_kernel(const float* __restrict__ A, int K, int j0, int nb,
                                                         float* __restrict__ Li) {
    __shared__ __align__(16) float smem[kFactorSmem];
    chol_factor(A, K, j0, nb, Li, smem);
}

// The panel of step j: block t < j writes Li[j][t], block t > j writes
// L[t][j]; block j does nothing.
__global__ void __launch_bounds__(256) chol_panel_kernel(const float* __restrict__ A, float* __restrict__ L,
                                                         float* __restrict__ Li, int K, int j) {
    __shared__ __align__(16) float smem[kShotSmem];
    const int t = blockIdx.x;
    if (t == j) return;
    const int j0 = 64 * j, t0 = 64 * t;
    const int nbj = min(64, K - j0), nt = min(64, K - t0);
    const float* Lijj = Li + (size_t)j0 * K + j0;
    if (t < j)
        tile_shot<false>(Lijj, K, A + (size_t)j0 * K + t0, K, Li + (size_t)j0 * K + t0, K, nbj, nt, nbj, 1.f, 0.f, smem);
    else
        tile_shot<true>(A + (size_t)t0 * K + j0, K, Lijj, K, L + (size_t)t0 * K + j0, K, nt, nbj, nbj, 1.f, 0.f, smem);
}

// The update of step j: block (c, r - j - 1) for c <= r (blocks above the
// block diagonal return at once).  The block of tile (j + 1, j + 1), the
// next step's diagonal block, goes on to factor it (its writes are visible
// to the block after a barrier) while the other tiles are updated.
__global__ void __launch_bounds__(256, 3) chol_update_kernel(float* __restrict__ A, const float* __restrict__ L,
                                                             float* __restrict__ Li, int K, int j) {
    __shared__ __align__(16) float smem[kShotSmem > kFactorSmem ? kShotSmem : kFactorSmem];
    const int c = blockIdx.x, r = j + 1 + blockIdx.y;
    if (c > r) return;
    const int j0 = 64 * j, r0 = 64 * r, c0 = 64 * c;
    const int nbj = min(64, K - j0), nr = min(64, K - r0), nc = min(64, K - c0);
    const float* P = L + (size_t)r0 * K + j0;
    float* Ct = A + (size_t)r0 * K + c0;
    const float beta = c == j ? 0.f : 1.f;
    if (c <= j)
        tile_shot<false>(P, K, Li + (size_t)j0 * K + c0, K, Ct, K, nr, nc, nbj, -1.f, beta, smem);
    else
        tile_shot<true>(P, K, L + (size_t)c0 * K + j0, K, Ct, K, nr, nc, nbj, -1.f, beta, smem);
    if (r == j + 1 && c == j + 1) {
        __syncthreads();
        chol_factor(A, K, r0, nr, Li, smem);
    }
}

// Li = L^-1 with L L^T = A (K x K; A is overwritten, L holds the panels).
wq_status chol_inverse(float* A, float* L, float* Li, int K, hipStream_t s) {
    const int T = (K + 63) / 64;
    hipLaunchKernelGGL(chol_block_kernel, dim3(1), dim3(256), 0, s, A, K, 0, min(64, K), Li);
    for (int j = 0; j < T; ++j) {
        if (T > 1) hipLaunchKernelGGL(chol_panel_kernel, dim3(T), dim3(256), 0, s, A, L, Li, K, j);
        if (j + 1 < T) hipLaunchKernelGGL(chol_update_kernel, dim3(T, T - j - 1), dim3(256), 0, s, A, L, Li, K, j);
        const wq_status st = wqh::launch_status();
        if (st != WQ_OK) return st;
    }
    return WQ_OK;
}

// Columns [32 H, 32 H + 32) of a block (see gptq_block_kernel); a group can
// start only at the first of them.
template <int BITS, bool SYM, int BC, int H>
__device__ __forceinline__ void gptq_half(float (&w)[BC], float (&e)[BC], uint32_t (&cw)[BC / 4], float& s, float& z,
                                          const float* __restrict__ us, const float* __restrict__ wrow, int K,
                                          int b0, int gs, int G, int n, bool live, uint16_t* __restrict__ scales,
                                          uint8_t* __restrict__ zeros) {
    constexpr float qmax = float((1 << BITS) - 1);
    const int col0 = b0 + 32 * H;
    if (col0 % gs == 0) {
        // RTN scale and zero of the group from its running weights: the
        // registers for the block's part, W32 (which holds every earlier
        // block's compensation) for a group reaching past the block
        float mn = INFINITY, mx = -INFINITY;
#pragma unroll
        for (int k = 32 * H; k < BC; ++k) {
            if (k < 32 * H + gs) {
                mn = fminf(mn, w[k]);
                mx = fmaxf(mx, w[k]);
            }
        }
        // 16-byte pieces: the group's columns past the block start and end
        // on multiples of 32
#pragma unroll 4
        for (int k = b0 + BC; k < col0 + gs; k += 4) {
            const f4 v = *reinterpret_cast<const f4*>(wrow + k);
            mn = fminf(fminf(mn, v[0]), fminf(fminf(v[1], v[2]), v[3]));
            mx = fmaxf(fmaxf(mx, v[0]), fmaxf(fmaxf(v[1], v[2]), v[3]));
        }
        const float amax = fmaxf(fabsf(mn), fabsf(mx));
        const float s32 = SYM ? __fdiv_rn(2.0f * amax, qmax) : __fdiv_rn(mx - mn, qmax);
        uint16_t sh = f2h(s32);
        if ((sh & 0x7FFFu) == 0) sh = 0x0400u;  // 2^-14
        s = h2f(sh);
        z = SYM ? float(1 << (BITS - 1)) : fminf(fmaxf(rintf(__fdiv_rn(-mn, s)), 0.f), qmax);
        if (live) {
            scales[(size_t)n * G + col0 / gs] = sh;
            if (!SYM) zeros[(size_t)n * G + col0 / gs] = uint8_t(z);
        }
    }
#pragma unroll
    for (int ii = 0; ii < 32; ++ii) {
        const int i = 32 * H + ii;
        const float q = fminf(fmaxf(rintf(__fdiv_rn(w[i], s)) + z, 0.f), qmax);
        cw[i / 4] |= uint32_t(q) << (8 * (i % 4));
        const float wq = h2f(f2h((q - z) * s));
        const float err = (w[i] - wq) / us[i * BC + i];
        e[i] = err;
#pragma unroll
        for (int j = i + 1; j < BC; ++j) w[j] = fmaf(-err, us[i * BC + j], w[j]);
    }
}

// One block of GPTQ columns [b0, b0 + BC) for 64 weight rows, one row per
// lane held in registers.  U's entries are the same for every lane: the
// block's BC x BC part of U is staged in LDS once and read as broadcasts
// (LDS reads return in order, so their waits pipeline).  The block's codes
// and errors leave as 16-byte stores at the end.
template <int BITS, bool SYM, int BC>
__global__ void __launch_bounds__(64) gptq_block_kernel(float* __restrict__ W32, const float* __restrict__ U, int N,
                                                        int K, int b0, int gs, uint8_t* __restrict__ codes,
                                                        uint16_t* __restrict__ scales, uint8_t* __restrict__ zeros,
                                                        float* __restrict__ Err, int ldE) {
    __shared__ __align__(16) float us[BC * BC];
    for (int v = threadIdx.x; v < BC * BC / 4; v += 64) {
        const int r = v / (BC / 4), c4 = v % (BC / 4);
        *reinterpret_cast<f4*>(&us[r * BC + 4 * c4]) =
            *reinterpret_cast<const f4*>(U + (size_t)(b0 + r) * K + b0 + 4 * c4);
    }
    __syncthreads();
    const int n = blockIdx.x * 64 + threadIdx.x;
    const bool live = n < N;
    const int nr = live ? n : N - 1;  // rows past N compute on a copy and store nothing
    const int G = K / gs;
    const float* wrow = W32 + (size_t)nr * K;
    float w[BC], e[BC];
#pragma unroll
    for (int v = 0; v < BC / 4; ++v) {
        const f4 t = *reinterpret_cast<const f4*>(wrow + b0 + 4 * v);
        w[4 * v] = t[0];
        w[4 * v + 1] = t[1];
        w[4 * v + 2] = t[2];
        w[4 * v + 3] = t[3];
    }
    // a block that starts inside a group continues with the scale and zero
    // an earlier launch chose at the group's first column
    float s = 1.f, z = SYM ? float(1 << (BITS - 1)) : 0.f;
    if (b0 % gs != 0) {
        s = h2f(scales[(size_t)nr * G + b0 / gs]);
        if (!SYM) z = float(zeros[(size_t)nr * G + b0 / gs]);
    }
    uint32_t cw[BC / 4];
#pragma unroll
    for (int v = 0; v < BC / 4; ++v) cw[v] = 0;
    // groups are multiples of 32 columns: a group can only start at i = 0 or 32
    gptq_half<BITS, SYM, BC, 0>(w, e, cw, s, z, us, wrow, K, b0, gs, G, n, live, scales, zeros);
    if constexpr (BC == 64) gptq_half<BITS, SYM, BC, 1>(w, e, cw, s, z, us, wrow, K, b0, gs, G, n, live, scales, zeros);
    if (live) {
        uint8_t* crow = codes + (size_t)n * K + b0;
#pragma unroll
        for (int v = 0; v < BC / 16; ++v)
            *reinterpret_cast<u4*>(crow + 16 * v) = u4{cw[4 * v], cw[4 * v + 1], cw[4 * v + 2], cw[4 * v + 3]};
        float* erow = Err + (size_t)n * ldE;
#pragma unroll
        for (int v = 0; v < BC / 4; ++v)
            *reinterpret_cast<f4*>(erow + 4 * v) = f4{e[4 * v], e[4 * v + 1], e[4 * v + 2], e[4 * v + 3]};
    }
}

// Workspace regions (256-byte aligned).
struct GptqLayout {
    size_t xt, H, A, L, Li, U, W32, Err, dead, diag, perm, cperm, total;
};

GptqLayout gptq_layout(int M, int N, int K) {
    GptqLayout Ly{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += (bytes + 255) & ~size_t(255);
        return at;
    };
    const size_t KK = size_t(K) * K * 4;
    Ly.xt = take(size_t(K) * M * 2);
    Ly.H = take(KK);
    Ly.A = take(KK);
    Ly.L = take(KK);
    Ly.Li = take(KK);
    Ly.U = take(KK);
    Ly.W32 = take(size_t(N) * K * 4);
    Ly.Err = take(size_t(N) * kGptqOuter * 4);
    Ly.dead = take(size_t(K));
    Ly.diag = take(size_t(K) * 4);
    Ly.perm = take(size_t(K) * 4);
    Ly.cperm = take(size_t(N) * K);
    Ly.total = off;
    return Ly;
}

bool gptq_args_ok(int M, int N, int K, int bits, int group_size, int* gs_out) {
    if (M <= 0 || N <= 0 || K <= 0 || K % 32 != 0 || M % 32 != 0) return false;
    if (bits != 2 && bits != 3 && bits != 4 && bits != 8) return false;
    const int gs = group_size == -1 ? K : group_size;
    if (gs <= 0 || gs % 32 != 0 || K % gs != 0) return false;
    // a group never straddles a lazy-update block unless it starts at one
    // (one group per row starts at column 0 only)
    if (gs != K && !(kGptqB % gs == 0 || gs % kGptqB == 0)) return false;
    *gs_out = gs;
    return true;
}

// Outer block width: 256 columns when no group can start inside an outer
// block and reach past it (the group size divides 256 or is a multiple of
// it), else 64 (one level).
int gptq_outer(int gs) { return (kGptqOuter % gs == 0 || gs % kGptqOuter == 0) ? kGptqOuter : kGptqB; }

// The column walk in two levels: inside an outer block, each 64-column
// launch is followed by the update of the outer block's later columns; after
// the outer block, one product carries all of its errors to the columns
// after it.  Err holds the outer block's errors, [N][outer].
template <int BITS, bool SYM>
wq_status gptq_blocks(float* W32, const float* U, int N, int K, int gs, uint8_t* codes, uint16_t* scales,
                      uint8_t* zeros, float* Err, hipStream_t s) {
    const int outer = gptq_outer(gs);
    wq_status st;
    for (int ob0 = 0; ob0 < K; ob0 += outer) {
        const int oe = min(ob0 + outer, K);
        for (int b0 = ob0; b0 < oe; b0 += kGptqB) {
            const int bc = min(kGptqB, oe - b0);  // 64, or 32 at the end
            float* eb = Err + (b0 - ob0);
            if (bc == kGptqB)
                hipLaunchKernelGGL((gptq_block_kernel<BITS, SYM, kGptqB>), dim3((N + 63) / 64), dim3(64), 0, s, W32,
                                   U, N, K, b0, gs, codes, scales, zeros, eb, outer);
            else
                hipLaunchKernelGGL((gptq_block_kernel<BITS, SYM, 32>), dim3((N + 63) / 64), dim3(64), 0, s, W32, U,
                                   N, K, b0, gs, codes, scales, zeros, eb, outer);
            if ((st = wqh::launch_status()) != WQ_OK) return st;
            const int rest_in = oe - b0 - bc;
            if (rest_in > 0 &&
                (st = sgemm_shot(N, rest_in, bc, -1.f, eb, outer, U + (size_t)b0 * K + b0 + bc, K, 1.f,
                                 W32 + b0 + bc, K, s)) != WQ_OK)
                return st;
        }
        const int rest = K - oe;
        if (rest > 0 && (st = sgemm_nn(N, rest, oe - ob0, -1.f, Err, outer, U + (size_t)ob0 * K + oe, K, 1.f,
                                       W32 + oe, K, s)) != WQ_OK)
            return st;
    }
    return WQ_OK;
}

}  // namespace

extern "C" size_t wq_gptq_workspace_size(int32_t M, int32_t N, int32_t K) {
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    return gptq_layout(M, N, K).total;
}

extern "C" wq_status wq_gptq_quantize(const uint16_t* x, const uint16_t* w, int32_t M, int32_t N, int32_t K,
                                      int32_t bits, int32_t group_size, int32_t symmetric, double damp,
                                      int32_t act_order, uint8_t* codes, uint16_t* scales, uint8_t* zeros,
                                      int32_t* g_idx, void* workspace, size_t workspace_bytes, void* stream) {
    if (!x || !w || !codes || !scales || !workspace) return WQ_ERR_ARG;
    if (act_order && !g_idx) return WQ_ERR_ARG;
    if (bits != 2 && bits != 3 && bits != 4 && bits != 8) return WQ_ERR_UNSUPPORTED;
    int gs = 0;
    if (!gptq_args_ok(M, N, K, bits, group_size, &gs)) return WQ_ERR_ARG;
    if (symmetric ? (zeros != nullptr) : (zeros == nullptr)) return WQ_ERR_ARG;
    if (!(damp >= 0.0 && damp < 1.0)) return WQ_ERR_ARG;
    if (!wqh::aligned16(x) || !wqh::aligned16(w) || !wqh::aligned16(workspace) || !wqh::aligned16(codes))
        return WQ_ERR_ARG;
    const GptqLayout Ly = gptq_layout(M, N, K);
    if (workspace_bytes < Ly.total) return WQ_ERR_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    uint16_t* xt = reinterpret_cast<uint16_t*>(ws + Ly.xt);
    float* H = reinterpret_cast<float*>(ws + Ly.H);
    float* A = reinterpret_cast<float*>(ws + Ly.A);
    float* L = reinterpret_cast<float*>(ws + Ly.L);
    float* Li = reinterpret_cast<float*>(ws + Ly.Li);
    float* U = reinterpret_cast<float*>(ws + Ly.U);
    float* W32 = reinterpret_cast<float*>(ws + Ly.W32);
    float* Err = reinterpret_cast<float*>(ws + Ly.Err);
    uint8_t* dead = reinterpret_cast<uint8_t*>(ws + Ly.dead);
    float* diag = reinterpret_cast<float*>(ws + Ly.diag);
    int32_t* perm = reinterpret_cast<int32_t*>(ws + Ly.perm);
    uint8_t* cdst = act_order ? reinterpret_cast<uint8_t*>(ws + Ly.cperm) : codes;
    const long long KK = (long long)K * K;
    auto grid_for = [](long long n) { return dim3(unsigned(std::min<long long>((n + 255) / 256, 65536))); };
    wq_status st;

    // H = x^T x, dead channels, damping
    hipLaunchKernelGGL(transpose_kernel, dim3((K + 31) / 32, (M + 31) / 32), dim3(256), 0, s, x, M, K, xt);
    if ((st = wqh::launch_status()) != WQ_OK) return st;
    // the library's LDS-tiled fp16 product
    if ((st = wqh::dense_f32(xt, xt, H, K, K, M, s)) != WQ_OK) return st;
    hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(1024), 0, s, H, K, float(damp), dead, diag);
    hipLaunchKernelGGL(rank_kernel, dim3((K + 255) / 256), dim3(256), 0, s, diag, K, act_order ? 1 : 0, perm);
    if ((st = wqh::launch_status()) != WQ_OK) return st;

    // L L^T = P H' P and Li = L^-1 (blocked, right-looking), U = P Li P,
    // with H' the Hessian in processing order
    hipLaunchKernelGGL(permute_reverse_kernel, grid_for(KK), dim3(256), 0, s, H, perm, K, A);
    if ((st = wqh::launch_status()) != WQ_OK) return st;
    if ((st = chol_inverse(A, L, Li, K, s)) != WQ_OK) return st;
    hipLaunchKernelGGL(upper_reverse_kernel, grid_for(KK), dim3(256), 0, s, Li, K, U);
    if ((st = wqh::launch_status()) != WQ_OK) return st;

    // the column walk with lazy block updates
    const long long NK = (long long)N * K;
    if (act_order)
        hipLaunchKernelGGL(init_w_kernel, grid_for(NK), dim3(256), 0, s, w, dead, perm, NK, K, W32);
    else
        hipLaunchKernelGGL(init_w_vec_kernel, grid_for(NK / 8), dim3(256), 0, s, w, dead, NK / 8, K, W32);
    if ((st = wqh::launch_status()) != WQ_OK) return st;
    const bool sym = symmetric != 0;
    switch (bits) {
        case 2: st = sym ? gptq_blocks<2, true>(W32, U, N, K, gs, cdst, scales, zeros, Err, s)
                         : gptq_blocks<2, false>(W32, U, N, K, gs, cdst, scales, zeros, Err, s); break;
        case 3: st = sym ? gptq_blocks<3, true>(W32, U, N, K, gs, cdst, scales, zeros, Err, s)
                         : gptq_blocks<3, false>(W32, U, N, K, gs, cdst, scales, zeros, Err, s); break;
        case 4: st = sym ? gptq_blocks<4, true>(W32, U, N, K, gs, cdst, scales, zeros, Err, s)
                         : gptq_blocks<4, false>(W32, U, N, K, gs, cdst, scales, zeros, Err, s); break;
        default: st = sym ? gptq_blocks<8, true>(W32, U, N, K, gs, cdst, scales, zeros, Err, s)
                          : gptq_blocks<8, false>(W32, U, N, K, gs, cdst, scales, zeros, Err, s); break;
    }
    if (st != WQ_OK || !act_order) return st;
    // back to the original channel order, and the group map
    hipLaunchKernelGGL(unpermute_kernel, grid_for(NK), dim3(256), 0, s, cdst, perm, NK, K, gs, codes, g_idx);
    return wqh::launch_status();
}
