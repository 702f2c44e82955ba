// GPTQ ("GPTQ, AWQ and the rules of post-training quantization", section
// "GPTQ: pay for the error with the other weights"): the columns of W are
// quantized one at a time in a fixed order (index order), and each column's
// rounding error is compensated on the columns not yet quantized through
// the inverse Hessian of the layer's reconstruction loss, written with a
// Cholesky factor; the compensation is applied lazily, a block of 64
// columns at a time, so most of the work is a matrix product.
//
//   H = x^T x (float32, matrix cores); a channel with H[k][k] = 0 gets
//   H[k][k] = 1 and a zero weight column; H += damp * mean(diag H) * I.
//   U = the upper Cholesky factor of H^-1 (H^-1 = U^T U), computed as
//   U = P L^-1 P with L L^T = P H P and P the index reversal, the factor
//   and its inverse by recursive halving (large fp32 matrix-core products).
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

constexpr int kCholB = 32;   // Cholesky / inverse block
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

// dst[i][j] = src[K-1-i][K-1-j] (both K x K float32).
__global__ void __launch_bounds__(256) reverse_kernel(const float* __restrict__ src, int K, float* __restrict__ dst) {
    const long long total = (long long)K * K;
    for (long long t = (long long)blockIdx.x * 256 + threadIdx.x; t < total; t += (long long)gridDim.x * 256) {
        const int i = int(t / K), j = int(t % K);
        dst[t] = src[(size_t)(K - 1 - i) * K + (K - 1 - j)];
    }
}

__global__ void __launch_bounds__(256) fill_kernel(float* __restrict__ p, long long n, float v) {
    for (long long t = (long long)blockIdx.x * 256 + threadIdx.x; t < n; t += (long long)gridDim.x * 256) p[t] = v;
}

// Processing order: perm[i] = the channel of rank i.  With act-order the
// rank is the position in descending diag order, ties by channel index (a
// stable sort); otherwise the identity.
__global__ void __launch_bounds__(256) rank_kernel(const float* __restrict__ diag, int K, int act_order,
                                                   int32_t* __restrict__ perm) {
    const int k = blockIdx.x * 256 + threadIdx.x;
    if (k >= K) return;
    if (!act_order) {
        perm[k] = k;
        return;
    }
    const float d = diag[k];
    int rank = 0;
    for (int j = 0; j < K; ++j) {
        const float e = diag[j];
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

// C = beta * C + alpha * A . opB in float32 on the matrix cores
// (v_mfma_f32_16x16x4f32), opB(k, j) = TB ? B[j][k] : B[k][j]; leading
// dimensions lda, ldb, ldc; Kd a multiple of 4.  A 64 x 64 output tile per
// 256-thread block, each wavefront a 32 x 32 quarter (2 x 2 instructions);
// k in steps of 32 through LDS, A as As[m][k] and opB as Bs[n][k] so that a
// lane reads four consecutive k of its row with one 16-byte load.  The
// four instructions of one such load take k = 4 * (lane / 16) + t for
// t = 0..3 in A and B alike: a permutation of the sum's terms.
template <bool TB>
__global__ void __launch_bounds__(256) sgemm_kernel(int M, int N, int Kd, float alpha, const float* __restrict__ A,
                                                    int lda, const float* __restrict__ B, int ldb, float beta,
                                                    float* __restrict__ C, int ldc, int lower_only) {
    constexpr int LD = 36;  // row stride in floats: 16-byte aligned, spreads banks
    __shared__ float As[64 * LD];
    __shared__ float Bs[64 * LD];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
    const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
    // lower_only: C's strictly upper 64 x 64 tiles are never read again
    if (lower_only && j0 > i0 + 63) return;
    f4 acc[2][2];
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
                const int gi = i0 + r, gk = k0 + k;
                As[r * LD + k] = (gi < M && gk < Kd) ? A[(size_t)gi * lda + gk] : 0.f;
            }
            if (TB) {
                const int n = e >> 5, k = e & 31;  // B[n][k]: consecutive k
                const int gj = j0 + n, gk = k0 + k;
                Bs[n * LD + k] = (gj < N && gk < Kd) ? B[(size_t)gj * ldb + gk] : 0.f;
            } else {
                const int k = e >> 6, n = e & 63;  // B[k][n]: consecutive n
                const int gj = j0 + n, gk = k0 + k;
                Bs[n * LD + k] = (gj < N && gk < Kd) ? B[(size_t)gk * ldb + gj] : 0.f;
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
    // lane holds rows 4 * lg + r of column li of each 16 x 16 block
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int gj = j0 + wn + 16 * j + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int gi = i0 + wm + 16 * i + 4 * lg + r;
                if (gi < M && gj < N) {
                    float* p = C + (size_t)gi * ldc + gj;
                    *p = (beta == 0.f ? 0.f : beta * *p) + alpha * acc[i][j][r];
                }
            }
        }
}

template <bool TB>
wq_status sgemm(int M, int N, int Kd, float alpha, const float* A, int lda, const float* B, int ldb, float beta,
                float* C, int ldc, hipStream_t s, bool lower_only = false) {
    if (M <= 0 || N <= 0) return WQ_OK;
    if (Kd % 4 != 0) return WQ_ERR_ARG;
    hipLaunchKernelGGL((sgemm_kernel<TB>), dim3((N + 63) / 64, (M + 63) / 64), dim3(256), 0, s, M, N, Kd, alpha, A,
                       lda, B, ldb, beta, C, ldc, lower_only ? 1 : 0);
    return wqh::launch_status();
}

// Factor the nb x nb diagonal block at A[j0][j0] (lower part; nb <= 32):
// L11 into L, its inverse into Li (both leading dimension K).  256 threads,
// thread t owns column t % 32 of rows t / 32 + 8 q (q = 0..3).  Outer-product
// elimination without the square roots, one barrier per step: after step j,
// a[r][c] (r, c > j) is the Schur complement and a[r][j] = L[r][j] *
// sqrt(p_j) with pivot p_j = a[j][j]; L[r][c] = a[r][c] / sqrt(p_c) at the
// end.  A pivot that is not positive (rounding) is clamped to 1e-30.  The
// inverse is forward elimination on the identity, also one barrier a step:
// t[r][c] -= L[r][j] * t[j][c] / L[j][j], rows divided by L[r][r] at the end.
__global__ void __launch_bounds__(256) chol_diag_kernel(const float* __restrict__ A, int K, int j0, int nb,
                                                        float* __restrict__ L, float* __restrict__ Li) {
    __shared__ float a[kCholB][kCholB + 1];
    __shared__ float t[kCholB][kCholB + 1];
    const int c = threadIdx.x & 31, rb = threadIdx.x >> 5;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = rb + 8 * q;
        a[r][c] = (r < nb && c < nb && c <= r) ? A[(size_t)(j0 + r) * K + j0 + c] : 0.f;
        t[r][c] = (r == c) ? 1.f : 0.f;
    }
    __syncthreads();
    for (int j = 0; j + 1 < nb; ++j) {
        const float inv_p = 1.f / fmaxf(a[j][j], 1e-30f);
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = rb + 8 * q;
            const bool upd = r > j && r < nb && c > j && c <= r;
            v[q] = upd ? a[r][c] - a[r][j] * a[c][j] * inv_p : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = rb + 8 * q;
            if (r > j && r < nb && c > j && c <= r) a[r][c] = v[q];
        }
        __syncthreads();
    }
    // L in place
    float lv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = rb + 8 * q;
        const float root = sqrtf(fmaxf(a[c][c], 1e-30f));
        lv[q] = (r < nb && c < nb && c <= r) ? (r == c ? root : a[r][c] / root) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) a[rb + 8 * q][c] = lv[q];
    __syncthreads();
    for (int j = 0; j + 1 < nb; ++j) {
        // row j of t is final (up to its division by L[j][j])
        const float inv_d = 1.f / a[j][j];
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = rb + 8 * q;
            const bool upd = r > j && r < nb && c <= j;
            v[q] = upd ? t[r][c] - a[r][j] * t[j][c] * inv_d : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = rb + 8 * q;
            if (r > j && r < nb && c <= j) t[r][c] = v[q];
        }
        __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = rb + 8 * q;
        if (r < nb && c < nb) {
            L[(size_t)(j0 + r) * K + j0 + c] = a[r][c];
            Li[(size_t)(j0 + r) * K + j0 + c] = (c <= r) ? t[r][c] / a[r][r] : 0.f;
        }
    }
}

// Recursive Cholesky with the inverse of the factor, on the block
// [n0, n0 + n) of A (lower part read; the trailing block is overwritten by
// its Schur complement):  with halves 1 and 2,
//   L11 = chol(A11), L21 = A21 . L11^-T, L22 = chol(A22 - L21 . L21^T),
//   inv(L) = [[Li11, 0], [-Li22 . L21 . Li11, Li22]].
// Blocks of kCholB go to chol_diag_kernel; everything else is large fp32
// products.  tmp: room for n * n / 4 floats.
wq_status chol_inverse(float* A, float* L, float* Li, int K, int n0, int n, float* tmp, hipStream_t s) {
    if (n <= kCholB) {
        hipLaunchKernelGGL(chol_diag_kernel, dim3(1), dim3(256), 0, s, A, K, n0, n, L, Li);
        return wqh::launch_status();
    }
    const int h = ((n / kCholB + 1) / 2) * kCholB, n2 = n - h, r0 = n0 + h;
    float* L21 = L + (size_t)r0 * K + n0;
    const float* Li11 = Li + (size_t)n0 * K + n0;
    wq_status st;
    if ((st = chol_inverse(A, L, Li, K, n0, h, tmp, s)) != WQ_OK) return st;
    if ((st = sgemm<true>(n2, h, h, 1.f, A + (size_t)r0 * K + n0, K, Li11, K, 0.f, L21, K, s)) != WQ_OK) return st;
    // the trailing update: only its lower triangle is read afterwards
    if ((st = sgemm<true>(n2, n2, h, -1.f, L21, K, L21, K, 1.f, A + (size_t)r0 * K + r0, K, s, true)) != WQ_OK)
        return st;
    if ((st = chol_inverse(A, L, Li, K, r0, n2, tmp, s)) != WQ_OK) return st;
    // tmp = L21 . Li11 (n2 x h), then Li21 = -Li22 . tmp
    if ((st = sgemm<false>(n2, h, h, 1.f, L21, K, Li11, K, 0.f, tmp, h, s)) != WQ_OK) return st;
    return sgemm<false>(n2, h, n2, -1.f, Li + (size_t)r0 * K + r0, K, tmp, h, 0.f, Li + (size_t)r0 * K + n0, K, s);
}

// Columns [32 H, 32 H + 32) of a block (see gptq_block_kernel); a group can
// start only at the first of them.
template <int BITS, bool SYM, int BC, int H>
__device__ __forceinline__ void gptq_half(float (&w)[BC], float (&e)[BC], uint32_t (&cw)[BC / 4], float& s, float& z,
                                          const float* __restrict__ urow, const float* __restrict__ wrow, int K,
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
#pragma unroll 4
        for (int k = b0 + BC; k < col0 + gs; ++k) {
            const float v = wrow[k];
            mn = fminf(mn, v);
            mx = fmaxf(mx, v);
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
        const float err = (w[i] - wq) / urow[(size_t)i * K + i];
        e[i] = err;
#pragma unroll
        for (int j = i + 1; j < BC; ++j) w[j] = fmaf(-err, urow[(size_t)i * K + j], w[j]);
    }
}

// One block of GPTQ columns [b0, b0 + BC) for 64 weight rows, one row per
// lane held in registers.  U's entries are the same for every lane (uniform
// loads); the block's codes and errors leave as 16-byte stores at the end.
template <int BITS, bool SYM, int BC>
__global__ void __launch_bounds__(64) gptq_block_kernel(float* __restrict__ W32, const float* __restrict__ U, int N,
                                                        int K, int b0, int gs, uint8_t* __restrict__ codes,
                                                        uint16_t* __restrict__ scales, uint8_t* __restrict__ zeros,
                                                        float* __restrict__ Err, int ldE) {
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
    const float* urow = U + (size_t)b0 * K + b0;
    // groups are multiples of 32 columns: a group can only start at i = 0 or 32
    gptq_half<BITS, SYM, BC, 0>(w, e, cw, s, z, urow, wrow, K, b0, gs, G, n, live, scales, zeros);
    if constexpr (BC == 64) gptq_half<BITS, SYM, BC, 1>(w, e, cw, s, z, urow, wrow, K, b0, gs, G, n, live, scales, zeros);
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
                (st = sgemm<false>(N, rest_in, bc, -1.f, eb, outer, U + (size_t)b0 * K + b0 + bc, K, 1.f,
                                   W32 + b0 + bc, K, s)) != WQ_OK)
                return st;
        }
        const int rest = K - oe;
        if (rest > 0 && (st = sgemm<false>(N, rest, oe - ob0, -1.f, Err, outer, U + (size_t)ob0 * K + oe, K, 1.f,
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
    if ((st = wqh::dense_f32(xt, xt, H, K, K, M, s)) != WQ_OK) return st;
    hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(1024), 0, s, H, K, float(damp), dead, diag);
    hipLaunchKernelGGL(rank_kernel, dim3((K + 255) / 256), dim3(256), 0, s, diag, K, act_order ? 1 : 0, perm);
    if ((st = wqh::launch_status()) != WQ_OK) return st;

    // L L^T = P H' P and Li = L^-1 (recursive halving), U = P Li P, with H'
    // the Hessian in processing order
    hipLaunchKernelGGL(permute_reverse_kernel, grid_for(KK), dim3(256), 0, s, H, perm, K, A);
    hipLaunchKernelGGL(fill_kernel, grid_for(KK), dim3(256), 0, s, L, KK, 0.f);
    hipLaunchKernelGGL(fill_kernel, grid_for(KK), dim3(256), 0, s, Li, KK, 0.f);
    if ((st = wqh::launch_status()) != WQ_OK) return st;
    // H is free once reversed into A: scratch for the inverse's products
    if ((st = chol_inverse(A, L, Li, K, 0, K, H, s)) != WQ_OK) return st;
    hipLaunchKernelGGL(reverse_kernel, grid_for(KK), dim3(256), 0, s, Li, K, U);
    if ((st = wqh::launch_status()) != WQ_OK) return st;

    // the column walk with lazy block updates
    const long long NK = (long long)N * K;
    hipLaunchKernelGGL(init_w_kernel, grid_for(NK), dim3(256), 0, s, w, dead, perm, NK, K, W32);
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
