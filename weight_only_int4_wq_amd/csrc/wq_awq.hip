// AWQ's search for the scaling exponent alpha ("GPTQ, AWQ and the rules of
// post-training quantization", section "AWQ: find the one percent that
// matters": per-channel scales s = (mean |x|)^alpha, alpha from a grid of 20
// points on [0, 1]).  Each grid point is scored by the squared output error
// of the rescaled, RTN-quantized layer against the original layer on the
// calibration activations:
//     loss(alpha) = sum over m, n of (x' . w_hat'^T - x . W^T)[m][n]^2,
// with x' = fp16(x / s), W' = fp16(W * s) quantized and dequantized to
// w_hat'.  The steps run on the library's own kernels: channel statistics,
// fold, division, quantization, packing and the matrix-core GEMM (fp32
// output).  The reference x . W^T comes from a plain fp16 matrix-core
// product (LDS-tiled) computed once per search; the squared differences are summed in
// float64 in a fixed order (deterministic).
#include "wq_gemm_common.h"

namespace {

using namespace wq;

// y32[m][n] = sum_k x[m][k] * w[n][k] (fp16 operands, fp32 accumulation;
// K a multiple of 32, x and w 16-byte aligned): 128 x 128 output tiles,
// four wavefronts of 64 x 64 (4 x 4 v_mfma_f32_16x16x32_f16).  k advances
// in stages of 32 through two LDS buffers (rows padded to 40 halves so
// that the sixteen rows of a fragment read fall on distinct banks); the
// next stage's 16-byte loads are in registers while the current stage is
// multiplied, one barrier per stage.  A lane's fragment is 8 consecutive k
// of one row, k = 8 * (lane / 16) + 0..7, the same in x and w.
constexpr int kDenseLd = 40;  // halves per LDS row

__global__ void __launch_bounds__(256) dense_ref_kernel(const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ w, float* __restrict__ y32,
                                                        int M, int N, int K) {
    constexpr int LD = kDenseLd;
    __shared__ __align__(16) uint16_t As[2][128 * LD];
    __shared__ __align__(16) uint16_t Bs[2][128 * LD];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int m0 = blockIdx.y * 128, n0 = blockIdx.x * 128;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    // stage loads: 128 rows x 32 halves = 512 pieces of 16 bytes per operand,
    // two per thread: row e / 4, halves 8 * (e % 4)
    u4 ra[2], rb[2];
    auto gload = [&](int k0) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int e = tid + 256 * q, r = e >> 2, c8 = 8 * (e & 3);
            const int gm = min(m0 + r, M - 1), gn = min(n0 + r, N - 1);
            ra[q] = *reinterpret_cast<const u4*>(x + (size_t)gm * K + k0 + c8);
            rb[q] = *reinterpret_cast<const u4*>(w + (size_t)gn * K + k0 + c8);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int e = tid + 256 * q, r = e >> 2, c8 = 8 * (e & 3);
            *reinterpret_cast<u4*>(&As[buf][r * LD + c8]) = ra[q];
            *reinterpret_cast<u4*>(&Bs[buf][r * LD + c8]) = rb[q];
        }
    };
    f4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};
    const int stages = K / 32;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int st = 0; st < stages; ++st) {
        const int buf = st & 1;
        if (st + 1 < stages) gload(32 * (st + 1));
        h8 a[4], b[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            a[t] = *reinterpret_cast<const h8*>(&As[buf][(wm + 16 * t + li) * LD + 8 * lg]);
            b[t] = *reinterpret_cast<const h8*>(&Bs[buf][(wn + 16 * t + li) * LD + 8 * lg]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        // the other buffer was last read in the previous stage, before the
        // barrier that ended it
        if (st + 1 < stages) sstore(buf ^ 1);
        __syncthreads();
    }
    // lane holds rows 4*lg + r of column li of each 16 x 16 block
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + wn + 16 * j + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm + 16 * i + 4 * lg + r;
                if (row < M && col < N) y32[(size_t)row * N + col] = acc[i][j][r];
            }
        }
}

constexpr int kSqBlocks = 1024;

// partial[b] = sum over this block's share of (a - b)^2 in float64; the
// share is a fixed grid-stride set of 4-element pieces (16-byte loads; a
// and b 16-byte aligned) plus the same stride over the last n % 4
// elements, and the block sums in a fixed tree order.
__global__ void __launch_bounds__(256) sqdiff_partial_kernel(const float* __restrict__ a, const float* __restrict__ b,
                                                             long long n, double* __restrict__ partial) {
    __shared__ double red[256];
    double acc = 0.0;
    const long long stride = (long long)gridDim.x * 256, t0 = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long n4 = n / 4;
    const f4* a4 = reinterpret_cast<const f4*>(a);
    const f4* b4 = reinterpret_cast<const f4*>(b);
#pragma unroll 2
    for (long long t = t0; t < n4; t += stride) {
        const f4 u = a4[t], v = b4[t];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const double d = double(u[e]) - double(v[e]);
            acc += d * d;
        }
    }
    for (long long t = 4 * n4 + t0; t < n; t += stride) {
        const double d = double(a[t]) - double(b[t]);
        acc += d * d;
    }
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) partial[blockIdx.x] = red[0];
}

// out[0] = sum of partial[0 .. n) in a fixed tree order (one block).
__global__ void __launch_bounds__(256) sum_partials_kernel(const double* __restrict__ partial, int n,
                                                           double* __restrict__ out) {
    __shared__ double red[256];
    double acc = 0.0;
    for (int t = threadIdx.x; t < n; t += 256) acc += partial[t];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[0] = red[0];
}

// Workspace regions of one search, each starting on a 256-byte boundary.
struct SearchLayout {
    size_t s_h, xf, wf, codes, scales, zeros, packed, yref, yq, partial, losses, total;
};

SearchLayout search_layout(int M, int N, int K, int bits, int G, int n_grid) {
    SearchLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += (bytes + 255) & ~size_t(255);
        return at;
    };
    const size_t MK = size_t(M) * K, NK = size_t(N) * K, MN = size_t(M) * N, NG = size_t(N) * G;
    L.s_h = take(size_t(K) * 2);
    L.xf = take(MK * 2);
    L.wf = take(NK * 2);
    L.codes = take(NK);
    L.scales = take(NG * 2);
    L.zeros = take(NG);
    L.packed = take(NK * size_t(bits) / 8);
    L.yref = take(MN * 4);
    L.yq = take(MN * 4);
    L.partial = take(size_t(kSqBlocks) * 8);
    L.losses = take(size_t(n_grid) * 8);
    L.total = off;
    return L;
}

bool search_args_ok(int M, int N, int K, int bits, int group_size, int n_grid, int* gs_out) {
    if (M <= 0 || N <= 0 || K <= 0 || K % 32 != 0 || n_grid < 2 || n_grid > 4096) return false;
    if (bits != 2 && bits != 3 && bits != 4 && bits != 8) return false;
    const int gs = group_size == -1 ? K : group_size;
    if (gs <= 0 || gs % 32 != 0 || K % gs != 0) return false;
    *gs_out = gs;
    return true;
}


// ------------------------------------------------ clipping threshold search

__device__ __forceinline__ float clip_h2f(uint16_t h) { return float(__builtin_bit_cast(_Float16, h)); }
__device__ __forceinline__ uint16_t clip_f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// t = fp16(fp32(r * amax)): the product is rounded to fp32 first.  Left to
// itself the compiler fuses the multiply and the conversion into one
// mixed-precision instruction that rounds only once, which picks the other
// fp16 neighbour when the fp32 product is an fp16 tie; the empty asm (no
// instruction) keeps the fp32 product in a register between the two.
__device__ __forceinline__ float clip_threshold(float r, float amax) {
    float p = r * amax;
    asm("" : "+v"(p));
    return clip_h2f(clip_f2h(p));
}

// AWQ's clipping-threshold search ("AutoAWQ vs The Stack v2", paragraph on
// scaling factors and clipping thresholds): one block per (64 output rows,
// group of GS input channels).  For each ratio r_i = fp32(1 - i / n_grid):
// t = fp16(r_i * max|w|) per row, the group clipped to [-t, t] and RTN-
// quantized (wq_quantize_rtn's rule, the group as one RTN group) in
// registers, d = w - w_hat staged in LDS as fp16, and
//   loss[n] = sum over m of (sum over k in the group of x[m][k] d[n][k])^2
// from fp16 matrix-core products (fp32 accumulation) over the calibration
// rows, 64 at a time.  Thread t holds row t / 4, quarter t % 4 of the group.
template <int BITS, bool SYM, int GS>
__global__ void __launch_bounds__(256) awq_clip_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                       int M, int N, int K, int n_grid, int n_ratios,
                                                       uint16_t* __restrict__ w_out, int32_t* __restrict__ best_out,
                                                       float* __restrict__ losses) {
    constexpr float qmax = float((1 << BITS) - 1);
    constexpr int Q = GS / 4;      // values per thread
    constexpr int LDD = GS + 8;    // LDS row stride (fp16)
    __shared__ uint16_t Ds[64 * LDD];
    __shared__ float red[2][64];
    const int tid = threadIdx.x, rr = tid >> 2, qq = tid & 3;
    const int n0 = blockIdx.x * 64, g = blockIdx.y, c0 = g * GS;
    const int G = K / GS;
    const int n = n0 + rr;
    const bool live = n < N;
    const uint16_t* wrow = w + (size_t)(live ? n : N - 1) * K + c0 + qq * Q;
    float wv[Q];
#pragma unroll
    for (int v = 0; v < Q / 8; ++v) {
        const u4 t = *reinterpret_cast<const u4*>(wrow + 8 * v);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            wv[8 * v + 2 * e] = clip_h2f(uint16_t(t[e] & 0xFFFFu));
            wv[8 * v + 2 * e + 1] = clip_h2f(uint16_t(t[e] >> 16));
        }
    }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < Q; ++j) amax = fmaxf(amax, fabsf(wv[j]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));

    const int lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int wmi = wave >> 1, wn = (wave & 1) * 32;
    float best_err = INFINITY;
    int best_i = 0;
    for (int i = 0; i < n_ratios; ++i) {
        const float r = float(1.0 - double(i) / double(n_grid));
        const float t = clip_threshold(r, amax);
        float mn = INFINITY, mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < Q; ++j) {
            const float c = fminf(fmaxf(wv[j], -t), t);
            mn = fminf(mn, c);
            mx = fmaxf(mx, c);
        }
        mn = fminf(mn, __shfl_xor(mn, 1));
        mn = fminf(mn, __shfl_xor(mn, 2));
        mx = fmaxf(mx, __shfl_xor(mx, 1));
        mx = fmaxf(mx, __shfl_xor(mx, 2));
        const float s32 = SYM ? __fdiv_rn(2.0f * fmaxf(fabsf(mn), fabsf(mx)), qmax) : __fdiv_rn(mx - mn, qmax);
        uint16_t sh = clip_f2h(s32);
        if ((sh & 0x7FFFu) == 0) sh = 0x0400u;  // 2^-14
        const float sc = clip_h2f(sh);
        const float z = SYM ? float(1 << (BITS - 1)) : fminf(fmaxf(rintf(__fdiv_rn(-mn, sc)), 0.f), qmax);
        uint16_t* drow = Ds + rr * LDD + qq * Q;
#pragma unroll
        for (int j = 0; j < Q; j += 2) {
            float dd[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float c = fminf(fmaxf(wv[j + e], -t), t);
                const float q = fminf(fmaxf(rintf(__fdiv_rn(c, sc)) + z, 0.f), qmax);
                dd[e] = wv[j + e] - clip_h2f(clip_f2h((q - z) * sc));
            }
            *reinterpret_cast<uint32_t*>(drow + j) = uint32_t(clip_f2h(dd[0])) | (uint32_t(clip_f2h(dd[1])) << 16);
        }
        __syncthreads();
        // squared group outputs: each wavefront a 32 (m) x 32 (n) quarter of
        // every 64 x 64 tile of x . d^T
        float sums[2] = {0.f, 0.f};
        for (int m0 = 0; m0 < M; m0 += 64) {
            f4 acc[2][2];
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b) acc[a][b] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < GS; k0 += 32) {
                h8 av[2], bv[2];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const int m = m0 + wmi * 32 + 16 * tt + li;
                    const h8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
                    av[tt] = m < M ? *reinterpret_cast<const h8*>(x + (size_t)m * K + c0 + k0 + 8 * lg) : zero8;
                    bv[tt] = *reinterpret_cast<const h8*>(Ds + (wn + 16 * tt + li) * LDD + k0 + 8 * lg);
                }
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int b = 0; b < 2; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[a], bv[b], acc[a][b], 0, 0, 0);
            }
            // lane holds rows 4 * lg + e of column li of each 16 x 16 block
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int e = 0; e < 4; ++e) sums[b] = fmaf(acc[a][b][e], acc[a][b][e], sums[b]);
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            sums[b] += __shfl_xor(sums[b], 16);
            sums[b] += __shfl_xor(sums[b], 32);
        }
        if (lg == 0) {
            red[wmi][wn + li] = sums[0];
            red[wmi][wn + 16 + li] = sums[1];
        }
        __syncthreads();
        const float err = red[0][rr] + red[1][rr];
        if (err < best_err) {
            best_err = err;
            best_i = i;
        }
        if (losses && live && qq == 0) losses[((size_t)n * G + g) * n_ratios + i] = err;
        __syncthreads();  // Ds and red are rewritten by the next ratio
    }
    if (live) {
        const float r = float(1.0 - double(best_i) / double(n_grid));
        const float t = clip_threshold(r, amax);
        uint16_t* orow = w_out + (size_t)n * K + c0 + qq * Q;
#pragma unroll
        for (int v = 0; v < Q / 8; ++v) {
            u4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint16_t lo = clip_f2h(fminf(fmaxf(wv[8 * v + 2 * e], -t), t));
                const uint16_t hi = clip_f2h(fminf(fmaxf(wv[8 * v + 2 * e + 1], -t), t));
                o[e] = uint32_t(lo) | (uint32_t(hi) << 16);
            }
            *reinterpret_cast<u4*>(orow + 8 * v) = o;
        }
        if (best_out && qq == 0) best_out[(size_t)n * G + g] = best_i;
    }
}

template <int BITS, bool SYM>
wq_status launch_clip(int gs, const uint16_t* x, const uint16_t* w, int M, int N, int K, int n_grid, int n_ratios,
                      uint16_t* w_out, int32_t* best, float* losses, hipStream_t s) {
    const dim3 grid((N + 63) / 64, K / gs), block(256);
    switch (gs) {
        case 32: hipLaunchKernelGGL((awq_clip_kernel<BITS, SYM, 32>), grid, block, 0, s, x, w, M, N, K, n_grid, n_ratios, w_out, best, losses); break;
        case 64: hipLaunchKernelGGL((awq_clip_kernel<BITS, SYM, 64>), grid, block, 0, s, x, w, M, N, K, n_grid, n_ratios, w_out, best, losses); break;
        case 128: hipLaunchKernelGGL((awq_clip_kernel<BITS, SYM, 128>), grid, block, 0, s, x, w, M, N, K, n_grid, n_ratios, w_out, best, losses); break;
        default: hipLaunchKernelGGL((awq_clip_kernel<BITS, SYM, 256>), grid, block, 0, s, x, w, M, N, K, n_grid, n_ratios, w_out, best, losses); break;
    }
    return wqh::launch_status();
}

}  // namespace

wq_status wqh::dense_f32(const uint16_t* x, const uint16_t* w, float* y32, int M, int N, int K, hipStream_t s) {
    if (M <= 0 || N <= 0) return WQ_OK;
    if (K % 32 != 0) return WQ_ERR_ARG;
    hipLaunchKernelGGL(dense_ref_kernel, dim3((N + 127) / 128, (M + 127) / 128), dim3(256), 0, s, x, w, y32, M, N, K);
    return wqh::launch_status();
}

extern "C" size_t wq_awq_search_workspace_size(int32_t M, int32_t N, int32_t K, int32_t bits, int32_t group_size,
                                               int32_t n_grid) {
    int gs = 0;
    if (!search_args_ok(M, N, K, bits, group_size, n_grid, &gs)) return 0;
    return search_layout(M, N, K, bits, K / gs, n_grid).total;
}

extern "C" wq_status wq_awq_search(const uint16_t* x, const uint16_t* w, int32_t M, int32_t N, int32_t K,
                                   int32_t bits, int32_t group_size, int32_t symmetric, int32_t n_grid,
                                   double* losses, int32_t* best, void* workspace, size_t workspace_bytes,
                                   void* stream) {
    int gs = 0;
    if (!x || !w || !losses || !workspace) return WQ_ERR_ARG;
    if (bits != 2 && bits != 3 && bits != 4 && bits != 8) return WQ_ERR_UNSUPPORTED;
    if (!search_args_ok(M, N, K, bits, group_size, n_grid, &gs)) return WQ_ERR_ARG;
    if (!wqh::aligned16(x) || !wqh::aligned16(w) || !wqh::aligned16(workspace)) return WQ_ERR_ARG;
    const int G = K / gs;
    const SearchLayout L = search_layout(M, N, K, bits, G, n_grid);
    if (workspace_bytes < L.total) return WQ_ERR_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    uint16_t* s_h = reinterpret_cast<uint16_t*>(ws + L.s_h);
    uint16_t* xf = reinterpret_cast<uint16_t*>(ws + L.xf);
    uint16_t* wf = reinterpret_cast<uint16_t*>(ws + L.wf);
    uint8_t* codes = reinterpret_cast<uint8_t*>(ws + L.codes);
    uint16_t* scales = reinterpret_cast<uint16_t*>(ws + L.scales);
    uint8_t* zeros = symmetric ? nullptr : reinterpret_cast<uint8_t*>(ws + L.zeros);
    uint32_t* packed = reinterpret_cast<uint32_t*>(ws + L.packed);
    float* yref = reinterpret_cast<float*>(ws + L.yref);
    float* yq = reinterpret_cast<float*>(ws + L.yq);
    double* partial = reinterpret_cast<double*>(ws + L.partial);
    double* dloss = reinterpret_cast<double*>(ws + L.losses);
    const long long mn = (long long)M * N;

    // the original layer's output, once
    wq_status st = wqh::dense_f32(x, w, yref, M, N, K, s);
    if (st != WQ_OK) return st;

    for (int i = 0; i < n_grid; ++i) {
        const double alpha = double(i) / double(n_grid - 1);
        if ((st = wq_awq_scales(x, M, K, alpha, s_h, stream)) != WQ_OK) return st;
        if ((st = wq_awq_fold(w, s_h, N, K, wf, stream)) != WQ_OK) return st;
        if ((st = wq_scale_act(x, s_h, M, K, xf, stream)) != WQ_OK) return st;
        if ((st = wq_quantize_rtn(wf, nullptr, N, K, bits, group_size, symmetric ? 1 : 0, codes, scales, zeros,
                                  stream)) != WQ_OK)
            return st;
        if ((st = wq_pack(codes, nullptr, K, N, bits, group_size, packed, nullptr, stream)) != WQ_OK) return st;
        if ((st = wqh::gemm_f32(xf, packed, scales, zeros, yq, M, N, K, bits, gs, s)) != WQ_OK) return st;
        hipLaunchKernelGGL(sqdiff_partial_kernel, dim3(kSqBlocks), dim3(256), 0, s, yq, yref, mn, partial);
        hipLaunchKernelGGL(sum_partials_kernel, dim3(1), dim3(256), 0, s, partial, kSqBlocks, dloss + i);
        if ((st = wqh::launch_status()) != WQ_OK) return st;
    }
    if (wqh::hip_status(hipMemcpyAsync(losses, dloss, size_t(n_grid) * 8, hipMemcpyDeviceToHost, s)) != WQ_OK)
        return WQ_ERR_HIP;
    if (wqh::hip_status(hipStreamSynchronize(s)) != WQ_OK) return WQ_ERR_HIP;
    if (best) {
        int b = 0;
        for (int i = 1; i < n_grid; ++i)
            if (losses[i] < losses[b]) b = i;
        *best = b;
    }
    return WQ_OK;
}

extern "C" wq_status wq_awq_clip(const uint16_t* x, const uint16_t* w, int32_t M, int32_t N, int32_t K, int32_t bits,
                                 int32_t group_size, int32_t symmetric, int32_t n_grid, int32_t n_ratios,
                                 uint16_t* w_out, int32_t* best, float* losses, void* stream) {
    if (!x || !w || !w_out) return WQ_ERR_ARG;
    if (bits != 2 && bits != 3 && bits != 4 && bits != 8) return WQ_ERR_UNSUPPORTED;
    if (M <= 0 || N <= 0 || K <= 0 || K % 32 != 0) return WQ_ERR_ARG;
    const int gs = group_size == -1 ? K : group_size;
    if (gs <= 0 || gs % 32 != 0 || K % gs != 0) return WQ_ERR_ARG;
    if (gs != 32 && gs != 64 && gs != 128 && gs != 256) return WQ_ERR_UNSUPPORTED;
    if (n_grid < 1 || n_ratios < 1 || n_ratios > n_grid || n_ratios > 1024) return WQ_ERR_ARG;
    if (!wqh::aligned16(x) || !wqh::aligned16(w) || !wqh::aligned16(w_out)) return WQ_ERR_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool sym = symmetric != 0;
    switch (bits) {
        case 2: return sym ? launch_clip<2, true>(gs, x, w, M, N, K, n_grid, n_ratios, w_out, best, losses, s)
                           : launch_clip<2, false>(gs, x, w, M, N, K, n_grid, n_ratios, w_out, best, losses, s);
        case 3: return sym ? launch_clip<3, true>(gs, x, w, M, N, K, n_grid, n_ratios, w_out, best, losses, s)
                           : launch_clip<3, false>(gs, x, w, M, N, K, n_grid, n_ratios, w_out, best, losses, s);
        case 4: return sym ? launch_clip<4, true>(gs, x, w, M, N, K, n_grid, n_ratios, w_out, best, losses, s)
                           : launch_clip<4, false>(gs, x, w, M, N, K, n_grid, n_ratios, w_out, best, losses, s);
        default: return sym ? launch_clip<8, true>(gs, x, w, M, N, K, n_grid, n_ratios, w_out, best, losses, s)
                            : launch_clip<8, false>(gs, x, w, M, N, K, n_grid, n_ratios, w_out, best, losses, s);
    }
}
