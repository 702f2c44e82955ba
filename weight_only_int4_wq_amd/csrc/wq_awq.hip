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
// product computed once per search; the squared differences are summed in
// float64 in a fixed order (deterministic).
#include "wq_gemm_common.h"

namespace {

using namespace wq;

// y32[m][n] = sum_k x[m][k] * w[n][k] (fp16 operands, fp32 accumulation):
// 64 x 64 output tiles, four wavefronts of 32 x 32 (2 x 2 v_mfma_f32_16x16x32_f16),
// fragments read straight from global memory (computed once per search).
__global__ void __launch_bounds__(256) dense_ref_kernel(const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ w, float* __restrict__ y32,
                                                        int M, int N, int K) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int m0 = blockIdx.y * 64 + (wave >> 1) * 32, n0 = blockIdx.x * 64 + (wave & 1) * 32;
    const uint16_t* ar[2];
    const uint16_t* br[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        ar[t] = x + (size_t)min(m0 + 16 * t + li, M - 1) * K + 8 * lg;
        br[t] = w + (size_t)min(n0 + 16 * t + li, N - 1) * K + 8 * lg;
    }
    f4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < K; k0 += 32) {
        h8 a[2], b[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            a[t] = *reinterpret_cast<const h8*>(ar[t] + k0);
            b[t] = *reinterpret_cast<const h8*>(br[t] + k0);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    // lane holds rows 4*lg + r of column li of each 16 x 16 block
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + 16 * j + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + 16 * i + 4 * lg + r;
                if (row < M && col < N) y32[(size_t)row * N + col] = acc[i][j][r];
            }
        }
}

constexpr int kSqBlocks = 1024;

// partial[b] = sum over this block's share of (a - b)^2 in float64; the
// share is a fixed grid-stride set and the block sums in a fixed tree order.
__global__ void __launch_bounds__(256) sqdiff_partial_kernel(const float* __restrict__ a, const float* __restrict__ b,
                                                             long long n, double* __restrict__ partial) {
    __shared__ double red[256];
    double acc = 0.0;
    for (long long t = (long long)blockIdx.x * 256 + threadIdx.x; t < n; t += (long long)gridDim.x * 256) {
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

}  // namespace

wq_status wqh::dense_f32(const uint16_t* x, const uint16_t* w, float* y32, int M, int N, int K, hipStream_t s) {
    if (M <= 0 || N <= 0) return WQ_OK;
    hipLaunchKernelGGL(dense_ref_kernel, dim3((N + 63) / 64, (M + 63) / 64), dim3(256), 0, s, x, w, y32, M, N, K);
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
