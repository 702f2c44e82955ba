// Quantization-side kernels: round-to-nearest group quantization, the AWQ
// per-channel scale, the AWQ weight fold and the activation division.
//
// Round-to-nearest as the baseline quantizer: "GPTQ, AWQ and the rules of
// post-training quantization", section "The problem both methods solve".
// AWQ rescaling (multiply input channel k of W by s_k, divide the matching
// activation by s_k, s_k = mean activation magnitude to the power alpha):
// same page, section "AWQ: find the one percent that matters".
#include <math.h>

#include <algorithm>

#include "wq_common.h"

namespace {

using namespace wq;

__device__ __forceinline__ float h2f(uint16_t h) { return float(__builtin_bit_cast(_Float16, h)); }
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// float64 -> fp16 with a single round-to-nearest-even (no detour through
// fp32, which could round twice).  Finite, non-negative inputs are all the
// AWQ scale produces; signs, infinities and NaN are handled for completeness.
__device__ uint16_t f64_to_f16_rne(double d) {
    const uint64_t b = __builtin_bit_cast(uint64_t, d);
    const uint16_t sign = uint16_t((b >> 48) & 0x8000u);
    const int exp = int((b >> 52) & 0x7FF);
    const uint64_t man = b & ((1ull << 52) - 1);
    if (exp == 0x7FF) return sign | 0x7C00u | (man ? 0x200u : 0u);
    if (exp == 0) return sign;  // float64 subnormal: far below the fp16 range
    const int e = exp - 1023;
    if (e > 15) return sign | 0x7C00u;
    const uint64_t sig = man | (1ull << 52);
    // fp16 normal numbers keep 10 fraction bits; subnormals are multiples of 2^-24
    const int shift = (e >= -14) ? 42 : 42 + (-14 - e);
    if (shift > 63) return sign;
    uint64_t q = sig >> shift;
    const uint64_t rem = sig & ((1ull << shift) - 1);
    const uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (q & 1))) ++q;
    uint32_t h;
    if (e >= -14)
        h = (uint32_t(e + 14) << 10) + uint32_t(q);  // q carries the implicit bit (1024)
    else
        h = uint32_t(q);  // subnormal; q == 1024 is the smallest normal
    if (h >= 0x7C00u) h = 0x7C00u;
    return sign | uint16_t(h);
}

// --------------------------------------------------------------- RTN ----
// One thread per (output column n, group j).  Two passes over the group's
// members: min/max (or max |w|), then the codes.
template <int BITS, bool SYM>
__global__ void __launch_bounds__(256) rtn_kernel(const uint16_t* __restrict__ w, const int32_t* __restrict__ perm,
                                                  int N, int K, int gs, uint8_t* __restrict__ codes,
                                                  uint16_t* __restrict__ scales, uint8_t* __restrict__ zeros) {
    constexpr int qmax = (1 << BITS) - 1;
    const int G = K / gs;
    const long long total = (long long)N * G;
    for (long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (long long)gridDim.x * blockDim.x) {
        const int n = int(t / G), j = int(t % G);
        const uint16_t* row = w + (size_t)n * K;
        float mn = INFINITY, mx = -INFINITY, amax = 0.f;
        for (int i = 0; i < gs; ++i) {
            const int k = perm ? perm[j * gs + i] : j * gs + i;
            const float v = h2f(row[k]);
            mn = fminf(mn, v);
            mx = fmaxf(mx, v);
            amax = fmaxf(amax, fabsf(v));
        }
        const float s32 = SYM ? __fdiv_rn(2.0f * amax, float(qmax)) : __fdiv_rn(mx - mn, float(qmax));
        uint16_t sh = f2h(s32);
        if ((sh & 0x7FFFu) == 0) sh = 0x0400u;  // 2^-14
        const float s = h2f(sh);
        float z;
        if (SYM) {
            z = float(1 << (BITS - 1));
        } else {
            z = fminf(fmaxf(rintf(__fdiv_rn(-mn, s)), 0.f), float(qmax));
            zeros[(size_t)n * G + j] = uint8_t(z);
        }
        scales[(size_t)n * G + j] = sh;
        uint8_t* crow = codes + (size_t)n * K;
        for (int i = 0; i < gs; ++i) {
            const int k = perm ? perm[j * gs + i] : j * gs + i;
            const float q = fminf(fmaxf(rintf(__fdiv_rn(h2f(row[k]), s)) + z, 0.f), float(qmax));
            crow[k] = uint8_t(q);
        }
    }
}

// Same quantizer, one block per output row, for the common case without a
// group permutation: (1) 16-byte loads of 8 weights record each 8-weight
// unit's min and max in LDS; (2) one thread per group reduces its units and
// derives scale and zero exactly as rtn_kernel does; (3) every unit is read
// again (from cache) and its 8 codes written as 8 bytes.  Same arithmetic,
// same results, bit for bit.
template <int BITS, bool SYM>
__global__ void __launch_bounds__(256) rtn_row_kernel(const uint16_t* __restrict__ w, int K, int gs,
                                                      uint8_t* __restrict__ codes, uint16_t* __restrict__ scales,
                                                      uint8_t* __restrict__ zeros) {
    constexpr int qmax = (1 << BITS) - 1;
    extern __shared__ float rtn_lds[];
    const int U = K / 8, G = K / gs, upg = gs / 8;
    float* umin = rtn_lds;
    float* umax = rtn_lds + U;
    float* gsc = rtn_lds + 2 * U;
    float* gz = gsc + G;
    const int n = blockIdx.x;
    const u4* row = reinterpret_cast<const u4*>(w + (size_t)n * K);
    // the row's 16-byte pieces stay in registers for the quantizing pass
    // (pieces past kCache * 256, for K > 16384, are read again)
    constexpr int kCache = 8;
    u4 cache[kCache];
#pragma unroll
    for (int i = 0; i < kCache; ++i) {
        const int u = threadIdx.x + 256 * i;
        cache[i] = u < U ? row[u] : u4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < kCache; ++i) {
        const int u = threadIdx.x + 256 * i;
        if (u >= U) break;
        const u4 v = cache[i];
        const uint32_t in[4] = {v.x, v.y, v.z, v.w};
        float mn = INFINITY, mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a = h2f(uint16_t(in[e])), b = h2f(uint16_t(in[e] >> 16));
            mn = fminf(mn, fminf(a, b));
            mx = fmaxf(mx, fmaxf(a, b));
        }
        umin[u] = mn;
        umax[u] = mx;
    }
    for (int u = threadIdx.x + 256 * kCache; u < U; u += 256) {
        const u4 v = row[u];
        const uint32_t in[4] = {v.x, v.y, v.z, v.w};
        float mn = INFINITY, mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float a = h2f(uint16_t(in[i])), b = h2f(uint16_t(in[i] >> 16));
            mn = fminf(mn, fminf(a, b));
            mx = fmaxf(mx, fmaxf(a, b));
        }
        umin[u] = mn;
        umax[u] = mx;
    }
    __syncthreads();
    for (int j = threadIdx.x; j < G; j += 256) {
        float mn = INFINITY, mx = -INFINITY;
        for (int u = j * upg; u < (j + 1) * upg; ++u) {
            mn = fminf(mn, umin[u]);
            mx = fmaxf(mx, umax[u]);
        }
        const float amax = fmaxf(fabsf(mn), fabsf(mx));
        const float s32 = SYM ? __fdiv_rn(2.0f * amax, float(qmax)) : __fdiv_rn(mx - mn, float(qmax));
        uint16_t sh = f2h(s32);
        if ((sh & 0x7FFFu) == 0) sh = 0x0400u;  // 2^-14
        const float sc = h2f(sh);
        float z;
        if (SYM) {
            z = float(1 << (BITS - 1));
        } else {
            z = fminf(fmaxf(rintf(__fdiv_rn(-mn, sc)), 0.f), float(qmax));
            zeros[(size_t)n * G + j] = uint8_t(z);
        }
        scales[(size_t)n * G + j] = sh;
        gsc[j] = sc;
        gz[j] = z;
    }
    __syncthreads();
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    u2* crow = reinterpret_cast<u2*>(codes + (size_t)n * K);
    auto quant = [&](int u, const u4& v) {
        const uint32_t in[4] = {v.x, v.y, v.z, v.w};
        const int j = u / upg;
        const float sc = gsc[j], z = gz[j];
        uint32_t q[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            q[2 * i] = uint32_t(fminf(fmaxf(rintf(__fdiv_rn(h2f(uint16_t(in[i])), sc)) + z, 0.f), float(qmax)));
            q[2 * i + 1] =
                uint32_t(fminf(fmaxf(rintf(__fdiv_rn(h2f(uint16_t(in[i] >> 16)), sc)) + z, 0.f), float(qmax)));
        }
        crow[u] = u2{q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24), q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24)};
    };
#pragma unroll
    for (int i = 0; i < kCache; ++i) {
        const int u = threadIdx.x + 256 * i;
        if (u < U) quant(u, cache[i]);
    }
    for (int u = threadIdx.x + 256 * kCache; u < U; u += 256) quant(u, row[u]);
}

// --------------------------------------------------------------- AWQ ----
// Float64 mean of |x| down each input channel.  A block owns 64 channels
// and 1024 threads: thread (c, r) = (t % 64, t / 64) sums rows r, r + 16,
// ... of channel c (a wavefront reads 64 consecutive channels of one row),
// then the 16 partial sums of a channel are added in phase order.
__global__ void __launch_bounds__(1024) awq_scales_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                          double alpha, uint16_t* __restrict__ s_out) {
    __shared__ double part[16][64];
    const int c = threadIdx.x & 63, r = threadIdx.x >> 6;
    const int k = blockIdx.x * 64 + c;
    double acc = 0.0;
    if (k < K)
        for (int m = r; m < M; m += 16) acc += fabs(double(h2f(x[(size_t)m * K + k])));
    part[r][c] = acc;
    __syncthreads();
    if (r != 0 || k >= K) return;
    acc = part[0][c];
    for (int i = 1; i < 16; ++i) acc += part[i][c];
    const double a = acc / double(M);
    const double s = (alpha == 0.5) ? sqrt(a) : pow(a, alpha);
    uint16_t h = f64_to_f16_rne(s);
    if ((h & 0x7FFFu) == 0) h = 0x0400u;
    s_out[k] = h;
}

// The same statistics with 16-byte loads (K a multiple of 64, x 16-byte
// aligned): thread t reads channels 8 (t % 8) .. + 7 of the block's 64 on
// rows t / 8, + 128, ... (one 16-byte load per row); the 8 row phases of a
// wavefront are added by lane shuffles and the 16 wavefronts' sums in
// wavefront order (fixed order, float64 throughout).
__device__ __forceinline__ double shfl_xor_f64(double v, int mask) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = uint32_t(__shfl_xor(int(uint32_t(b)), mask));
    const uint32_t hi = uint32_t(__shfl_xor(int(uint32_t(b >> 32)), mask));
    return __builtin_bit_cast(double, (uint64_t(hi) << 32) | lo);
}

__global__ void __launch_bounds__(1024) awq_scales_vec_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                              double alpha, uint16_t* __restrict__ s_out) {
    __shared__ double part[16][64];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int cg = t & 7, rp = t >> 3;
    const int k0 = blockIdx.x * 64 + 8 * cg;
    double acc[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    for (int m = rp; m < M; m += 128) {
        const u4 v = *reinterpret_cast<const u4*>(x + (size_t)m * K + k0);
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] += fabs(double(h2f(uint16_t(w4[i] & 0xFFFFu))));
            acc[2 * i + 1] += fabs(double(h2f(uint16_t(w4[i] >> 16))));
        }
    }
    // lanes cg, cg + 8, ..., cg + 56 of a wavefront hold the same channels
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        acc[j] += shfl_xor_f64(acc[j], 8);
        acc[j] += shfl_xor_f64(acc[j], 16);
        acc[j] += shfl_xor_f64(acc[j], 32);
    }
    if (lane < 8) {
#pragma unroll
        for (int j = 0; j < 8; ++j) part[wave][8 * cg + j] = acc[j];
    }
    __syncthreads();
    if (t >= 64) return;
    const int k = blockIdx.x * 64 + t;
    double a = part[0][t];
    for (int i = 1; i < 16; ++i) a += part[i][t];
    a /= double(M);
    const double sv = (alpha == 0.5) ? sqrt(a) : pow(a, alpha);
    uint16_t h = f64_to_f16_rne(sv);
    if ((h & 0x7FFFu) == 0) h = 0x0400u;
    s_out[k] = h;
}

__global__ void __launch_bounds__(256) awq_fold_kernel(const uint16_t* __restrict__ w, const uint16_t* __restrict__ s,
                                                       long long total, int K, uint16_t* __restrict__ w_out) {
    for (long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (long long)gridDim.x * blockDim.x) {
        const int k = int(t % K);
        w_out[t] = f2h(h2f(w[t]) * h2f(s[k]));  // exact fp32 product, one rounding
    }
}

// The fold with 16-byte loads and stores (K a multiple of 8, pointers
// 16-byte aligned): 8 weights per thread, the same exact products.
__global__ void __launch_bounds__(256) awq_fold_vec_kernel(const uint16_t* __restrict__ w,
                                                           const uint16_t* __restrict__ s, long long total8, int K,
                                                           uint16_t* __restrict__ w_out) {
    const int K8 = K / 8;
    for (long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x; t < total8;
         t += (long long)gridDim.x * blockDim.x) {
        const int k0 = int(t % K8) * 8;
        const u4 v = reinterpret_cast<const u4*>(w)[t];
        const u4 sv = *reinterpret_cast<const u4*>(s + k0);
        const uint32_t in[4] = {v.x, v.y, v.z, v.w}, sc[4] = {sv.x, sv.y, sv.z, sv.w};
        uint32_t out[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = h2f(uint16_t(in[i])) * h2f(uint16_t(sc[i]));
            const float hi = h2f(uint16_t(in[i] >> 16)) * h2f(uint16_t(sc[i] >> 16));
            out[i] = uint32_t(f2h(lo)) | (uint32_t(f2h(hi)) << 16);  // exact fp32 products, one rounding
        }
        reinterpret_cast<u4*>(w_out)[t] = u4{out[0], out[1], out[2], out[3]};
    }
}

// x_out = fp16(x / s), 8 elements per thread (K is a multiple of 32, so rows
// split into whole 8-element groups).
// Thread (blockIdx.x, threadIdx.x) owns 8-channel block kb of every row in
// its row range: s and its conversions are read once, RU rows' loads go out
// together before any division, and no per-element index division is needed.
constexpr int kScaleActRows = 4;
__global__ void __launch_bounds__(256) scale_act_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ s,
                                                        int M, int K, int rows_per_block, uint16_t* __restrict__ x_out) {
    constexpr int RU = kScaleActRows;
    const int K8 = K / 8;
    const int kb = blockIdx.x * blockDim.x + threadIdx.x;
    if (kb >= K8) return;
    const u4 sv = reinterpret_cast<const u4*>(s)[kb];
    const uint32_t sc[4] = {sv.x, sv.y, sv.z, sv.w};
    float sf[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        sf[2 * i] = h2f(uint16_t(sc[i]));
        sf[2 * i + 1] = h2f(uint16_t(sc[i] >> 16));
    }
    const int m_begin = blockIdx.y * rows_per_block;
    const int m_end = min(M, m_begin + rows_per_block);
    for (int m0 = m_begin; m0 < m_end; m0 += RU) {
        u4 v[RU];
#pragma unroll
        for (int u = 0; u < RU; ++u)
            v[u] = reinterpret_cast<const u4*>(x)[size_t(min(m0 + u, m_end - 1)) * K8 + kb];
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            if (m0 + u >= m_end) break;
            const uint32_t in[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
            uint32_t out[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float lo = __fdiv_rn(h2f(uint16_t(in[i])), sf[2 * i]);
                const float hi = __fdiv_rn(h2f(uint16_t(in[i] >> 16)), sf[2 * i + 1]);
                out[i] = uint32_t(f2h(lo)) | (uint32_t(f2h(hi)) << 16);
            }
            reinterpret_cast<u4*>(x_out)[size_t(m0 + u) * K8 + kb] = u4{out[0], out[1], out[2], out[3]};
        }
    }
}

int grid_for(long long work, int block, long long cap = 65536) {
    long long g = (work + block - 1) / block;
    if (g > cap) g = cap;
    if (g < 1) g = 1;
    return int(g);
}

template <int BITS>
wq_status launch_rtn(const uint16_t* w, const int32_t* perm, int N, int K, int gs, bool sym, uint8_t* codes,
                     uint16_t* scales, uint8_t* zeros, hipStream_t s) {
    // per-row kernel: no permutation, 16-byte weight rows, 8-byte code rows,
    // unit and group tables within 64 KB of LDS
    const size_t lds = size_t(K / 8) * 8 + size_t(K / gs) * 8;
    if (!perm && wqh::aligned16(w) && (reinterpret_cast<uintptr_t>(codes) & 7u) == 0 && lds <= 65536) {
        if (sym)
            hipLaunchKernelGGL((rtn_row_kernel<BITS, true>), dim3(N), dim3(256), lds, s, w, K, gs, codes, scales,
                               zeros);
        else
            hipLaunchKernelGGL((rtn_row_kernel<BITS, false>), dim3(N), dim3(256), lds, s, w, K, gs, codes, scales,
                               zeros);
        return wqh::launch_status();
    }
    const long long work = (long long)N * (K / gs);
    const dim3 grid(grid_for(work, 256)), block(256);
    if (sym)
        hipLaunchKernelGGL((rtn_kernel<BITS, true>), grid, block, 0, s, w, perm, N, K, gs, codes, scales, zeros);
    else
        hipLaunchKernelGGL((rtn_kernel<BITS, false>), grid, block, 0, s, w, perm, N, K, gs, codes, scales, zeros);
    return wqh::launch_status();
}

}  // namespace

extern "C" wq_status wq_quantize_rtn(const uint16_t* w, const int32_t* perm, int32_t N, int32_t K, int32_t bits,
                                     int32_t group_size, int32_t symmetric, uint8_t* codes, uint16_t* scales,
                                     uint8_t* zeros, void* stream) {
    if (!w || !codes || !scales || N <= 0 || K <= 0 || K % 32) return WQ_ERR_ARG;
    if (!wqh::bits_ok(bits)) return WQ_ERR_UNSUPPORTED;
    const int gs = wqh::resolve_group(K, group_size);
    if (!gs) return WQ_ERR_ARG;
    if (symmetric ? (zeros != nullptr) : (zeros == nullptr)) return WQ_ERR_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (bits) {
        case 2: return launch_rtn<2>(w, perm, N, K, gs, symmetric, codes, scales, zeros, s);
        case 3: return launch_rtn<3>(w, perm, N, K, gs, symmetric, codes, scales, zeros, s);
        case 4: return launch_rtn<4>(w, perm, N, K, gs, symmetric, codes, scales, zeros, s);
        default: return launch_rtn<8>(w, perm, N, K, gs, symmetric, codes, scales, zeros, s);
    }
}

extern "C" wq_status wq_awq_scales(const uint16_t* x, int32_t M, int32_t K, double alpha, uint16_t* s_out,
                                   void* stream) {
    if (!x || !s_out || M <= 0 || K <= 0) return WQ_ERR_ARG;
    if (!(alpha >= 0.0 && alpha <= 1.0)) return WQ_ERR_ARG;
    if (K % 64 == 0 && wqh::aligned16(x))
        hipLaunchKernelGGL(awq_scales_vec_kernel, dim3(K / 64), dim3(1024), 0, static_cast<hipStream_t>(stream), x,
                           int(M), int(K), alpha, s_out);
    else
        hipLaunchKernelGGL(awq_scales_kernel, dim3((K + 63) / 64), dim3(1024), 0, static_cast<hipStream_t>(stream),
                           x, int(M), int(K), alpha, s_out);
    return wqh::launch_status();
}

extern "C" wq_status wq_awq_fold(const uint16_t* w, const uint16_t* s, int32_t N, int32_t K, uint16_t* w_out,
                                 void* stream) {
    if (!w || !s || !w_out || N <= 0 || K <= 0) return WQ_ERR_ARG;
    const long long total = (long long)N * K;
    if (K % 8 == 0 && wqh::aligned16(w) && wqh::aligned16(s) && wqh::aligned16(w_out))
        hipLaunchKernelGGL(awq_fold_vec_kernel, dim3(grid_for(total / 8, 256, 8192)), dim3(256), 0,
                           static_cast<hipStream_t>(stream), w, s, total / 8, int(K), w_out);
    else
        hipLaunchKernelGGL(awq_fold_kernel, dim3(grid_for(total, 256)), dim3(256), 0,
                           static_cast<hipStream_t>(stream), w, s, total, int(K), w_out);
    return wqh::launch_status();
}

extern "C" wq_status wq_scale_act(const uint16_t* x, const uint16_t* s, int32_t M, int32_t K, uint16_t* x_out,
                                  void* stream) {
    if (M < 0 || K <= 0 || K % 32) return WQ_ERR_ARG;
    if (M == 0) return WQ_OK;  // empty problem: no pointer is read
    if (!x || !s || !x_out) return WQ_ERR_ARG;
    if (!wqh::aligned16(x) || !wqh::aligned16(x_out) || !wqh::aligned16(s)) return WQ_ERR_ARG;
    // about 4096 blocks: K/2048 column strips times row ranges of at least
    // kScaleActRows rows
    const int K8 = K / 8;
    const int gx = (K8 + 255) / 256;
    int gy = std::max(1, std::min(M, 4096 / gx));
    int rows = (M + gy - 1) / gy;
    rows = std::max(rows, std::min(M, kScaleActRows));
    gy = (M + rows - 1) / rows;
    hipLaunchKernelGGL(scale_act_kernel, dim3(gx, gy), dim3(256), 0, static_cast<hipStream_t>(stream), x, s, int(M),
                       int(K), rows, x_out);
    return wqh::launch_status();
}
