// Packed-format kernels: act-order packing order, pack, unpack and dequant.
//
// Per-group scales and zero-points, the 2/3/4/8-bit widths and desc_act come
// from "AutoGPTQ vs The Stack v2" (first capability paragraph).  The layout
// itself (little-endian bitstream per row, act-order columns in stable
// g_idx order) is this library's own and is spelled out in include/wq.h.
#include <vector>

#include "wq_common.h"

namespace {

using namespace wq;

// ---------------------------------------------------------------- perm --
// One thread per group: scan g_idx in channel order and emit the group's
// members in increasing k, which is exactly the stable sort by group.  A
// group with more than gs members writes only its first gs; the host-side
// check after the kernel rejects any map whose groups are not all of size gs.
__global__ void __launch_bounds__(256) act_order_perm_kernel(const int32_t* __restrict__ g_idx, int K,
                                                             int gs, int G, int32_t* __restrict__ perm) {
    extern __shared__ int32_t s_gidx[];
    const bool staged = (size_t(K) * 4 <= 64 * 1024);
    if (staged) {
        for (int k = threadIdx.x; k < K; k += blockDim.x) s_gidx[k] = g_idx[k];
        __syncthreads();
    }
    const int32_t* src = staged ? s_gidx : g_idx;
    for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < G; j += gridDim.x * blockDim.x) {
        int count = 0;
        for (int k = 0; k < K; ++k) {
            if (src[k] == j) {
                if (count < gs) perm[j * gs + count] = k;
                ++count;
            }
        }
    }
}

// -------------------------------------------------------------- pack ----
// One thread per (row, 32-code chunk): gather the chunk's codes (through
// perm) and write its `bits` words.
template <int BITS>
__global__ void __launch_bounds__(256) pack_kernel(const uint8_t* __restrict__ codes,
                                                   const int32_t* __restrict__ perm, int K, int N,
                                                   uint32_t* __restrict__ packed) {
    const int chunks = K / 32;
    const long long total = (long long)N * chunks;
    for (long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (long long)gridDim.x * blockDim.x) {
        const int n = int(t / chunks), c = int(t % chunks);
        const uint8_t* row = codes + (size_t)n * K;
        uint32_t words[BITS];
#pragma unroll
        for (int i = 0; i < BITS; ++i) words[i] = 0;
        for (int j = 0; j < 32; ++j) {
            const int kp = c * 32 + j;
            const int k = perm ? perm[kp] : kp;
            const uint32_t q = row[k] & ((1u << BITS) - 1u);
            const int bit = j * BITS;
            words[bit >> 5] |= q << (bit & 31);
            if ((bit & 31) + BITS > 32) words[(bit >> 5) + 1] |= q >> (32 - (bit & 31));
        }
        uint32_t* dst = packed + (size_t)n * (K / 32) * BITS + (size_t)c * BITS;
#pragma unroll
        for (int i = 0; i < BITS; ++i) dst[i] = words[i];
    }
}

// Packing without a permutation from 16-byte aligned codes: the chunk's 32
// codes arrive in two 16-byte loads and its words leave in vector stores
// (same bitstream as pack_kernel).
template <int BITS>
__global__ void __launch_bounds__(256) pack_vec_kernel(const uint8_t* __restrict__ codes, int K, int N,
                                                       uint32_t* __restrict__ packed) {
    const int chunks = K / 32;
    const long long total = (long long)N * chunks;
    for (long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (long long)gridDim.x * blockDim.x) {
        const u4* src = reinterpret_cast<const u4*>(codes + (size_t)t * 32);  // row n, chunk c = t
        const u4 a = src[0], b = src[1];
        const uint32_t in[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        uint32_t words[BITS];
#pragma unroll
        for (int i = 0; i < BITS; ++i) words[i] = 0;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const uint32_t q = (in[j >> 2] >> (8 * (j & 3))) & ((1u << BITS) - 1u);
            const int bit = j * BITS;
            words[bit >> 5] |= q << (bit & 31);
            if ((bit & 31) + BITS > 32) words[(bit >> 5) + 1] |= q >> (32 - (bit & 31));
        }
        uint32_t* dst = packed + (size_t)t * BITS;
        if constexpr (BITS == 4) {
            *reinterpret_cast<u4*>(dst) = u4{words[0], words[1], words[2], words[3]};
        } else if constexpr (BITS == 8) {
            reinterpret_cast<u4*>(dst)[0] = u4{words[0], words[1], words[2], words[3]};
            reinterpret_cast<u4*>(dst)[1] = u4{words[4], words[5], words[6], words[7]};
        } else {
#pragma unroll
            for (int i = 0; i < BITS; ++i) dst[i] = words[i];
        }
    }
}

// ----------------------------------------------- unpack and dequant -----
// One thread per (row, chunk): decode with the same routine the GEMV/GEMM
// kernels use and scatter back to original channel order.
template <int BITS, bool DEQUANT>
__global__ void __launch_bounds__(256) unpack_kernel(const uint32_t* __restrict__ packed,
                                                     const uint16_t* __restrict__ scales,
                                                     const uint8_t* __restrict__ zeros,
                                                     const int32_t* __restrict__ perm, int K, int N,
                                                     int gs, uint8_t* __restrict__ codes_out,
                                                     uint16_t* __restrict__ w_out) {
    const int chunks = K / 32;
    const int G = K / gs;
    const long long total = (long long)N * chunks;
    for (long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (long long)gridDim.x * blockDim.x) {
        const int n = int(t / chunks), c = int(t % chunks);
        const uint32_t* src = packed + (size_t)n * chunks * BITS + (size_t)c * BITS;
        uint32_t w[BITS];
#pragma unroll
        for (int i = 0; i < BITS; ++i) w[i] = src[i];
        uint32_t h[16];
        decode_chunk<BITS>(w, h);
        uint32_t zz = 0, ss = 0;
        if (DEQUANT) {
            const int g = (c * 32) / gs;
            const uint32_t z = zeros ? uint32_t(zeros[(size_t)n * G + g]) : (1u << (BITS - 1));
            zz = zero_pair(z);
            ss = scale_pair(scales[(size_t)n * G + g]);
        }
#pragma unroll
        for (int p = 0; p < 16; ++p) {
            const int b = p >> 2, i = p & 3;
            const int kp0 = c * 32 + 8 * b + i, kp1 = kp0 + 4;
            const int k0 = perm ? perm[kp0] : kp0;
            const int k1 = perm ? perm[kp1] : kp1;
            if (DEQUANT) {
                const uint32_t v = as_u32(dequant_pair(h[p], zz, ss));
                w_out[(size_t)n * K + k0] = uint16_t(v & 0xFFFFu);
                w_out[(size_t)n * K + k1] = uint16_t(v >> 16);
            } else {
                codes_out[(size_t)n * K + k0] = uint8_t(h[p] & 0xFFu);
                codes_out[(size_t)n * K + k1] = uint8_t((h[p] >> 16) & 0xFFu);
            }
        }
    }
}

int grid_for(long long work, int block) {
    long long g = (work + block - 1) / block;
    if (g > 65536) g = 65536;
    if (g < 1) g = 1;
    return int(g);
}

template <template <int> class F, typename... A>
wq_status dispatch_bits(int bits, A... a) {
    switch (bits) {
        case 2: return F<2>::run(a...);
        case 3: return F<3>::run(a...);
        case 4: return F<4>::run(a...);
        case 8: return F<8>::run(a...);
    }
    return WQ_ERR_UNSUPPORTED;
}

template <int BITS>
struct PackRun {
    static wq_status run(const uint8_t* codes, const int32_t* perm, int K, int N, uint32_t* packed,
                         hipStream_t s) {
        const long long work = (long long)N * (K / 32);
        if (!perm && wqh::aligned16(codes))
            hipLaunchKernelGGL(pack_vec_kernel<BITS>, dim3(grid_for(work, 256)), dim3(256), 0, s, codes, K, N,
                               packed);
        else
            hipLaunchKernelGGL(pack_kernel<BITS>, dim3(grid_for(work, 256)), dim3(256), 0, s, codes, perm, K,
                               N, packed);
        return wqh::launch_status();
    }
};

template <int BITS>
struct UnpackRun {
    static wq_status run(const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                         const int32_t* perm, int K, int N, int gs, uint8_t* codes, uint16_t* w,
                         hipStream_t s) {
        const long long work = (long long)N * (K / 32);
        if (w)
            hipLaunchKernelGGL((unpack_kernel<BITS, true>), dim3(grid_for(work, 256)), dim3(256), 0, s,
                               packed, scales, zeros, perm, K, N, gs, codes, w);
        else
            hipLaunchKernelGGL((unpack_kernel<BITS, false>), dim3(grid_for(work, 256)), dim3(256), 0, s,
                               packed, scales, zeros, perm, K, N, gs, codes, w);
        return wqh::launch_status();
    }
};

}  // namespace

extern "C" wq_status wq_act_order_perm(const int32_t* g_idx, int32_t K, int32_t group_size, int32_t* perm,
                                       void* stream) {
    if (!g_idx || !perm || K <= 0 || K % 32) return WQ_ERR_ARG;
    const int gs = wqh::resolve_group(K, group_size);
    if (!gs) return WQ_ERR_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int G = K / gs;
    const size_t lds = (size_t(K) * 4 <= 64 * 1024) ? size_t(K) * 4 : 0;
    hipLaunchKernelGGL(act_order_perm_kernel, dim3((G + 255) / 256), dim3(256), lds, s, g_idx, int(K), gs, G,
                       perm);
    wq_status st = wqh::launch_status();
    if (st != WQ_OK) return st;
    // Validate on the host: every group id in range and perm a permutation
    // that lists each group's channels in a run of exactly gs entries.
    std::vector<int32_t> hg(K), hp(K);
    st = wqh::hip_status(hipMemcpyAsync(hg.data(), g_idx, size_t(K) * 4, hipMemcpyDeviceToHost, s));
    if (st == WQ_OK) st = wqh::hip_status(hipMemcpyAsync(hp.data(), perm, size_t(K) * 4, hipMemcpyDeviceToHost, s));
    if (st == WQ_OK) st = wqh::hip_status(hipStreamSynchronize(s));
    if (st != WQ_OK) return st;
    std::vector<uint8_t> seen(K, 0);
    for (int k = 0; k < K; ++k)
        if (hg[k] < 0 || hg[k] >= G) return WQ_ERR_ARG;
    for (int kp = 0; kp < K; ++kp) {
        const int k = hp[kp];
        if (k < 0 || k >= K || seen[k] || hg[k] != kp / gs) return WQ_ERR_ARG;
        seen[k] = 1;
    }
    return WQ_OK;
}

extern "C" wq_status wq_pack(const uint8_t* codes, const int32_t* g_idx, int32_t K, int32_t N, int32_t bits,
                             int32_t group_size, uint32_t* packed, int32_t* perm, void* stream) {
    if (!codes || !packed || K <= 0 || N <= 0 || K % 32) return WQ_ERR_ARG;
    if (!wqh::bits_ok(bits)) return WQ_ERR_UNSUPPORTED;
    if (!wqh::aligned16(packed)) return WQ_ERR_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int32_t* use_perm = nullptr;
    if (g_idx) {
        if (!perm) return WQ_ERR_ARG;
        const wq_status st = wq_act_order_perm(g_idx, K, group_size, perm, stream);
        if (st != WQ_OK) return st;
        use_perm = perm;
    }
    return dispatch_bits<PackRun>(bits, codes, use_perm, int(K), int(N), packed, s);
}

extern "C" wq_status wq_unpack(const uint32_t* packed, const int32_t* perm, int32_t K, int32_t N, int32_t bits,
                               uint8_t* codes, void* stream) {
    if (!codes || !packed || K <= 0 || N <= 0 || K % 32) return WQ_ERR_ARG;
    if (!wqh::bits_ok(bits)) return WQ_ERR_UNSUPPORTED;
    if (!wqh::aligned16(packed)) return WQ_ERR_ARG;
    return dispatch_bits<UnpackRun>(bits, packed, (const uint16_t*)nullptr, (const uint8_t*)nullptr, perm,
                                    int(K), int(N), int(K), codes, (uint16_t*)nullptr,
                                    static_cast<hipStream_t>(stream));
}

extern "C" wq_status wq_dequant(const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                                const int32_t* perm, int32_t K, int32_t N, int32_t bits, int32_t group_size,
                                uint16_t* w, void* stream) {
    if (!w || !packed || !scales || K <= 0 || N <= 0 || K % 32) return WQ_ERR_ARG;
    if (!wqh::bits_ok(bits)) return WQ_ERR_UNSUPPORTED;
    const int gs = wqh::resolve_group(K, group_size);
    if (!gs || !wqh::aligned16(packed)) return WQ_ERR_ARG;
    return dispatch_bits<UnpackRun>(bits, packed, scales, zeros, perm, int(K), int(N), gs, (uint8_t*)nullptr,
                                    w, static_cast<hipStream_t>(stream));
}
