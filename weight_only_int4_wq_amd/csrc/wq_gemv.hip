// Decode GEMV: y[M][N] = x[M][K] . dequant(Wq)^T for small M (1..16).
//
// Single-token generation is memory-bound with almost no weight reuse, so
// the kernel is built to stream the packed weights once at full HBM rate
// ("AutoAWQ vs Unsloth", WQLinear_* paragraph on GEMV kernels for
// single-token generation; weights stay packed and are dequantized on the
// fly, "AutoAWQ vs The Stack v2", WQLinear_* paragraph).
//
// Work split: a 256-thread block owns 4*RW consecutive output columns, one
// wavefront per RW of them.  Lanes of a wavefront stride over the 32-code
// chunks of a weight row (consecutive lanes read consecutive 16-byte
// pieces: coalesced 128-bit loads), so every lane holds a K-slice partial sum
// per (column, activation row); the partials are reduced across the
// wavefront with butterfly shuffles at the end (split-K inside the wave, no
// atomics, deterministic).  The activations are staged once per block in
// LDS, in the pair order the decoder produces, gathered through perm for
// act-order; long K is processed in LDS-sized slabs.
#include "wq_common.h"

namespace {

using namespace wq;

template <int BITS>
__device__ __forceinline__ void load_chunk(const uint32_t* p, uint32_t* w) {
    if constexpr (BITS == 4) {
        const u4 v = __builtin_nontemporal_load(reinterpret_cast<const u4*>(p));
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else if constexpr (BITS == 8) {
        const u4 a = __builtin_nontemporal_load(reinterpret_cast<const u4*>(p));
        const u4 b = __builtin_nontemporal_load(reinterpret_cast<const u4*>(p) + 1);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else if constexpr (BITS == 2) {
        typedef uint32_t u2 __attribute__((ext_vector_type(2)));
        const u2 v = __builtin_nontemporal_load(reinterpret_cast<const u2*>(p));
        w[0] = v.x; w[1] = v.y;
    } else {
        w[0] = __builtin_nontemporal_load(p);
        w[1] = __builtin_nontemporal_load(p + 1);
        w[2] = __builtin_nontemporal_load(p + 2);
    }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

template <int BITS, int MT, int RW>
__global__ void __launch_bounds__(256) gemv_kernel(const uint16_t* __restrict__ x,
                                                   const uint32_t* __restrict__ packed,
                                                   const uint16_t* __restrict__ scales,
                                                   const uint8_t* __restrict__ zeros,
                                                   const int32_t* __restrict__ perm, uint16_t* __restrict__ y,
                                                   int M, int N, int K, int gs, int slab) {
    extern __shared__ u4 xs[];  // [MT][slab / 8] 8-element blocks, staging order
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n_base = (blockIdx.x * 4 + wave) * RW;
    const int chunks = K / 32;
    const int G = K / gs;
    const int slab_blocks = slab / 8;

    float acc[RW][MT];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;

    for (int k0 = 0; k0 < K; k0 += slab) {
        const int kn = min(slab, K - k0);
        const int nb = kn / 8;
        // ---- stage x[:, k0:k0+kn] in pair order (gathered through perm)
        for (int t = threadIdx.x; t < MT * nb; t += 256) {
            const int m = t / nb, b = t - m * nb;
            u4 v = {0u, 0u, 0u, 0u};
            if (m < M) {
                const uint16_t* xr = x + (size_t)m * K;
                const int kk = k0 + 8 * b;
                if (perm) {
                    uint32_t e[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) e[i] = xr[perm[kk + i]];
                    v.x = e[0] | (e[1] << 16); v.y = e[2] | (e[3] << 16);
                    v.z = e[4] | (e[5] << 16); v.w = e[6] | (e[7] << 16);
                } else {
                    v = *reinterpret_cast<const u4*>(xr + kk);
                }
            }
            xs[m * slab_blocks + b] = stage_block(v);
        }
        __syncthreads();

        const int cn = kn / 32;
        const int c0 = k0 / 32;
        for (int c = lane; c < cn; c += 64) {
            const int cg = c0 + c;
            const int g = (cg * 32) / gs;
            uint32_t w[RW][BITS];
            uint32_t zz[RW], ss[RW];
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const int n = n_base + r;
                if (n < N) {
                    load_chunk<BITS>(packed + (size_t)n * chunks * BITS + (size_t)cg * BITS, w[r]);
                    const uint32_t z = zeros ? uint32_t(zeros[(size_t)n * G + g]) : (1u << (BITS - 1));
                    zz[r] = zero_pair(z);
                    ss[r] = scale_pair(scales[(size_t)n * G + g]);
                } else {
#pragma unroll
                    for (int i = 0; i < BITS; ++i) w[r][i] = 0u;
                    zz[r] = zero_pair(0);
                    ss[r] = 0u;
                }
            }
            // activations of this chunk: 4 blocks = 16 pairs per row
            const u4* xc = xs + 4 * c;
            if constexpr (MT <= 4) {
                uint32_t xp[MT][16];
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const u4 v = xc[m * slab_blocks + b];
                        xp[m][4 * b] = v.x; xp[m][4 * b + 1] = v.y;
                        xp[m][4 * b + 2] = v.z; xp[m][4 * b + 3] = v.w;
                    }
#pragma unroll
                for (int r = 0; r < RW; ++r) {
                    uint32_t h[16];
                    decode_chunk<BITS>(w[r], h);
#pragma unroll
                    for (int p = 0; p < 16; ++p) {
                        const h2 wv = dequant_pair(h[p], zz[r], ss[r]);
#pragma unroll
                        for (int m = 0; m < MT; ++m)
                            acc[r][m] = __builtin_amdgcn_fdot2(wv, as_h2(xp[m][p]), acc[r][m], false);
                    }
                }
            } else {
#pragma unroll
                for (int r = 0; r < RW; ++r) {
                    uint32_t h[16];
                    decode_chunk<BITS>(w[r], h);
                    h2 wv[16];
#pragma unroll
                    for (int p = 0; p < 16; ++p) wv[p] = dequant_pair(h[p], zz[r], ss[r]);
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            const u4 v = xc[m * slab_blocks + b];
                            acc[r][m] = __builtin_amdgcn_fdot2(wv[4 * b], as_h2(v.x), acc[r][m], false);
                            acc[r][m] = __builtin_amdgcn_fdot2(wv[4 * b + 1], as_h2(v.y), acc[r][m], false);
                            acc[r][m] = __builtin_amdgcn_fdot2(wv[4 * b + 2], as_h2(v.z), acc[r][m], false);
                            acc[r][m] = __builtin_amdgcn_fdot2(wv[4 * b + 3], as_h2(v.w), acc[r][m], false);
                        }
                    }
                }
            }
        }
        __syncthreads();
    }

    // ---- split-K reduction across the wavefront, one fp16 rounding
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        const int n = n_base + r;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const float v = wave_sum(acc[r][m]);
            if (lane == 0 && n < N && m < M) y[(size_t)m * N + n] = __builtin_bit_cast(uint16_t, (_Float16)v);
        }
    }
}

constexpr size_t kLdsBudget = 64 * 1024;

template <int BITS, int MT>
wq_status launch_mt(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                    const int32_t* perm, uint16_t* y, int M, int N, int K, int gs, hipStream_t s) {
    constexpr int RW = (MT <= 2) ? 4 : 2;
    int slab = int(kLdsBudget / (size_t(MT) * 2));
    slab = (slab / 32) * 32;
    if (slab > K) slab = K;
    const size_t lds = size_t(MT) * slab * 2;
    const int blocks = (N + 4 * RW - 1) / (4 * RW);
    hipLaunchKernelGGL((gemv_kernel<BITS, MT, RW>), dim3(blocks), dim3(256), lds, s, x, packed, scales, zeros, perm,
                       y, M, N, K, gs, slab);
    return wqh::launch_status();
}

template <int BITS>
wq_status launch_bits(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                      const int32_t* perm, uint16_t* y, int M, int N, int K, int gs, hipStream_t s) {
    if (M <= 1) return launch_mt<BITS, 1>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
    if (M <= 2) return launch_mt<BITS, 2>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
    if (M <= 4) return launch_mt<BITS, 4>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
    if (M <= 8) return launch_mt<BITS, 8>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
    return launch_mt<BITS, 16>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
}

}  // namespace

namespace wqh {
wq_status check_linear_args(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint16_t* y,
                            int M, int N, int K, int bits, int group_size, int* gs_out);
}

extern "C" wq_status wq_gemv(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                             const int32_t* perm, uint16_t* y, int32_t M, int32_t N, int32_t K, int32_t bits,
                             int32_t group_size, void* workspace, size_t workspace_bytes, void* stream) {
    (void)workspace;
    (void)workspace_bytes;
    int gs = 0;
    const wq_status st = wqh::check_linear_args(x, packed, scales, y, M, N, K, bits, group_size, &gs);
    if (st != WQ_OK) return st;
    if (M > 16) return WQ_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return WQ_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (bits) {
        case 2: return launch_bits<2>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
        case 3: return launch_bits<3>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
        case 4: return launch_bits<4>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
        default: return launch_bits<8>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
    }
}
