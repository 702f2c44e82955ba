// Skinny matrix-core kernel for small batches (2 <= M <= 16):
// y[M][N] = x[M][K] . dequant(Wq)^T with the weights streamed once from HBM.
//
// A batch of a few tokens is still bound by the weight stream (at M = 16 the
// layer does 64 flops per packed byte against a ridge of about 315), but at
// M activation rows a vector-ALU GEMV spends M fp16-pair dot products per
// weight pair and runs out of ALU long before memory.  Here the products go
// to the matrix cores ("AutoAWQ vs The Stack v2", WQLinear_* paragraph: a
// GEMM variant for batches, a GEMV variant for single tokens; this is the
// bridge between the two) and the vector ALU only decodes and dequantizes.
//
// One v_mfma_f32_16x16x32_f16 multiplies a 16 x 32 activation fragment by a
// 32 x 16 weight fragment.  Lane l supplies activation row l % 16 (rows at
// or past M repeat the last real row; their outputs are discarded) and
// weight row n0 + l % 16, both at k-block l / 16 of the 32.  A lane's 16-byte
// load holds one 32-code chunk, i.e. four k-blocks: it feeds four
// instructions, the k-blocks of four consecutive chunks spread over the four
// lane groups.  One wavefront load instruction therefore reads 16 rows x 64
// bytes; each lane loads two chunks four apart per step, so every step reads
// whole 128-byte lines of 16 rows (8 chunks = 256 k per row).
//
// Work split: output rows are cut into 16-row tiles and block b owns a
// contiguous range of tiles.  The block's eight wavefronts split each tile's
// steps (wavefront w takes steps w, w + 8, ...), so even a 4096-row layer
// keeps every compute unit streaming; at the end of a tile each wavefront
// writes its 16 x 16 partial product to LDS, and after a barrier the block
// adds the eight partials in a fixed order (deterministic) into an output
// buffer in LDS, written to y after the last tile.  Weight loads run D steps
// ahead across tile boundaries and are issued unconditionally (only the last
// D items refill conditionally), so the compiler's wait counts stay exact;
// the barriers wait for LDS only.
//
// The activations are staged once per block in LDS, each row padded by 16
// bytes (conflict-free fragment reads), in the decoder's pair order (codes
// i and i + 4 of an 8-code block share a pair), and every weight is
// dequantized exactly as in wq_dequant: fp16((q - z) * s), one rounding,
// then multiplied in the matrix cores with fp32 accumulation.
#include <algorithm>

#include "wq_common.h"

namespace {

using namespace wq;

typedef _Float16 h8v __attribute__((ext_vector_type(8)));

constexpr int kSkinnyWaves = 8;

template <int BITS>
__device__ __forceinline__ void load_chunk_nt(const uint32_t* p, uint32_t* w) {
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

// Decoder of the pair order above for one chunk: 16 fp16 pairs, pair 4b + i
// holding codes 8b + i and 8b + i + 4 as exact fp16 integers B + q, B = 1024
// for i = 0, 2 and kOdd<BITS> for i = 1, 3 (4-bit: the upper nibble of a byte
// is exposed in place under exponent 0x5400, fp16 64, whose mantissa step at
// bit 4 is exactly 1).
template <int BITS>
constexpr uint32_t kOdd = BITS == 4 ? 64u : 1024u;

template <int BITS>
__device__ __forceinline__ void decode_pairs(const uint32_t* w, uint32_t* h) {
    if constexpr (BITS == 4) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t v = w[b], v8 = v >> 8;
            h[4 * b + 0] = and_or(v, 0x000F000Fu, kMagic2);
            h[4 * b + 1] = and_or(v, 0x00F000F0u, 0x54005400u);
            h[4 * b + 2] = and_or(v8, 0x000F000Fu, kMagic2);
            h[4 * b + 3] = and_or(v8, 0x00F000F0u, 0x54005400u);
        }
    } else {
        decode_chunk<BITS>(w, h);
    }
}

// Sum over the 16 lanes of a DPP row, valid in every lane of the row: quad
// permutes, then half-row and row mirrors (fixed order).
__device__ __forceinline__ float row16_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
    return v;
}

// x' = fp16(fp32(x) / fp32(s)) for 8 activations, correctly rounded
// division then one rounding (the AWQ input scaling of wq_scale_act).
__device__ __forceinline__ u4 divide_block(u4 v, u4 t) {
    const uint32_t in[4] = {v.x, v.y, v.z, v.w}, st[4] = {t.x, t.y, t.z, t.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = __fdiv_rn(float(__builtin_bit_cast(_Float16, uint16_t(in[i]))),
                                   float(__builtin_bit_cast(_Float16, uint16_t(st[i]))));
        const float hi = __fdiv_rn(float(__builtin_bit_cast(_Float16, uint16_t(in[i] >> 16))),
                                   float(__builtin_bit_cast(_Float16, uint16_t(st[i] >> 16))));
        o[i] = uint32_t(__builtin_bit_cast(uint16_t, (_Float16)lo)) |
               (uint32_t(__builtin_bit_cast(uint16_t, (_Float16)hi)) << 16);
    }
    return u4{o[0], o[1], o[2], o[3]};
}

// EX: act_scale (nullable, fp16 [K]) divides the activations while they are
// staged, bit-identical to wq_scale_act; bias (nullable, fp16 [N]) is added
// to the fp32 sums before the output rounding.
// FACT (group size a multiple of 128 and K a multiple of 256): the matrix
// cores multiply the decoded codes B + q themselves, and each 128-channel
// group's product C (one group for all four lane groups of an instruction:
// they hold four consecutive chunks) is corrected once per lane,
//     sum_k x_k (q_k - z) s = s (C - (1024 + z) Xe - (kOdd + z) Xo),
// with Xe, Xo the sums of the group's activations over the pairs of base
// 1024 and base kOdd, computed when x is staged.  Otherwise every weight is
// dequantized, fp16((q - z) s), before the product.
template <int BITS, int D, bool HAS_Z, bool EX, bool FACT>
__global__ void __launch_bounds__(64 * kSkinnyWaves) skinny_kernel(const uint16_t* __restrict__ x,
                                                                 const uint32_t* __restrict__ packed,
                                                                 const uint16_t* __restrict__ scales,
                                                                 const uint8_t* __restrict__ zeros,
                                                                 uint16_t* __restrict__ y, int M, int N, int K,
                                                                 GroupDiv gd, int tpb,
                                                                 const uint16_t* __restrict__ act_scale,
                                                                 const uint16_t* __restrict__ bias) {
    constexpr int WPB = kSkinnyWaves;
    extern __shared__ u4 smem[];
    const int CN = K / 32;
    const int G = chunk_group(CN - 1, gd) + 1;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const int li = lane & 15, lg = lane >> 4;

    // LDS: x rows [M][K * 2 + 16 bytes], partials [2][WPB][64 lanes][4],
    // outputs [tpb][M][16] (fp32), [FACT] group sums float2 [K / 128][16],
    // the block's scales u16 [tpb * 16][G] and zero-points u8 [tpb * 16][G]
    const int xrs = K * 2 + 16;
    char* lds = reinterpret_cast<char*>(smem);
    float* red = reinterpret_cast<float*>(lds + size_t(M) * xrs);
    float* outb = red + 2 * WPB * 256;
    float2* xsum = reinterpret_cast<float2*>(outb + size_t(tpb) * M * 16);
    uint16_t* ssc = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(xsum) + (FACT ? K : 0));
    uint8_t* szr = reinterpret_cast<uint8_t*>(ssc + size_t(tpb) * 16 * G);

    const int n_tiles = (N + 15) / 16;
    const int t0 = blockIdx.x * tpb;
    const int T = max(0, min(tpb, n_tiles - t0));
    const int RB = max(0, min(T * 16, N - t0 * 16));  // rows of this block
    const int sc_n = RB * G;                          // their scale entries
    const size_t sbase = size_t(t0) * 16 * G;
    const int steps = (CN + 7) / 8;                                // 256-k steps per row
    const int my = wave < steps ? (steps - wave + WPB - 1) / WPB : 0;  // steps per tile of this wavefront
    const int items = T * my;

    // ---- activations, first batch: up to XU 8-element blocks per thread
    // are loaded before the weights (vector-memory loads complete in issue
    // order, so staging them waits for these only); x is contiguous [M][K],
    // block e is row e / K8, block e % K8
    const int K8 = K / 8;
    const int total = M * K8;
    constexpr int NT = 64 * WPB;
    constexpr int XU = 16;
    const int nx = (total + NT - 1) / NT;  // blocks per thread
    u4 xv[XU], xs_[XU];
#pragma unroll
    for (int u = 0; u < XU; ++u) {
        if (u < nx) {
            const int e = min(int(threadIdx.x) + NT * u, total - 1);
            xv[u] = *reinterpret_cast<const u4*>(x + size_t(e) * 8);
            if constexpr (EX) {
                if (act_scale) xs_[u] = *reinterpret_cast<const u4*>(act_scale + size_t(e % K8) * 8);
            }
        }
    }

    // ---- the block's scales and zero-points (contiguous: its rows are
    // consecutive), coalesced, also before the weights: a per-lane load of
    // its row's scale at every step would touch 16 rows' lines per
    // instruction, which costs more than the weight loads themselves
    constexpr int SU = 8;
    const int ns = (sc_n + NT - 1) / NT;
    uint32_t sv[SU], zv[SU];
#pragma unroll
    for (int u = 0; u < SU; ++u) {
        if (u < ns) {
            const int e = min(int(threadIdx.x) + NT * u, sc_n - 1);
            sv[u] = scales[sbase + e];
            if constexpr (HAS_Z) zv[u] = zeros[sbase + e];
        }
    }

    // ---- weights: issue cursor (tile ordinal it, step ordinal ij); loads
    // are unconditional and the cursor stops at the last item
    uint32_t wr[D][2][BITS];
    int it = 0, ij = 0, ii = 0;
    auto issue = [&](int d) {
        const int tile = t0 + min(it, max(T - 1, 0));
        const int n = min(tile * 16 + li, N - 1);
        const int s = wave + WPB * ij;
        const char* rowp = reinterpret_cast<const char*>(packed) + size_t(n) * CN * BITS * 4;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int c = min(8 * s + 4 * p + lg, CN - 1);
            load_chunk_nt<BITS>(reinterpret_cast<const uint32_t*>(rowp + uint32_t(c) * uint32_t(BITS * 4)), wr[d][p]);
        }
        if (ii + 1 < items) {
            ++ii;
            if (++ij == my) {
                ij = 0;
                ++it;
            }
        }
    };
#pragma unroll
    for (int d = 0; d < D; ++d) issue(d);
    __builtin_amdgcn_sched_barrier(0);

    // ---- scales and zero-points to LDS
#pragma unroll
    for (int u = 0; u < SU; ++u) {
        const int e = int(threadIdx.x) + NT * u;
        if (u < ns && e < sc_n) {
            ssc[e] = uint16_t(sv[u]);
            if constexpr (HAS_Z) szr[e] = uint8_t(zv[u]);
        }
    }
    for (int e = int(threadIdx.x) + NT * SU; e < sc_n; e += NT) {
        ssc[e] = scales[sbase + e];
        if constexpr (HAS_Z) szr[e] = zeros[sbase + e];
    }

    // ---- stage the activations: row m, 8-element block j at byte
    // m * xrs + 16 j, in pair order
    {
        // e runs over consecutive blocks in consecutive lanes and K8 is a
        // multiple of 16, so the 16 blocks of a 128-channel group sit in one
        // 16-lane row of a wavefront: their sums reduce by DPP (fixed order)
        auto put = [&](int e, u4 v, u4 t) {
            if constexpr (EX) {
                if (act_scale) v = divide_block(v, t);
            }
            const int m = e / K8;
            const int j = e - m * K8;
            const u4 o = stage_block(v);
            *reinterpret_cast<u4*>(lds + size_t(m) * xrs + 16 * j) = o;
            if constexpr (FACT) {
                const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
                float se = __builtin_amdgcn_fdot2(as_h2(o.x), one, 0.f, false);
                se = __builtin_amdgcn_fdot2(as_h2(o.z), one, se, false);
                float so = __builtin_amdgcn_fdot2(as_h2(o.y), one, 0.f, false);
                so = __builtin_amdgcn_fdot2(as_h2(o.w), one, so, false);
                se = row16_sum(se);
                so = row16_sum(so);
                if ((lane & 15) == 0) xsum[(j >> 4) * 16 + m] = make_float2(se, so);
            }
        };
#pragma unroll
        for (int u = 0; u < XU; ++u) {
            const int e = int(threadIdx.x) + NT * u;
            if (e < total) put(e, xv[u], xs_[u]);
        }
        // the rest (large M * K), batch by batch
        for (int e0 = int(threadIdx.x) + NT * XU; e0 < total; e0 += NT * XU) {
#pragma unroll
            for (int u = 0; u < XU; ++u) {
                const int e = min(e0 + NT * u, total - 1);
                xv[u] = *reinterpret_cast<const u4*>(x + size_t(e) * 8);
                if constexpr (EX) {
                    if (act_scale) xs_[u] = *reinterpret_cast<const u4*>(act_scale + size_t(e % K8) * 8);
                }
            }
#pragma unroll
            for (int u = 0; u < XU; ++u)
                if (e0 + NT * u < total) put(e0 + NT * u, xv[u], xs_[u]);
        }
    }
    __syncthreads();

    // ---- stream
    // two accumulators (one per chunk of a step) halve the dependent chain
    // of matrix instructions
    f4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
    const char* xrow = lds + size_t(min(li, M - 1)) * xrs;
    int cj = 0, ct = 0;  // compute cursor: step ordinal in the tile, tile ordinal
    auto tile_end = [&](int tord, f4 v) {
        float* mine = red + ((tord & 1) * WPB + wave) * 256 + lane * 4;
        *reinterpret_cast<f4*>(mine) = v;
        // workgroup barrier: its fences wait for LDS only (weight loads in
        // flight stay in flight), and the compiler keeps its own count of
        // those loads across it (a hand-written wait here made it drop a
        // later wait on a refilled slot)
        __syncthreads();
        // output (m, n): lane 16 (m / 4) + n, element m % 4 of each partial
        for (int o = threadIdx.x; o < M * 16; o += 64 * WPB) {
            const int m = o >> 4, nn = o & 15;
            const float* src = red + (tord & 1) * WPB * 256 + (16 * (m >> 2) + nn) * 4 + (m & 3);
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < WPB; ++w) sum += src[w * 256];
            outb[(tord * M + m) * 16 + nn] = sum;
        }
    };
    // One item: the step of slot d (its loads arrived with the D ahead).
    auto compute = [&](int d) {
                    const int s = wave + WPB * cj;
                    const int srow = min(ct * 16 + li, RB - 1) * G;  // this lane's row in ssc / szr
#pragma unroll
                    for (int p = 0; p < 2; ++p) {
                        const int c = 8 * s + 4 * p + lg;
                        const int sg = srow + chunk_group(min(c, CN - 1), gd);
                        const uint32_t sr_ = ssc[sg];
                        const uint32_t zr_ = HAS_Z ? uint32_t(szr[sg]) : (1u << (BITS - 1));
                        uint32_t h[16];
                        decode_pairs<BITS>(wr[d][p], h);
                        if constexpr (FACT) {
                            f4 cp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const u4 bv = {h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]};
                                const h8v av = *reinterpret_cast<const h8v*>(xrow + 64 * c + 16 * q);
                                cp = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(h8v, bv), cp, 0, 0,
                                                                           0);
                            }
                            // correction of the group's product: rows 4 lg + r
                            const float4* xg = reinterpret_cast<const float4*>(xsum + ((8 * s + 4 * p) >> 2) * 16 + 4 * lg);
                            const float4 x01 = xg[0], x23 = xg[1];
                            const float zf = float(zr_);
                            const float ce = -(1024.f + zf), co = -(float(kOdd<BITS>) + zf);
                            const float sf = float(__builtin_bit_cast(_Float16, uint16_t(sr_)));
                            f4& a = p == 0 ? acc : acc2;
                            a[0] = __builtin_fmaf(sf, __builtin_fmaf(co, x01.y, __builtin_fmaf(ce, x01.x, cp[0])), a[0]);
                            a[1] = __builtin_fmaf(sf, __builtin_fmaf(co, x01.w, __builtin_fmaf(ce, x01.z, cp[1])), a[1]);
                            a[2] = __builtin_fmaf(sf, __builtin_fmaf(co, x23.y, __builtin_fmaf(ce, x23.x, cp[2])), a[2]);
                            a[3] = __builtin_fmaf(sf, __builtin_fmaf(co, x23.w, __builtin_fmaf(ce, x23.z, cp[3])), a[3]);
                            continue;
                        }
                        const bool kval = c < CN;
                        const uint32_t z = zr_;
                        const uint32_t ze = (0x6400u | z) * 0x10001u;
                        const uint32_t zo = BITS == 4 ? (0x5400u + (z << 4)) * 0x10001u : ze;
                        const uint32_t ss = kval ? scale_pair(uint16_t(sr_)) : 0u;
                        const int cc = min(c, CN - 1);
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            uint32_t f[4];
                            f[0] = as_u32((as_h2(h[4 * q + 0]) - as_h2(ze)) * as_h2(ss));
                            f[1] = as_u32((as_h2(h[4 * q + 1]) - as_h2(zo)) * as_h2(ss));
                            f[2] = as_u32((as_h2(h[4 * q + 2]) - as_h2(ze)) * as_h2(ss));
                            f[3] = as_u32((as_h2(h[4 * q + 3]) - as_h2(zo)) * as_h2(ss));
                            const u4 bv = {f[0], f[1], f[2], f[3]};
                            // x fragment: row li, k = 32 cc' + 8 q where the
                            // lane group's chunk is cc' = c
                            const h8v av = *reinterpret_cast<const h8v*>(xrow + 64 * cc + 16 * q);
                            if (p == 0)
                                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(h8v, bv), acc, 0,
                                                                            0, 0);
                            else
                                acc2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(h8v, bv), acc2,
                                                                             0, 0, 0);
                        }
                    }
                    };
    // after an item (and its slot's refill): the tile's last step ends it
    auto advance = [&]() {
        if (++cj == my) {
            tile_end(ct, acc + acc2);
            acc = f4{0.f, 0.f, 0.f, 0.f};
            acc2 = f4{0.f, 0.f, 0.f, 0.f};
            cj = 0;
            ++ct;
        }
    };
    if (my == 0) {
        for (int t = 0; t < T; ++t) tile_end(t, acc);
    } else {
        // full rounds: every refill loads a real item, unconditionally
        int q0 = 0;
        for (; q0 + 2 * D <= items; q0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                compute(d);
                issue(d);  // before a tile end's barrier: the loads stay D ahead
                advance();
            }
        }
        // the last items: refill only what is left (no repeated loads to
        // wait for at the end)
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (q0 + d < items) {
                compute(d);
                if (q0 + d + D < items) issue(d);
                advance();
            }
        }
#pragma unroll
        for (int d = 0; d < D; ++d)
            if (q0 + D + d < items) {
                compute(d);
                advance();
            }
    }
    // ---- outputs
    __syncthreads();
    for (int o = threadIdx.x; o < T * M * 16; o += 64 * WPB) {
        const int tord = o / (M * 16), r = o - tord * M * 16;
        const int m = r >> 4, n = (t0 + tord) * 16 + (r & 15);
        if (n < N) {
            float v = outb[o];
            if constexpr (EX) {
                if (bias) v += float(__builtin_bit_cast(_Float16, bias[n]));
            }
            y[size_t(m) * N + n] = __builtin_bit_cast(uint16_t, (_Float16)v);
        }
    }
}

}  // namespace

namespace wqh {

// LDS bytes of the skinny kernel for M rows, K channels and tpb tiles per block.
static size_t skinny_lds(int M, int K, int G, int tpb, bool fact) {
    return size_t(M) * (size_t(K) * 2 + 16) + 2 * kSkinnyWaves * 256 * 4 + size_t(tpb) * M * 16 * 4 +
           (fact ? size_t(K) : 0) + size_t(tpb) * 16 * G * 3;
}

// Launch the skinny kernel; WQ_ERR_UNSUPPORTED when it does not apply
// (act-order, M outside 1..16, K below 256, or activations beyond the LDS
// limit).
wq_status skinny_gemv(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                      const int32_t* perm, uint16_t* y, int M, int N, int K, int bits, int gs, hipStream_t s,
                      const uint16_t* act_scale, const uint16_t* bias) {
    if (perm || M < 1 || M > 16 || K < 256) return WQ_ERR_UNSUPPORTED;
    int dev = 0, cus = 256, lds_max = 64 * 1024;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && v > 0)
            lds_max = v;
    }
    const int n_tiles = (N + 15) / 16;
    const int blocks = std::min(n_tiles, cus);
    const int tpb = (n_tiles + blocks - 1) / blocks;
    const bool fact = gs % 128 == 0 && K % 256 == 0;
    const size_t lds = skinny_lds(M, K, K / gs, tpb, fact);
    if (lds > size_t(lds_max)) return WQ_ERR_UNSUPPORTED;
    const GroupDiv gd = group_magic(gs);
    constexpr int D = 2;
    auto go = [&](auto kern) {
        if (lds > 64 * 1024)
            (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                      int(lds));
        hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * kSkinnyWaves), lds, s, x, packed, scales, zeros, y, M, N, K,
                           gd, tpb, act_scale, bias);
        return launch_status();
    };
    const bool ex = act_scale || bias;
#define WQ_SKINNY_GO2(B, F)                                                                                 \
    return ex ? (zeros ? go(skinny_kernel<B, D, true, true, F>) : go(skinny_kernel<B, D, false, true, F>)) \
              : (zeros ? go(skinny_kernel<B, D, true, false, F>) : go(skinny_kernel<B, D, false, false, F>))
#define WQ_SKINNY_GO(B)          \
    if (fact) WQ_SKINNY_GO2(B, true); \
    WQ_SKINNY_GO2(B, false)
    switch (bits) {
        case 2: WQ_SKINNY_GO(2);
        case 3: WQ_SKINNY_GO(3);
        case 4: WQ_SKINNY_GO(4);
        default: WQ_SKINNY_GO(8);
    }
#undef WQ_SKINNY_GO
#undef WQ_SKINNY_GO2
}

}  // namespace wqh
