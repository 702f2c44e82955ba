// Skinny matrix-core kernel for small batches (2 <= M <= 32):
// y[M][N] = x[M][K] . dequant(Wq)^T with the weights streamed once from HBM.
//
// A batch of a few tokens is still bound by the weight stream (at M = 16 the
// layer does 64 flops per packed byte against a ridge of about 315), but at
// M activation rows a vector-ALU GEMV spends M fp16-pair dot products per
// weight pair and runs out of ALU long before memory.  Here the products go
// to the matrix cores ("AutoAWQ vs The Stack v2", WQLinear_* paragraph: a
// GEMM variant for batches, a GEMV variant for single tokens; this is the
// bridge between the two) and the vector ALU only decodes the codes.
//
// One v_mfma_f32_16x16x32_f16 multiplies a 16 x 32 activation fragment by a
// 32 x 16 weight fragment.  Lane l supplies activation row l % 16 (rows at
// or past M repeat the last real row; their outputs are discarded) and
// weight row n0 + l % 16, both at k-block l / 16 of the 32.  With 17 to 32
// rows (MF = 2) every decoded weight fragment feeds a second instruction for
// activation rows 16..31.  A lane's 16-byte
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
// The activations are staged in LDS, each row padded by 16 bytes
// (conflict-free fragment reads), in the decoder's pair order (codes i and
// i + 4 of an 8-code block share a pair).  When M rows of K channels do not
// fit, K is cut into slabs of KS channels (a multiple of 256): the block
// streams all its tiles over one slab, adds the slab's sums into the output
// buffer, stages the next slab and goes on (the weight loads stay in flight
// across the switch).  A wavefront with no step of a slab (fewer than eight
// steps) runs one masked step per tile so every wavefront meets every barrier.
// The scales and zero-points of the block's rows and the slab's groups are
// staged alongside.
#include <algorithm>
#include <type_traits>

#include "wq_common.h"

namespace {

using namespace wq;

typedef _Float16 h8v __attribute__((ext_vector_type(8)));

constexpr int kSkinnyWaves = 8;
// Most activation rows the kernel takes (two 16-row fragments).
constexpr int kSkinnyMaxM = 32;

// weight loads in flight per lane, in steps of two 16-byte chunks
#ifndef WQ_SKINNY_D
#define WQ_SKINNY_D 2
#endif

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

// Slab geometry, the same in every block.
struct SlabGeo {
    int KS;    // channels per slab (multiple of 256); the last slab may be shorter
    int GSL;   // scale entries per staged row (groups any slab touches, at most)
};

// EX: act_scale (nullable, fp16 [K]) divides the activations while they are
// staged, bit-identical to wq_scale_act; bias (nullable, fp16 [N]) is added
// to the fp32 sums before the output rounding.
// ZSUB (group size a multiple of 128): the decoded pairs B + q have B + z
// subtracted in fp16, which is exact (both are integers below 2048), so the
// matrix cores multiply x by q - z itself; the four chunks of one
// instruction group are 128 channels of one group, so its product is
// scaled once per lane, in fp32, before it joins the accumulator:
//     sum_k x_k (q_k - z) s = s * sum_k x_k (q_k - z).
// Otherwise every weight is dequantized, fp16((q - z) s), before the product.
// SLABS: K is cut into several slabs (without it the slab switch is compiled
// out, which keeps the streaming loop's scalar state small).
// SPLIT: K is cut into slabs across blocks instead: the grid is one group of
// blocks per slab, a block stages its slab once for its tiles and writes the
// fp32 sums of that slab to part[slab][M][N] (bias and rounding are left to
// skinny_sum_kernel).  No block changes slab, so no wavefront waits at a
// slab change for activations queued behind the weight loads in flight.
// MF: 16-row activation fragments per weight fragment (M <= 16 * MF).
template <int BITS, int D, bool HAS_Z, bool EX, bool ZSUB, bool SLABS, bool SPLIT, int MF>
__global__ void __launch_bounds__(64 * kSkinnyWaves) skinny_kernel(const uint16_t* __restrict__ x,
                                                                 const uint32_t* __restrict__ packed,
                                                                 const uint16_t* __restrict__ scales,
                                                                 const uint8_t* __restrict__ zeros,
                                                                 uint16_t* __restrict__ y, int M, int N, int K,
                                                                 GroupDiv gd, int tpb, SlabGeo geo,
                                                                 const uint16_t* __restrict__ act_scale,
                                                                 const uint16_t* __restrict__ bias,
                                                                 float* __restrict__ part) {
    static_assert(!(SLABS && SPLIT), "one slab per block in the split form");
    constexpr int WPB = kSkinnyWaves;
    constexpr int NT = 64 * WPB;
    extern __shared__ u4 smem[];
    const int CN = K / 32;
    const int G = chunk_group(CN - 1, gd) + 1;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const int li = lane & 15, lg = lane >> 4;
    const int KS = geo.KS, GSL = geo.GSL;
    const int KSc = KS / 32;                   // chunks per slab
    const int nslab = SLABS ? (CN + KSc - 1) / KSc : 1;
    // SPLIT: block group s0 (bps blocks) takes slab s0 of every tile
    const int bps = SPLIT ? int(gridDim.x) / ((CN + KSc - 1) / KSc) : int(gridDim.x);
    const int s0 = SPLIT ? int(blockIdx.x) / bps : 0;
    const int bix = int(blockIdx.x) - s0 * bps;

    // LDS: x rows [M][KS * 2 + 16 bytes], partials [2][WPB][MF][64 lanes][4],
    // outputs [tpb][M][16] (fp32), the block's scales u16 [tpb * 16][GSL]
    // and zero-points u8 [tpb * 16][GSL] of the current slab
    const int xrs = KS * 2 + 16;
    char* lds = reinterpret_cast<char*>(smem);
    float* red = reinterpret_cast<float*>(lds + size_t(M) * xrs);
    float* outb = red + 2 * WPB * 256 * MF;
    uint16_t* ssc = reinterpret_cast<uint16_t*>(outb + size_t(tpb) * M * 16);
    uint8_t* szr = reinterpret_cast<uint8_t*>(ssc + size_t(tpb) * 16 * GSL);

    const int n_tiles = (N + 15) / 16;
    const int t0 = bix * tpb;
    const int T = max(0, min(tpb, n_tiles - t0));
    const int RB = max(0, min(T * 16, N - t0 * 16));  // rows of this block

    // steps (256 channels) of slab s, and this wavefront's steps per tile
    // there (at least one: a wavefront past the slab's steps runs one masked
    // step)
    auto slab_steps = [&](int s) { return (min(KSc, CN - s * KSc) + 7) / 8; };
    auto my_of = [&](int s) { return max(1, (slab_steps(s) - wave + WPB - 1) / WPB); };
    const int my_first = my_of(s0);
    const int items = SPLIT ? T * my_first : T * ((nslab - 1) * my_first + my_of(nslab - 1));

    // the slab's first group and its number of groups
    auto slab_g0 = [&](int s) { return chunk_group(s * KSc, gd); };
    auto slab_ng = [&](int s) { return chunk_group(min(CN, (s + 1) * KSc) - 1, gd) - slab_g0(s) + 1; };

    // ---- first slab, first batch of activations and scales, loaded before
    // the weights (vector-memory loads complete in issue order, so staging
    // them waits for these only).  Thread t stages 8-element blocks
    // j = t, t + NT, ... of every row; the first batch is j = t, rows below
    // XU (fewer with the division, whose temporaries would spill)
    constexpr int XU = EX ? 8 : 16;
    const int kb0 = s0 * KS;               // first channel of the first slab
    const int KB0 = min(KS, K - kb0) / 8;  // real blocks per row in it
    u4 xv[XU], xs0 = {0u, 0u, 0u, 0u};
    {
        const int j = min(int(threadIdx.x), KB0 - 1);
#pragma unroll
        for (int u = 0; u < XU; ++u)
            if (u < M) xv[u] = *reinterpret_cast<const u4*>(x + size_t(u) * K + kb0 + 8 * j);
        if constexpr (EX) {
            if (act_scale) xs0 = *reinterpret_cast<const u4*>(act_scale + kb0 + 8 * j);
        }
    }
    // scale entries of the block's rows and a slab's groups: entry e is row
    // e / ng, group g0 + e % ng (the division by the float reciprocal is
    // exact while e < 2^21: (e + 0.5) / ng stays at least 0.5 / ng away from
    // an integer, farther than the rounding error)
    auto sc_index = [&](int e, int ng, float inv, int g0) {
        const int r = int((float(e) + 0.5f) * inv);
        return size_t(min(t0 * 16 + r, N - 1)) * G + g0 + (e - r * ng);
    };
    constexpr int SU = 8;
    uint32_t sv[SU], zv[SU];
    const int ng0 = slab_ng(s0);
    const float inv0 = 1.0f / float(ng0);
    const int sc_n0 = RB * ng0;
    {
        const int g0 = slab_g0(s0);
#pragma unroll
        for (int u = 0; u < SU; ++u) {
            const size_t gi = sc_index(min(int(threadIdx.x) + NT * u, max(sc_n0 - 1, 0)), ng0, inv0, g0);
            sv[u] = scales[gi];
            if constexpr (HAS_Z) zv[u] = zeros[gi];
        }
    }

    // ---- weights: issue cursor (slab is, tile ordinal it, step ordinal
    // ij); loads are unconditional and the cursor stops at the last item
    uint32_t wr[D][2][BITS];
    // (the lane's row pointer and the step's first chunk are kept up to
    // date incrementally: the per-item work is two adds)
    int is = s0, it = 0, ij = 0, ii = 0, imy = my_first;
    int icb = s0 * KSc + 8 * wave;  // global chunk of the step's first 32-code chunk
    auto row_ptr = [&](int t) {
        const int n = min((t0 + min(t, max(T - 1, 0))) * 16 + li, N - 1);
        return reinterpret_cast<const char*>(packed) + size_t(n) * CN * BITS * 4;
    };
    const char* irow = row_ptr(0);
    auto issue = [&](int d) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int c = min(icb + 4 * p + lg, CN - 1);
            load_chunk_nt<BITS>(reinterpret_cast<const uint32_t*>(irow + uint32_t(c) * uint32_t(BITS * 4)), wr[d][p]);
        }
        if (ii + 1 < items) {
            ++ii;
            icb += 8 * WPB;
            if (++ij == imy) {
                ij = 0;
                if (++it == T) {
                    it = 0;
                    ++is;
                    imy = my_of(is);
                }
                icb = is * KSc + 8 * wave;
                irow = row_ptr(it);
            }
        }
    };
#pragma unroll
    for (int d = 0; d < D; ++d) issue(d);
    __builtin_amdgcn_sched_barrier(0);

    // ---- staging of slab s: activations (zero past K), scales, zero-points
    auto put_x = [&](int m, int j, u4 v, u4 t) {
        if constexpr (EX) {
            if (act_scale) v = divide_block(v, t);
        }
        *reinterpret_cast<u4*>(lds + size_t(m) * xrs + 16 * j) = stage_block(v);
    };
    auto put_zero = [&](int m, int j) {
        *reinterpret_cast<u4*>(lds + size_t(m) * xrs + 16 * j) = u4{0u, 0u, 0u, 0u};
    };
    auto put_sc = [&](int e, uint32_t s, uint32_t z) {
        ssc[e] = uint16_t(s);
        if constexpr (HAS_Z) szr[e] = uint8_t(z);
    };
    auto stage_rest = [&](int s, int jfirst, int mfirst) {
        // blocks j >= jfirst of slab s (rows from mfirst in the first one);
        // zeros past the end of K
        const int kb = s * KS;
        const int KBr = min(KS, K - kb) / 8;
        for (int j = jfirst, m0 = mfirst; j < KS / 8; j += NT, m0 = 0) {
            if (j >= KBr) {
                for (int m = m0; m < M; ++m) put_zero(m, j);
                continue;
            }
            u4 t = {0u, 0u, 0u, 0u};
            if constexpr (EX) {
                if (act_scale) t = *reinterpret_cast<const u4*>(act_scale + kb + 8 * j);
            }
            for (int mb = m0; mb < M; mb += XU) {
                u4 v[XU];
#pragma unroll
                for (int u = 0; u < XU; ++u)
                    if (mb + u < M) v[u] = *reinterpret_cast<const u4*>(x + size_t(mb + u) * K + kb + 8 * j);
#pragma unroll
                for (int u = 0; u < XU; ++u)
                    if (mb + u < M) put_x(mb + u, j, v[u], t);
            }
        }
    };
    auto stage_scales = [&](int s, int efirst) {
        const int ng = slab_ng(s), g0 = slab_g0(s);
        const float inv = 1.0f / float(ng);
        for (int e = efirst; e < RB * ng; e += NT) {
            const size_t gi = sc_index(e, ng, inv, g0);
            put_sc(e, scales[gi], HAS_Z ? uint32_t(zeros[gi]) : 0u);
        }
    };
    {
        const int j = int(threadIdx.x);
        if (j < KB0) {
#pragma unroll
            for (int u = 0; u < XU; ++u)
                if (u < M) put_x(u, j, xv[u], xs0);
        }
        stage_rest(s0, j, j < KB0 ? XU : 0);
#pragma unroll
        for (int u = 0; u < SU; ++u) {
            const int e = int(threadIdx.x) + NT * u;
            if (e < sc_n0) put_sc(e, sv[u], HAS_Z ? zv[u] : 0u);
        }
        stage_scales(s0, int(threadIdx.x) + NT * SU);
    }
    __syncthreads();

    // ---- stream
    // two accumulators (one per chunk of a step) halve the dependent chain
    // of matrix instructions
    f4 acc[MF], acc2[MF];
#pragma unroll
    for (int f = 0; f < MF; ++f) acc[f] = acc2[f] = f4{0.f, 0.f, 0.f, 0.f};
    const char* xrow[MF];
#pragma unroll
    for (int f = 0; f < MF; ++f) xrow[f] = lds + size_t(min(li + 16 * f, M - 1)) * xrs;
    int cs = s0, ct = 0, cj = 0, cmy = my_first, te = 0;  // compute cursor, tile ends so far
    int css8 = 8 * slab_steps(s0), cg0 = slab_g0(s0), cng = ng0;
    int ccb = 8 * wave;                                   // the step's first chunk within the slab
    int srow = min(li, RB - 1) * cng;                     // this lane's row in ssc / szr
    auto tile_end = [&](const f4 (&v)[MF]) {
#pragma unroll
        for (int f = 0; f < MF; ++f) {
            float* mine = red + (((te & 1) * WPB + wave) * MF + f) * 256 + lane * 4;
            *reinterpret_cast<f4*>(mine) = v[f];
        }
        // workgroup barrier: its fences wait for LDS only (weight loads in
        // flight stay in flight), and the compiler keeps its own count of
        // those loads across it
        __syncthreads();
        // output (m, n): fragment m / 16, lane 16 (m % 16 / 4) + n, element
        // m % 4 of each partial; thread o always owns the same outputs, so the
        // slabs add up without further synchronization
        for (int o = threadIdx.x; o < M * 16; o += NT) {
            const int m = o >> 4, nn = o & 15, f = m >> 4, mm = m & 15;
            const float* src = red + ((te & 1) * WPB * MF + f) * 256 + (16 * (mm >> 2) + nn) * 4 + (mm & 3);
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < WPB; ++w) sum += src[w * 256 * MF];
            float* dst = outb + (ct * M + m) * 16 + nn;
            *dst = (SPLIT || cs == 0) ? sum : *dst + sum;
        }
        ++te;
    };
    // One item: the step of slab cs, tile ct, step ordinal cj, from slot d.
    auto compute = [&](int d) {
        const bool live = ccb < css8;  // else a masked step
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int cl = min(ccb + 4 * p + lg, KSc - 1);  // chunk within the slab
            // ZSUB: the four chunks of the instruction group share the group
            const int sg = srow - cg0 +
                           (ZSUB ? chunk_group(min(cs * KSc + ccb + 4 * p, CN - 1), gd)
                                 : chunk_group(min(cs * KSc + cl, CN - 1), gd));
            // read unconditionally, then mask (a read under the condition
            // would wait for the LDS at once)
            const uint32_t sr_ = uint32_t(ssc[sg]) & (live ? 0xFFFFu : 0u);
            const uint32_t z = HAS_Z ? uint32_t(szr[sg]) : (1u << (BITS - 1));
            const uint32_t ze = (0x6400u | z) * 0x10001u;
            const uint32_t zo = BITS == 4 ? (0x5400u + (z << 4)) * 0x10001u : ze;
            uint32_t h[16];
            decode_pairs<BITS>(wr[d][p], h);
            f4 (&a)[MF] = p == 0 ? acc : acc2;
            if constexpr (ZSUB) {
                f4 cp[MF];
#pragma unroll
                for (int f = 0; f < MF; ++f) cp[f] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    u4 bv;
                    bv.x = as_u32(as_h2(h[4 * q + 0]) - as_h2(ze));
                    bv.y = as_u32(as_h2(h[4 * q + 1]) - as_h2(zo));
                    bv.z = as_u32(as_h2(h[4 * q + 2]) - as_h2(ze));
                    bv.w = as_u32(as_h2(h[4 * q + 3]) - as_h2(zo));
#pragma unroll
                    for (int f = 0; f < MF; ++f) {
                        const h8v av = *reinterpret_cast<const h8v*>(xrow[f] + 64 * cl + 16 * q);
                        cp[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(h8v, bv), cp[f], 0, 0, 0);
                    }
                }
                const float sf = float(__builtin_bit_cast(_Float16, uint16_t(sr_)));
#pragma unroll
                for (int f = 0; f < MF; ++f)
#pragma unroll
                    for (int r = 0; r < 4; ++r) a[f][r] = __builtin_fmaf(sf, cp[f][r], a[f][r]);
            } else {
                const uint32_t ss = scale_pair(uint16_t(sr_));
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    u4 bv;
                    bv.x = as_u32((as_h2(h[4 * q + 0]) - as_h2(ze)) * as_h2(ss));
                    bv.y = as_u32((as_h2(h[4 * q + 1]) - as_h2(zo)) * as_h2(ss));
                    bv.z = as_u32((as_h2(h[4 * q + 2]) - as_h2(ze)) * as_h2(ss));
                    bv.w = as_u32((as_h2(h[4 * q + 3]) - as_h2(zo)) * as_h2(ss));
                    // x fragment: row li (+ 16 f), k = 32 cl + 8 q (the lane group's chunk)
#pragma unroll
                    for (int f = 0; f < MF; ++f) {
                        const h8v av = *reinterpret_cast<const h8v*>(xrow[f] + 64 * cl + 16 * q);
                        a[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(h8v, bv), a[f], 0, 0, 0);
                    }
                }
            }
        }
    };
    // after an item: the tile's last step ends the tile, the slab's last
    // tile stages the next slab (every wavefront has left the slab's
    // activations by the tile end's barrier)
    auto advance = [&]() {
        ccb += 8 * WPB;
        if (++cj == cmy) {
            f4 v[MF];
#pragma unroll
            for (int f = 0; f < MF; ++f) {
                v[f] = acc[f] + acc2[f];
                acc[f] = acc2[f] = f4{0.f, 0.f, 0.f, 0.f};
            }
            tile_end(v);
            cj = 0;
            ccb = 8 * wave;
            if (++ct == T) {
                ct = 0;
                if (SLABS && cs + 1 < nslab) {
                    ++cs;
                    stage_rest(cs, int(threadIdx.x), 0);
                    stage_scales(cs, int(threadIdx.x));
                    __syncthreads();
                    cmy = my_of(cs);
                    css8 = 8 * slab_steps(cs);
                    cg0 = slab_g0(cs);
                    cng = slab_ng(cs);
                }
            }
            srow = min(ct * 16 + li, RB - 1) * cng;
        }
    };
    {
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
    for (int o = threadIdx.x; o < T * M * 16; o += NT) {
        const int tord = o / (M * 16), r = o - tord * M * 16;
        const int m = r >> 4, n = (t0 + tord) * 16 + (r & 15);
        if (n < N) {
            float v = outb[o];
            if constexpr (SPLIT) {
                part[(size_t(s0) * M + m) * N + n] = v;
            } else {
                if constexpr (EX) {
                    if (bias) v += float(__builtin_bit_cast(_Float16, bias[n]));
                }
                y[size_t(m) * N + n] = __builtin_bit_cast(uint16_t, (_Float16)v);
            }
        }
    }
}

// y[m][n] = fp16(sum over slabs s of part[s][m][n] (+ bias[n])), the slabs
// added in order, as the block-serial form accumulates them.
__global__ void __launch_bounds__(256) skinny_sum_kernel(const float* __restrict__ part, int nsl, int M, int N,
                                                         const uint16_t* __restrict__ bias,
                                                         uint16_t* __restrict__ y) {
    const size_t MN = size_t(M) * N;
    for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < MN; i += size_t(gridDim.x) * blockDim.x) {
        float v = part[i];
        for (int sl = 1; sl < nsl; ++sl) v += part[size_t(sl) * MN + i];
        if (bias) v += float(__builtin_bit_cast(_Float16, bias[i % size_t(N)]));
        y[i] = __builtin_bit_cast(uint16_t, (_Float16)v);
    }
}

// The same for N a multiple of 4: four outputs of one row per thread, 16-byte
// loads of each slab's partials, one 8-byte store (same additions, same order).
__global__ void __launch_bounds__(256) skinny_sum4_kernel(const float4* __restrict__ part, int nsl, int M, int N,
                                                          const uint16_t* __restrict__ bias,
                                                          uint2* __restrict__ y) {
    const size_t MN4 = size_t(M) * N / 4;
    const int N4 = N / 4;
    for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < MN4; i += size_t(gridDim.x) * blockDim.x) {
        float4 v = part[i];
        for (int sl = 1; sl < nsl; ++sl) {
            const float4 w = part[size_t(sl) * MN4 + i];
            v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
        }
        if (bias) {
            const int n = 4 * int(i % size_t(N4));
            v.x += float(__builtin_bit_cast(_Float16, bias[n]));
            v.y += float(__builtin_bit_cast(_Float16, bias[n + 1]));
            v.z += float(__builtin_bit_cast(_Float16, bias[n + 2]));
            v.w += float(__builtin_bit_cast(_Float16, bias[n + 3]));
        }
        const uint32_t lo = uint32_t(__builtin_bit_cast(uint16_t, (_Float16)v.x)) |
                            (uint32_t(__builtin_bit_cast(uint16_t, (_Float16)v.y)) << 16);
        const uint32_t hi = uint32_t(__builtin_bit_cast(uint16_t, (_Float16)v.z)) |
                            (uint32_t(__builtin_bit_cast(uint16_t, (_Float16)v.w)) << 16);
        y[i] = uint2{lo, hi};
    }
}

}  // namespace

namespace wqh {

// LDS bytes of the skinny kernel for M rows, slabs of KS channels, tpb
// tiles per block and GSL scale entries per row.
static size_t skinny_lds(int M, int KS, int tpb, int GSL) {
    const int MF = M > 16 ? 2 : 1;
    return size_t(M) * (size_t(KS) * 2 + 16) + 2 * kSkinnyWaves * 256 * 4 * MF + size_t(tpb) * M * 16 * 4 +
           size_t(tpb) * 16 * GSL * 3;
}

// Launch geometry of the skinny kernel.
struct SkinnyPlan {
    int blocks = 0, tpb = 0, nsl = 1;  // nsl: slabs of the split form (1: not split)
    SlabGeo geo{0, 0};
    size_t lds = 0;
    size_t part_bytes = 0;  // fp32 partials of the split form
};

// Plan for cus compute units and lds_max bytes of LDS per block; the split
// form is taken when K needs several slabs and ws_bytes holds its partials.
// false when no geometry fits.
static bool skinny_plan(int M, int N, int K, int gs, int cus, int lds_max, size_t ws_bytes, SkinnyPlan& p) {
    const int n_tiles = (N + 15) / 16;
    const int Kp = (K + 255) / 256 * 256;
    const int G = (K + gs - 1) / gs;
    // one slab: every block stages all of K once
    p.blocks = std::min(n_tiles, cus);
    p.tpb = (n_tiles + p.blocks - 1) / p.blocks;
    if (skinny_lds(M, Kp, p.tpb, G) <= size_t(lds_max)) {
        p.geo = SlabGeo{Kp, G};
        p.lds = skinny_lds(M, Kp, p.tpb, G);
        return true;
    }
    // K in slabs of KS channels (a multiple of 256); groups per slab at most
    // KS / gs + 1 (+ 1 for a group cut by the slab's start)
    auto slab_of = [&](int nslab) { return ((Kp / 256 + nslab - 1) / nslab) * 256; };
    // split form: nsl groups of bps blocks, group s taking slab s of every
    // tile, fewest slabs that fit
    for (int nslab = 2; nslab <= Kp / 256; ++nslab) {
        const int KS = slab_of(nslab);
        const int nsl = (K + KS - 1) / KS;  // slabs this slab size gives
        const int bps = std::max(1, cus / nsl);
        const int tpb = (n_tiles + bps - 1) / bps;
        const int GSL = std::min(G, KS / gs + 2);
        if (skinny_lds(M, KS, tpb, GSL) > size_t(lds_max)) continue;
        const size_t need = size_t(nsl) * size_t(M) * size_t(N) * 4;
        if (need > ws_bytes) break;
        p.blocks = bps * nsl;
        p.tpb = tpb;
        p.nsl = nsl;
        p.geo = SlabGeo{KS, GSL};
        p.lds = skinny_lds(M, KS, tpb, GSL);
        p.part_bytes = need;
        return true;
    }
    // without the workspace: each block walks the slabs in turn
    for (int nslab = 2; nslab <= Kp / 256; ++nslab) {
        const int KS = slab_of(nslab);
        const int GSL = std::min(G, KS / gs + 2);
        if (skinny_lds(M, KS, p.tpb, GSL) <= size_t(lds_max)) {
            p.geo = SlabGeo{KS, GSL};
            p.lds = skinny_lds(M, KS, p.tpb, GSL);
            return true;
        }
    }
    return false;
}

// Compute units and LDS bytes per block of the current device.
static void skinny_device(int& cus, int& lds_max) {
    int dev = 0;
    cus = 256;
    lds_max = 64 * 1024;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && v > 0)
            lds_max = v;
    }
}

// Workspace bytes the skinny kernel's split form may use for M x N x K on
// the current device, for any group size (group size 32 has the most scale
// entries per slab, so it needs the most slabs); 0 when K fits in one slab.
size_t skinny_workspace_bytes(int M, int N, int K) {
    if (M < 1 || M > kSkinnyMaxM || K < 256 || N < 1) return 0;
    int cus = 0, lds_max = 0;
    skinny_device(cus, lds_max);
    SkinnyPlan p;
    if (!skinny_plan(M, N, K, 32, cus, lds_max, ~size_t(0), p)) return 0;
    return p.part_bytes;
}

// Launch the skinny kernel; WQ_ERR_UNSUPPORTED when it does not apply
// (act-order, M outside 1..32, K below 256).  workspace (nullable,
// ws_bytes): room for the split form's fp32 partials.
wq_status skinny_gemv(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                      const int32_t* perm, uint16_t* y, int M, int N, int K, int bits, int gs, hipStream_t s,
                      const uint16_t* act_scale, const uint16_t* bias, void* workspace, size_t ws_bytes) {
    if (perm || M < 1 || M > kSkinnyMaxM || K < 256) return WQ_ERR_UNSUPPORTED;
    int cus = 0, lds_max = 0;
    skinny_device(cus, lds_max);
    SkinnyPlan plan;
    if (!skinny_plan(M, N, K, gs, cus, lds_max, workspace ? ws_bytes : 0, plan)) return WQ_ERR_UNSUPPORTED;
    const GroupDiv gd = group_magic(gs);
    const bool zsub = gs % 128 == 0;
    const bool split = plan.nsl > 1;
    const bool slabs = !split && plan.geo.KS < K;
    float* part = split ? static_cast<float*>(workspace) : nullptr;
    constexpr int D = WQ_SKINNY_D;
    auto go = [&](auto kern) {
        if (plan.lds > 64 * 1024)
            (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                      int(plan.lds));
        hipLaunchKernelGGL(kern, dim3(plan.blocks), dim3(64 * kSkinnyWaves), plan.lds, s, x, packed, scales, zeros, y,
                           M, N, K, gd, plan.tpb, plan.geo, act_scale, bias, part);
        wq_status st = launch_status();
        if (st != WQ_OK || !split) return st;
        const size_t MN = size_t(M) * N;
        // the workspace and y are 16-byte aligned (checked by the entry points)
        if (N % 4 == 0) {
            const int sb = int(std::min<size_t>((MN / 4 + 255) / 256, size_t(cus) * 8));
            hipLaunchKernelGGL(skinny_sum4_kernel, dim3(sb), dim3(256), 0, s, reinterpret_cast<const float4*>(part),
                               plan.nsl, M, N, bias, reinterpret_cast<uint2*>(y));
            return launch_status();
        }
        const int sb = int(std::min<size_t>((MN + 255) / 256, size_t(cus) * 8));
        hipLaunchKernelGGL(skinny_sum_kernel, dim3(sb), dim3(256), 0, s, part, plan.nsl, M, N, bias, y);
        return launch_status();
    };
    const bool ex = act_scale || bias;
    // pick the instantiation: bits, zero-points, fused epilogue, ZSUB, slab form
    auto pick = [&](auto bits_c) -> wq_status {
        constexpr int B = decltype(bits_c)::value;
        auto by_mf = [&](auto z_c, auto ex_c, auto zs_c, auto mf_c) -> wq_status {
            constexpr bool Z = decltype(z_c)::value, E = decltype(ex_c)::value, F = decltype(zs_c)::value;
            constexpr int MF = decltype(mf_c)::value;
            if (split) return go(skinny_kernel<B, D, Z, E, F, false, true, MF>);
            return slabs ? go(skinny_kernel<B, D, Z, E, F, true, false, MF>)
                         : go(skinny_kernel<B, D, Z, E, F, false, false, MF>);
        };
        auto by_slab = [&](auto z_c, auto ex_c, auto zs_c) -> wq_status {
            return M > 16 ? by_mf(z_c, ex_c, zs_c, std::integral_constant<int, 2>{})
                          : by_mf(z_c, ex_c, zs_c, std::integral_constant<int, 1>{});
        };
        auto by_zsub = [&](auto z_c, auto ex_c) -> wq_status {
            return zsub ? by_slab(z_c, ex_c, std::true_type{}) : by_slab(z_c, ex_c, std::false_type{});
        };
        auto by_ex = [&](auto z_c) -> wq_status {
            return ex ? by_zsub(z_c, std::true_type{}) : by_zsub(z_c, std::false_type{});
        };
        return zeros ? by_ex(std::true_type{}) : by_ex(std::false_type{});
    };
    switch (bits) {
        case 2: return pick(std::integral_constant<int, 2>{});
        case 3: return pick(std::integral_constant<int, 3>{});
        case 4: return pick(std::integral_constant<int, 4>{});
        default: return pick(std::integral_constant<int, 8>{});
    }
}

}  // namespace wqh
