// Decode GEMV: y[M][N] = x[M][K] . dequant(Wq)^T for small M (1..16).
//
// Single-token generation is memory-bound with almost no weight reuse, so
// the kernel is built to stream the packed weights once at full HBM rate
// ("AutoAWQ vs Unsloth", WQLinear_* paragraph on GEMV kernels for
// single-token generation; weights stay packed and are dequantized on the
// fly, "AutoAWQ vs The Stack v2", WQLinear_* paragraph).
//
// Work split: a 256-thread block owns 4*R consecutive output columns, one
// wavefront per R of them.  Lanes of a wavefront stride over the 32-code
// chunks of a weight row (consecutive lanes read consecutive 16-byte pieces:
// coalesced 128-bit loads), so every lane holds a K-slice partial sum per
// (column, activation row); the partials are reduced across the wavefront
// with butterfly shuffles at the end (split-K inside the wave, no atomics,
// deterministic).  Each lane keeps D chunk iterations of weight loads in
// flight (a rolling register pipeline), and the first ones are issued before
// the activations are staged so the two latencies overlap.  Activations are
// staged once per block in LDS, in the pair order the decoder produces,
// gathered through perm for act-order; long K runs in LDS-sized slabs.
#include <algorithm>

#include "wq_common.h"

namespace {

using namespace wq;

typedef int32_t i4 __attribute__((ext_vector_type(4)));

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

// Buffer resource over `bytes` bytes at p (word 3: raw 32-bit data format).
// An access through it adds a 32-bit lane offset to a wave-uniform base held
// in scalar registers, so a lane's address costs no 64-bit vector arithmetic;
// offsets at or past `bytes` read 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, int(bytes), 0x00020000);
}
constexpr int kBufNT = 2;  // cache policy: nontemporal

// One chunk (32 codes, 4 * BITS bytes) at byte offset off of a row resource.
// (Whole-vector bit casts only: a bit cast of one element of a vector
// reads element 0.)
template <int BITS>
__device__ __forceinline__ void load_chunk_buf(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t* w) {
    if constexpr (BITS == 4) {
        const u4 v = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kBufNT));
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else if constexpr (BITS == 8) {
        const u4 a = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kBufNT));
        const u4 b = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16u, 0, kBufNT));
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else if constexpr (BITS == 2) {
        typedef uint32_t u2 __attribute__((ext_vector_type(2)));
        const u2 v = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kBufNT));
        w[0] = v.x; w[1] = v.y;
    } else {
        const u4 v = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b96(rs, off, 0, kBufNT));
        w[0] = v.x; w[1] = v.y; w[2] = v.z;
    }
}

// Sum over the 64 lanes of a wavefront; the result is valid in every lane.
// Within each row of 16 lanes the partial sums move through DPP (quad
// permutes, then half-row and row mirrors); the four row sums are then read
// out with readlane and added in a fixed order (deterministic).
__device__ __forceinline__ float wave_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (r0 + r1) + (r2 + r3);
}

// Sum over the 64 lanes of a wavefront, valid in lane 63 only: DPP steps
// within each row of 16 lanes (quad permutes, half-row and row mirrors) leave
// the row sum in every lane of the row, then row broadcasts add row 0 into
// row 1, row 2 into row 3, and rows 0+1 into rows 2 and 3.  Six instructions,
// fixed order (deterministic).
__device__ __forceinline__ float wave_sum_last(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false));
    return v;
}

// Per-row pointers of the R output columns a wavefront owns.
template <int BITS, int R>
struct Rows {
    const uint32_t* w[R];
    const uint16_t* s[R];
    const uint8_t* z[R];
    bool ok[R];
};

// Raw operands of one chunk of each of the R rows: packed words, the group's
// zero-point byte and fp16 scale bits, and whether the chunk is real.
template <int BITS, int R>
struct Slot {
    uint32_t w[R][BITS];
    uint32_t z[R], s[R];
    bool ok[R];
};

// Issue the loads of one chunk (32 codes) of each of the R rows.  Loads are
// unconditional (an out-of-range row or chunk reads chunk 0 of row 0
// instead) and their results are only converted at use, so the compiler can
// keep all of them in flight.
template <int BITS, int R, bool HAS_Z>
__device__ __forceinline__ void issue_chunk(const Rows<BITS, R>& rows, GroupDiv gd, int cg, bool valid,
                                            Slot<BITS, R>& sl) {
    const int cgc = valid ? cg : 0;
    const int g = chunk_group(cgc, gd);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        sl.ok[r] = valid && rows.ok[r];
        load_chunk<BITS>(rows.w[r] + cgc * BITS, sl.w[r]);
        sl.s[r] = rows.s[r][g];
        if constexpr (HAS_Z)
            sl.z[r] = rows.z[r][g];
        else
            sl.z[r] = 1u << (BITS - 1);
    }
}

// Dequantize one chunk of each row and accumulate its dot product with the
// staged activations.  LDS holds, per activation row m, four planes (one per
// 8-code block of a chunk) of one 16-byte entry per chunk: the entry of chunk
// c, block b, row m is xs[(m * 4 + b) * CN + c], so the lanes of a wavefront
// (consecutive chunks) read consecutive 16-byte words.
template <int BITS, int MT, int R>
__device__ __forceinline__ void compute_chunk(const u4* xc, int CN, const Slot<BITS, R>& sl, float (&acc)[R][MT]) {
    uint32_t zz[R], ss[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        zz[r] = zero_pair(sl.z[r]);
        ss[r] = sl.ok[r] ? scale_pair(uint16_t(sl.s[r])) : 0u;  // zero weight outside the matrix
    }
    if constexpr (MT <= 4) {
        uint32_t xp[MT][16];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const u4 v = xc[(m * 4 + b) * CN];
                xp[m][4 * b] = v.x; xp[m][4 * b + 1] = v.y;
                xp[m][4 * b + 2] = v.z; xp[m][4 * b + 3] = v.w;
            }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            uint32_t h[16];
            decode_chunk<BITS>(sl.w[r], h);
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
        for (int r = 0; r < R; ++r) {
            uint32_t h[16];
            decode_chunk<BITS>(sl.w[r], h);
            h2 wv[16];
#pragma unroll
            for (int p = 0; p < 16; ++p) wv[p] = dequant_pair(h[p], zz[r], ss[r]);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const u4 v = xc[(m * 4 + b) * CN];
                    acc[r][m] = __builtin_amdgcn_fdot2(wv[4 * b], as_h2(v.x), acc[r][m], false);
                    acc[r][m] = __builtin_amdgcn_fdot2(wv[4 * b + 1], as_h2(v.y), acc[r][m], false);
                    acc[r][m] = __builtin_amdgcn_fdot2(wv[4 * b + 2], as_h2(v.z), acc[r][m], false);
                    acc[r][m] = __builtin_amdgcn_fdot2(wv[4 * b + 3], as_h2(v.w), acc[r][m], false);
                }
            }
        }
    }
}

// General kernel (any K, M <= 16): R rows per wavefront, one block per 4*R
// rows, activations staged in LDS-sized slabs, D chunk iterations of loads in
// flight per lane.  Dequantizes every weight to fp16 exactly as wq_dequant.
template <int BITS, int MT, int R, int D, bool HAS_Z>
__global__ void __launch_bounds__(256) gemv_slab_kernel(const uint16_t* __restrict__ x,
                                                   const uint32_t* __restrict__ packed,
                                                   const uint16_t* __restrict__ scales,
                                                   const uint8_t* __restrict__ zeros,
                                                   const int32_t* __restrict__ perm, uint16_t* __restrict__ y,
                                                   int M, int N, int K, int gs, GroupDiv gd, int slab) {
    extern __shared__ u4 xs[];  // [MT][4][CN] 16-byte entries, staging order
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n_base = (blockIdx.x * 4 + wave) * R;
    const int chunks = K / 32;
    const int G = K / gs;
    const int CN = slab / 32;
    const size_t row_words = (size_t)chunks * BITS;

    Rows<BITS, R> rows;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int n = n_base + r;
        rows.ok[r] = n < N;
        const int nn = rows.ok[r] ? n : 0;
        rows.w[r] = packed + (size_t)nn * row_words;
        rows.s[r] = scales + (size_t)nn * G;
        rows.z[r] = HAS_Z ? zeros + (size_t)nn * G : nullptr;
    }

    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;

    Slot<BITS, R> slot[D];

    for (int k0 = 0; k0 < K; k0 += slab) {
        const int kn = min(slab, K - k0);
        const int nb = kn / 8;
        const int cn = kn / 32;
        const int c0 = k0 / 32;
        const int J = (cn + 63) / 64;  // chunk iterations of this lane group

        // ---- weights first: the first D iterations' loads go out before the
        // activations are staged, so both latencies overlap
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int c = lane + 64 * d;
            issue_chunk<BITS, R, HAS_Z>(rows, gd, c0 + c, c < cn, slot[d]);
        }
        // ---- stage x[:, k0:k0+kn] in pair order (gathered through perm)
#pragma unroll
        for (int m = 0; m < MT; ++m)
        for (int bb = threadIdx.x; bb < nb; bb += 256) {
            u4 v = {0u, 0u, 0u, 0u};
            if (m < M) {
                const uint16_t* xr = x + (size_t)m * K;
                const int kk = k0 + 8 * bb;
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
            xs[(m * 4 + (bb & 3)) * CN + (bb >> 2)] = stage_block(v);
        }
        __syncthreads();

        // ---- rolling pipeline: compute iteration j from slot j % D, then
        // refill that slot with iteration j + D.  The body has no branches
        // (a chunk past the end computes with a zero scale from a clamped
        // LDS address, and refills past the end load a valid dummy chunk),
        // so each wait covers exactly the slot about to be used.
        for (int j0 = 0; j0 < J; j0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int c = lane + 64 * (j0 + d);
                compute_chunk<BITS, MT, R>(xs + min(c, cn - 1), CN, slot[d], acc);
                const int cx = c + 64 * D;
                issue_chunk<BITS, R, HAS_Z>(rows, gd, c0 + cx, cx < cn, slot[d]);
            }
        }
        __syncthreads();
    }

    // ---- split-K reduction across the wavefront, one fp16 rounding
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const float v = wave_sum(acc[r][m]);
            if (lane == 0 && rows.ok[r] && m < M)
                y[(size_t)m * N + n_base + r] = __builtin_bit_cast(uint16_t, (_Float16)v);
        }
    }
}


// Streaming-kernel decoder: the pair order of decode_chunk (pair i of a block
// holds codes i and i + 4) with cheaper 4-bit extraction.  Codes sitting at
// bits 4..7 of a 16-bit half are exposed where they are, under the exponent
// 0x5400 (fp16 64, whose mantissa step at bit 4 is exactly 1), giving 64 + q;
// codes at bits 0..3 get 0x6400 (1024 + q).  One shift by 8 brings the upper
// two nibbles of each half down, so a word costs 1 shift + 4 and-or instead of
// 3 + 4.  Pairs 0 and 2 of each block carry offset 1024, pairs 1 and 3 carry
// kOddBase<BITS> (64 for 4-bit; other widths use decode_chunk throughout).
template <int BITS>
constexpr float kOddBase = BITS == 4 ? 64.f : 1024.f;

template <int BITS>
__device__ __forceinline__ void decode_chunk_split(const uint32_t* w, uint32_t* h) {
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


// Streaming kernel (M <= 4 and the whole activation row fits in LDS).
//
// Persistent wavefronts: the grid is sized to the machine and wavefront w of
// the grid takes row groups w, w + W, w + 2W, ... (R output columns each).
// A lane walks the flat sequence of (row group, chunk iteration) pairs with a
// D-deep rolling register pipeline, so weight loads stay in flight across row
// group boundaries; the activations and their chunk sums are staged once per
// block.  Each slot holds CPL consecutive chunks (CPL * 32 codes, one group)
// of each of the R rows; consecutive lanes read consecutive CPL * 16 bytes.
//
// Arithmetic per slot (CPL chunks of one group) and activation row m: with
// h = B + q the exact fp16 integers of decode_chunk_split (B = 1024 on the
// even pairs of a block, kOddBase on the odd ones), A = sum_k x_k * h_k
// accumulated in fp32 by fp16-pair dot products, and Xe, Xo the sums of x
// over the even and the odd pairs,
//     sum_k x_k * (q_k - z) * s = s * (A - (1024 + z) * Xe - (kOddBase + z) * Xo)
// exactly in real arithmetic; the kernel evaluates the right-hand side in
// fp32 (one fused multiply-add each).  This skips the per-weight fp16
// subtract and multiply; the rounding differs from multiplying by fp16
// dequantized weights by about 2^-12 relative per weight, averaged over K.
// Wavefronts per block of the streaming kernel (the activations are staged
// once per block).
constexpr int kStreamWaves = 4;

template <int BITS, int R, int CPL>
struct WideSlot {
    uint32_t w[R][CPL][BITS];
    uint32_t z[R], s[R];
    bool ok[R];
};

template <int BITS, int MT, int R, int D, int CPL, bool HAS_Z, bool GATHER, bool SILU = false, bool EX = false,
          int WPB = kStreamWaves, bool EARLY = false>
__global__ void __launch_bounds__(64 * WPB) gemv_stream_kernel(const uint16_t* __restrict__ x,
                                                          const uint32_t* __restrict__ packed,
                                                          const uint16_t* __restrict__ scales,
                                                          const uint8_t* __restrict__ zeros,
                                                          const int32_t* __restrict__ perm,
                                                          uint16_t* __restrict__ y, int M, int N, int K,
                                                          GroupDiv gd, const uint16_t* __restrict__ act_scale,
                                                          const uint16_t* __restrict__ bias) {
    // EX: act_scale (nullable, fp16 [K]) divides the activations while they
    // are staged, x' = fp16(fp32(x) / fp32(s)) exactly as the separate
    // scaling kernel does; bias (nullable, fp16 [N]) is added to the fp32
    // sums before the output rounding (before the SiLU with SILU).
    // LDS: u4 xs[MT][4][CPL][CNP] (activation pairs), then float2 xsum[MT][CNP]
    // (per slot: sum of x over pairs 0 and 2 of every block, over pairs 1 and 3)
    extern __shared__ u4 xs[];
    const int CN = K / 32;       // chunks per row
    const int CNP = CN / CPL;    // slots per row
    float2* xsum = reinterpret_cast<float2*>(xs + MT * 4 * CN);
    // act-order: one activation row in its natural order, copied with
    // coalesced loads, then gathered through perm from LDS
    u4* xnat4 = xs + MT * 4 * CN + (MT * CNP + 1) / 2;
    const uint16_t* xnat = reinterpret_cast<const uint16_t*>(xnat4);
    const int lane = threadIdx.x & 63;
    // wave-uniform (readfirstlane): row-group positions and row addresses
    // live in scalar registers, lanes only add their chunk offset
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const int G = chunk_group(CN - 1, gd) + 1;
    const size_t row_words = (size_t)CN * BITS;
    // group of chunk c = floor((c + 0.5) / d), d chunks per group, by the
    // float reciprocal: exact while c < 2^21, since (c + 0.5) / d stays at
    // least 0.5 / d away from an integer, farther than the rounding error
    const float ginv = 1.0f / float(gd.chunks);
    // With SILU the N rows are a stacked gate (rows [0, N/2)) and up
    // (rows [N/2, N)) projection: row group g is the pair (g, g + N/2) and
    // the epilogue writes y[m][g] = silu(gate) * up, N/2 outputs per row.
    static_assert(!SILU || R == 2, "the fused gate/up epilogue pairs two rows");
    const int half = N / 2;
    const int n_groups = SILU ? half : (N + R - 1) / R;
    const int J = (CNP + 63) / 64;  // slot iterations per row group

    const int wg0 = blockIdx.x * WPB + wave;
    const int wstride = gridDim.x * WPB;
    const int my_groups = wg0 < n_groups ? (n_groups - wg0 + wstride - 1) / wstride : 0;
    const int T = my_groups * J;  // flat (row group, slot iteration) count of this wave

    // issue-side and compute-side positions in the flat sequence (the
    // compute side's row group is counted by c_k below)
    int i_rg = wg0, i_j = 0, c_j = 0;

    // Loads are issued unconditionally: a wait-count merge at a branch around
    // them would make every later wait drain all loads in flight.  The issue
    // position stops at the wavefront's last one (t = T - 1); the refills past
    // it read the first 16 bytes of the last row group's rows in every lane
    // (one cache line per row: re-reading the chunks loaded last could fetch
    // them from memory again, since those loads bypass the caches' retention),
    // and lanes past a row's end re-read its last chunk (same cache lines; no
    // address is shared by the whole grid).
    WideSlot<BITS, R, CPL> slot[D];
    auto issue = [&](WideSlot<BITS, R, CPL>& sl, int t) {
        const bool tv = t < T;  // wave-uniform
        const int cp = lane + 64 * i_j;
        const bool valid = tv && cp < CNP;
        const int cpc = tv ? (cp < CNP ? cp : CNP - 1) : 0;
        const int g = int(__builtin_fmaf(float(cpc * CPL), ginv, 0.5f * ginv));
        const uint32_t woff = uint32_t(cpc) * uint32_t(CPL * BITS * 4);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int n = SILU ? i_rg + r * half : i_rg * R + r;
            const bool nok = n < N;  // wave-uniform
            const int nn = __builtin_amdgcn_readfirstlane(nok ? n : N - 1);
            sl.ok[r] = valid && nok;
            // row bases wave-uniform (buffer resources in scalar registers),
            // lane offsets 32-bit
            const auto rw = buf_rsrc(reinterpret_cast<const char*>(packed) + size_t(nn) * row_words * 4,
                                     uint32_t(row_words * 4));
#pragma unroll
            for (int e = 0; e < CPL; ++e) load_chunk_buf<BITS>(rw, woff + uint32_t(e * BITS * 4), sl.w[r][e]);
            sl.s[r] = __builtin_amdgcn_raw_buffer_load_b16(
                buf_rsrc(reinterpret_cast<const char*>(scales) + size_t(nn) * G * 2, uint32_t(G * 2)), uint32_t(g) * 2u,
                0, 0);
            if constexpr (HAS_Z)
                sl.z[r] = __builtin_amdgcn_raw_buffer_load_b8(
                    buf_rsrc(reinterpret_cast<const char*>(zeros) + size_t(nn) * G, uint32_t(G)), uint32_t(g), 0, 0);
            else
                sl.z[r] = 1u << (BITS - 1);
        }
        if (t + 1 < T) {  // advance (no memory access on either path)
            const bool wrap = (i_j + 1 == J);
            i_j = wrap ? 0 : i_j + 1;
            i_rg += wrap ? wstride : 0;
        }
    };

    // ---- activation loads of the first staging pass go out before the
    // weight loads: vector-memory loads complete in issue order, so loads
    // issued after the weights could only be staged once every one of those
    // weights had arrived.  Issued first, they arrive after one cache round
    // trip and the staging overlaps the weights' HBM latency.
    auto load_block = [&](int m, int c, int b) -> u4 {
        const size_t xrow = (size_t)(m < M ? m : 0) * K;
        u4 v;
        if constexpr (GATHER) {
            const i4 p0 = *reinterpret_cast<const i4*>(perm + 32 * c + 8 * b);
            const i4 p1 = *reinterpret_cast<const i4*>(perm + 32 * c + 8 * b + 4);
            const uint16_t* xr = xnat;  // the row being staged
            v.x = uint32_t(xr[p0.x]) | (uint32_t(xr[p0.y]) << 16);
            v.y = uint32_t(xr[p0.z]) | (uint32_t(xr[p0.w]) << 16);
            v.z = uint32_t(xr[p1.x]) | (uint32_t(xr[p1.y]) << 16);
            v.w = uint32_t(xr[p1.z]) | (uint32_t(xr[p1.w]) << 16);
            (void)xrow;
        } else {
            v = *reinterpret_cast<const u4*>(x + xrow + 32 * c + 8 * b);
        }
        return v;  // rows m >= M are zeroed when staged
    };
    // the 8 scales of block b of chunk c (act-order: through perm)
    auto load_sblock = [&](int c, int b) -> u4 {
        if constexpr (GATHER) {
            uint32_t el[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) el[i] = act_scale[perm[32 * c + 8 * b + i]];
            return u4{el[0] | (el[1] << 16), el[2] | (el[3] << 16), el[4] | (el[5] << 16), el[6] | (el[7] << 16)};
        } else {
            return *reinterpret_cast<const u4*>(act_scale + 32 * c + 8 * b);
        }
    };
    // x' = fp16(x / s) for 8 activations
    auto scale_block = [&](u4 v, u4 t) -> u4 {
        const uint32_t in[4] = {v.x, v.y, v.z, v.w}, sv[4] = {t.x, t.y, t.z, t.w};
        uint32_t out[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = __fdiv_rn(float(__builtin_bit_cast(_Float16, uint16_t(in[i]))),
                                       float(__builtin_bit_cast(_Float16, uint16_t(sv[i]))));
            const float hi = __fdiv_rn(float(__builtin_bit_cast(_Float16, uint16_t(in[i] >> 16))),
                                       float(__builtin_bit_cast(_Float16, uint16_t(sv[i] >> 16))));
            out[i] = uint32_t(__builtin_bit_cast(uint16_t, (_Float16)lo)) |
                     (uint32_t(__builtin_bit_cast(uint16_t, (_Float16)hi)) << 16);
        }
        return u4{out[0], out[1], out[2], out[3]};
    };
    // sv: the slot's scales (EX with act_scale only)
    auto stage_slot = [&](int m, int cp, const u4 (&v)[CPL][4], const u4 (&sv)[CPL][4]) {
        float se = 0.f, so = 0.f;
        const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int e = 0; e < CPL; ++e)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                u4 raw = v[e][b];
                if constexpr (EX) {
                    if (act_scale) raw = scale_block(raw, sv[e][b]);
                }
                const u4 o = m < M ? stage_block(raw) : u4{0u, 0u, 0u, 0u};
                xs[((m * 4 + b) * CPL + e) * CNP + cp] = o;
                se = __builtin_amdgcn_fdot2(as_h2(o.x), one, se, false);
                so = __builtin_amdgcn_fdot2(as_h2(o.y), one, so, false);
                se = __builtin_amdgcn_fdot2(as_h2(o.z), one, se, false);
                so = __builtin_amdgcn_fdot2(as_h2(o.w), one, so, false);
            }
        xsum[m * CNP + cp] = make_float2(se, so);
    };
    // The first PRE passes (slot threadIdx.x + p * NT of every activation
    // row) are loaded up front, clamped to the last slot so that loads and
    // stores are unconditional; a pass that starts past the last slot is
    // skipped.  A gather through perm needs the perm values first, so with
    // act-order the weights still go out first.
    constexpr int NT = 64 * WPB;
    constexpr int PRE = (MT == 1 && !GATHER) ? 2 : 1;
    u4 xpre[PRE][MT][CPL][4];
    u4 spre[PRE][CPL][4];  // scales, loaded with the activations (EX)
    auto load_pre = [&]() {
#pragma unroll
        for (int p = 0; p < PRE; ++p) {
            if (p > 0 && p * NT >= CNP) break;  // wave-uniform
            const int cp = min(int(threadIdx.x) + p * NT, CNP - 1);
            if constexpr (EX) {
                if (act_scale) {
#pragma unroll
                    for (int e = 0; e < CPL; ++e)
#pragma unroll
                        for (int b = 0; b < 4; ++b) spre[p][e][b] = load_sblock(cp * CPL + e, b);
                }
            }
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int e = 0; e < CPL; ++e)
#pragma unroll
                    for (int b = 0; b < 4; ++b) xpre[p][m][e][b] = load_block(m, cp * CPL + e, b);
        }
    };
    if constexpr (!GATHER) load_pre();
#pragma unroll
    for (int d = 0; d < D; ++d) issue(slot[d], d);
    // keep the staging arithmetic below every weight load (it would wait for
    // the activations and hold back the loads scheduled after it)
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (GATHER) {
        // one activation row at a time: its natural order into LDS with
        // coalesced loads, then gathered through perm while staging
        const int K8 = K / 8;
        for (int m = 0; m < MT; ++m) {
            for (int i = threadIdx.x; i < K8; i += NT)
                xnat4[i] = m < M ? reinterpret_cast<const u4*>(x)[(size_t)m * K8 + i] : u4{0u, 0u, 0u, 0u};
            __syncthreads();
            for (int cp = threadIdx.x; cp < CNP; cp += NT) {
                u4 v[CPL][4], sv[CPL][4];
#pragma unroll
                for (int e = 0; e < CPL; ++e)
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        v[e][b] = load_block(m, cp * CPL + e, b);
                        if constexpr (EX) {
                            if (act_scale) sv[e][b] = load_sblock(cp * CPL + e, b);
                        }
                    }
                stage_slot(m, cp, v, sv);
            }
            __syncthreads();  // the row buffer is rewritten for the next row
        }
    } else {
        // ---- stage activations (pair order) and per-slot sums, once per
        // block; threads past the last slot rewrite it with the same values
#pragma unroll
        for (int p = 0; p < PRE; ++p) {
            if (p > 0 && p * NT >= CNP) break;
            const int cp = min(int(threadIdx.x) + p * NT, CNP - 1);
#pragma unroll
            for (int m = 0; m < MT; ++m) stage_slot(m, cp, xpre[p][m], spre[p]);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            for (int cp = threadIdx.x + PRE * NT; cp < CNP; cp += NT) {
                u4 v[CPL][4], sv[CPL][4];
#pragma unroll
                for (int e = 0; e < CPL; ++e)
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        v[e][b] = load_block(m, cp * CPL + e, b);
                        if constexpr (EX) {
                            if (act_scale) sv[e][b] = load_sblock(cp * CPL + e, b);
                        }
                    }
                stage_slot(m, cp, v, sv);
            }
        }
    }

    __syncthreads();

    float acc[R][MT], out[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = out[r][m] = 0.f;
    int c_k = 0;  // ordinal of the compute side's row group in this wavefront

    for (int t0 = 0; t0 < T; t0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int t = t0 + d;
            // ---- take iteration t out of slot d; EARLY refills the slot with
            // iteration t + D at once, so that the refill is in flight while
            // t is decoded and summed (otherwise after the sums)
            const WideSlot<BITS, R, CPL> cur = slot[d];
            if constexpr (EARLY) issue(slot[d], t + D);
            // ---- compute iteration t
            {
                const int cp = min(lane + 64 * c_j, CNP - 1);
                float2 X[MT];
#pragma unroll
                for (int m = 0; m < MT; ++m) X[m] = xsum[m * CNP + cp];
                float a[R][MT];
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int m = 0; m < MT; ++m) a[r][m] = 0.f;
#pragma unroll
                for (int e = 0; e < CPL; ++e) {
                    uint32_t xp[MT][16];
#pragma unroll
                    for (int m = 0; m < MT; ++m)
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            const u4 v = xs[((m * 4 + b) * CPL + e) * CNP + cp];
                            xp[m][4 * b] = v.x; xp[m][4 * b + 1] = v.y;
                            xp[m][4 * b + 2] = v.z; xp[m][4 * b + 3] = v.w;
                        }
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        uint32_t h[16];
                        decode_chunk_split<BITS>(cur.w[r][e], h);
#pragma unroll
                        for (int m = 0; m < MT; ++m)
#pragma unroll
                            for (int p = 0; p < 16; ++p)
                                a[r][m] = __builtin_amdgcn_fdot2(as_h2(h[p]), as_h2(xp[m][p]), a[r][m], false);
                    }
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float sf =
                        cur.ok[r] ? float(__builtin_bit_cast(_Float16, uint16_t(cur.s[r]))) : 0.f;
                    const float zf = float(cur.z[r]);
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        float t = __builtin_fmaf(-(1024.f + zf), X[m].x, a[r][m]);
                        t = __builtin_fmaf(-(kOddBase<BITS> + zf), X[m].y, t);
                        acc[r][m] = __builtin_fmaf(sf, t, acc[r][m]);
                    }
                }
            }
            // ---- end of a row group: reduce across the wavefront and keep
            // the sums in the `out` registers of lane k * R + r, k the group's
            // ordinal in this wavefront (no store inside the loop: a store on
            // some paths would also make the wait counts conservative)
            if (c_j == J - 1 && t < T) {
                const int k = c_k * (SILU ? 1 : R);
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        const float v = __builtin_bit_cast(
                            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wave_sum_last(acc[r][m])), 63));
                        acc[r][m] = 0.f;
                        out[r][m] = lane == k + (SILU ? 0 : r) ? v : out[r][m];
                    }
                ++c_k;
            }
            c_j = c_j + 1 == J ? 0 : c_j + 1;
            if constexpr (!EARLY) issue(slot[d], t + D);
        }
    }
    // ---- outputs: lane k * R + r holds row R * (wg0 + k * wstride) + r (with
    // SILU: lane k holds gate/up pair wg0 + k * wstride)
    const int k = SILU ? lane : lane / R;
    if (k < my_groups) {
        const int rg = wg0 + k * wstride;
        if constexpr (SILU) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                float g = out[0][m], u = out[1][m];
                if constexpr (EX) {
                    if (bias) {
                        g += float(__builtin_bit_cast(_Float16, bias[rg]));
                        u += float(__builtin_bit_cast(_Float16, bias[rg + half]));
                    }
                }
                const float v = g / (1.0f + expf(-g)) * u;
                if (m < M) y[(size_t)m * half + rg] = __builtin_bit_cast(uint16_t, (_Float16)v);
            }
        } else {
            const int r = lane % R;
            const int n = rg * R + r;
            if (n < N) {
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    float v = 0.f;
#pragma unroll
                    for (int q = 0; q < R; ++q) v = q == r ? out[q][m] : v;
                    if constexpr (EX) {
                        if (bias) v += float(__builtin_bit_cast(_Float16, bias[n]));
                    }
                    if (m < M) y[(size_t)m * N + n] = __builtin_bit_cast(uint16_t, (_Float16)v);
                }
            }
        }
    }
}

constexpr size_t kLdsBudget = 64 * 1024;

template <int BITS, int MT, int R, int D>
wq_status launch_cfg(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                     const int32_t* perm, uint16_t* y, int M, int N, int K, int gs, hipStream_t s) {
    int slab = int(kLdsBudget / (size_t(MT) * 2));
    slab = (slab / 32) * 32;
    if (slab > K) slab = K;
    const size_t lds = size_t(MT) * slab * 2;
    const int blocks = (N + 4 * R - 1) / (4 * R);
    const GroupDiv gd = wqh::group_magic(gs);
    if (zeros)
        hipLaunchKernelGGL((gemv_slab_kernel<BITS, MT, R, D, true>), dim3(blocks), dim3(256), lds, s, x, packed,
                           scales, zeros, perm, y, M, N, K, gs, gd, slab);
    else
        hipLaunchKernelGGL((gemv_slab_kernel<BITS, MT, R, D, false>), dim3(blocks), dim3(256), lds, s, x, packed,
                           scales, zeros, perm, y, M, N, K, gs, gd, slab);
    return wqh::launch_status();
}

// LDS bytes the streaming kernel stages: fp16 activations plus one fp32 sum
// per slot, per activation row.
inline size_t stream_lds_bytes(int MT, int K, int cpl, bool gather = false) {
    const size_t sums = (size_t(MT) * (K / (32 * cpl)) + 1) / 2 * 16;
    return size_t(MT) * K * 2 + sums + (gather ? size_t(K) * 2 : 0);
}

// Launch shape of the streaming kernel: resident blocks per CU of the
// default shape (R = 2 rows per wavefront, D = 2 slots, refill after the
// sums).
#ifndef WQ_GEMV_BPC
#define WQ_GEMV_BPC 3
#endif
#ifndef WQ_GEMV_CPL
#define WQ_GEMV_CPL 1
#endif
constexpr int kStreamBlocksPerCU = WQ_GEMV_BPC;

// Compute units and LDS bytes per compute unit of the current device
// (MI355X values when the query fails).
struct CuLimits {
    int cus = 256;
    size_t lds = 160 * 1024;
};
inline CuLimits cu_limits() {
    CuLimits c;
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess) return c;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) c.cus = v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) == hipSuccess && v > 0)
        c.lds = size_t(v);
    return c;
}

template <int BITS, int MT, int R, int D, int CPL, bool SILU = false, bool EX = false, int WPB = kStreamWaves,
          bool EARLY = false>
wq_status launch_stream(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                        const int32_t* perm, uint16_t* y, int M, int N, int K, int gs, hipStream_t s,
                        const uint16_t* act_scale = nullptr, const uint16_t* bias = nullptr,
                        int bpc = kStreamBlocksPerCU) {
    const CuLimits cl = cu_limits();
    const size_t lds = stream_lds_bytes(MT, K, CPL, perm != nullptr);
    // One round of resident blocks (more wavefronts in flight beat equal
    // shares: measured): at most bpc per CU and no more than the CU's LDS
    // holds (a block past those would wait for a whole earlier block),
    // unless a wavefront would take more than 64 / R row groups (it keeps
    // one finished output per lane until its end).
    const int per_cu = std::max(1, std::min(bpc, int(cl.lds / lds)));
    const int n_groups = SILU ? N / 2 : (N + R - 1) / R;
    const int max_per_wave = SILU ? 64 : 64 / R;
    int blocks = (n_groups + WPB - 1) / WPB;
    if (blocks > cl.cus * per_cu) blocks = cl.cus * per_cu;
    blocks = std::max(blocks, (n_groups + WPB * max_per_wave - 1) / (WPB * max_per_wave));
    const GroupDiv gd = wqh::group_magic(gs);
    if (zeros && perm)
        hipLaunchKernelGGL((gemv_stream_kernel<BITS, MT, R, D, CPL, true, true, SILU, EX, WPB, EARLY>), dim3(blocks),
                           dim3(64 * WPB), lds, s, x, packed, scales, zeros, perm, y, M, N, K, gd, act_scale, bias);
    else if (zeros)
        hipLaunchKernelGGL((gemv_stream_kernel<BITS, MT, R, D, CPL, true, false, SILU, EX, WPB, EARLY>), dim3(blocks),
                           dim3(64 * WPB), lds, s, x, packed, scales, zeros, perm, y, M, N, K, gd, act_scale, bias);
    else if (perm)
        hipLaunchKernelGGL((gemv_stream_kernel<BITS, MT, R, D, CPL, false, true, SILU, EX, WPB, EARLY>), dim3(blocks),
                           dim3(64 * WPB), lds, s, x, packed, scales, zeros, perm, y, M, N, K, gd, act_scale, bias);
    else
        hipLaunchKernelGGL((gemv_stream_kernel<BITS, MT, R, D, CPL, false, false, SILU, EX, WPB, EARLY>), dim3(blocks),
                           dim3(64 * WPB), lds, s, x, packed, scales, zeros, perm, y, M, N, K, gd, act_scale, bias);
    return wqh::launch_status();
}

// Launch shape by layer (measured on the decode and 70B shapes at M = 1):
// - K <= 4096 (at most two slot iterations per row group): one slot per
//   wavefront refilled before its sums, four blocks per CU;
// - activations too long for three blocks per CU in LDS (K above about 24K):
//   8-wavefront blocks, two per CU, one slot refilled before its sums, so the
//   CU keeps 16 wavefronts;
// - otherwise (and for M > 1) two slots refilled after the sums, three blocks
//   per CU.
template <int BITS, int MT, int CPL>
wq_status launch_stream_cpl(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                            const uint8_t* zeros, const int32_t* perm, uint16_t* y, int M, int N, int K, int gs,
                            hipStream_t s) {
    if constexpr (MT == 1) {
        const size_t lds = stream_lds_bytes(MT, K, CPL, perm != nullptr);
        if (3 * lds > cu_limits().lds)
            return launch_stream<BITS, MT, 2, 1, CPL, false, false, 8, true>(x, packed, scales, zeros, perm, y, M, N,
                                                                             K, gs, s, nullptr, nullptr, 2);
        if (K <= 4096)
            return launch_stream<BITS, MT, 2, 1, CPL, false, false, kStreamWaves, true>(
                x, packed, scales, zeros, perm, y, M, N, K, gs, s, nullptr, nullptr, 4);
    }
    return launch_stream<BITS, MT, 2, 2, CPL>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
}

// Streaming kernel when the activations fit in LDS and M <= 4 (two chunks
// per slot when every pair of chunks shares a group); otherwise the slab
// kernel.
template <int BITS, int MT>
wq_status launch_mt(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                    const int32_t* perm, uint16_t* y, int M, int N, int K, int gs, hipStream_t s) {
    if constexpr (MT > 4) {
        return launch_cfg<BITS, MT, 1, 2>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
    } else {
        constexpr int CPL = WQ_GEMV_CPL;
        if (CPL > 1 && K % (32 * CPL) == 0 && gs % (32 * CPL) == 0 &&
            stream_lds_bytes(MT, K, CPL, perm != nullptr) <= kLdsBudget)
            return launch_stream_cpl<BITS, MT, CPL>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
        if (stream_lds_bytes(MT, K, 1, perm != nullptr) <= kLdsBudget)
            return launch_stream_cpl<BITS, MT, 1>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
        if (N < 8192) return launch_cfg<BITS, MT, 1, 2>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
        if (N < 16384) return launch_cfg<BITS, MT, 2, 2>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
        return launch_cfg<BITS, MT, 4, 2>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
    }
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

// Fused gate/up projection with SiLU: the streaming kernel with the paired
// rows (g, g + N/2) and the silu(gate) * up epilogue.
template <int BITS>
wq_status launch_silu(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                      const int32_t* perm, uint16_t* y, int M, int N, int K, int gs, hipStream_t s) {
    const int MT = M <= 1 ? 1 : M <= 2 ? 2 : 4;
    if (stream_lds_bytes(MT, K, 1, perm != nullptr) > kLdsBudget) return WQ_ERR_UNSUPPORTED;
    if (M <= 1) return launch_stream<BITS, 1, 2, 2, 1, true>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
    if (M <= 2) return launch_stream<BITS, 2, 2, 2, 1, true>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
    return launch_stream<BITS, 4, 2, 2, 1, true>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
}

// The streaming kernel with the activation scaling and bias epilogue (M <= 4,
// activations within the LDS budget).
template <int BITS>
wq_status launch_ex(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                    const int32_t* perm, const uint16_t* act_scale, const uint16_t* bias, uint16_t* y, int M, int N,
                    int K, int gs, bool silu, hipStream_t s) {
    const int MT = M <= 1 ? 1 : M <= 2 ? 2 : 4;
    if (stream_lds_bytes(MT, K, 1, perm != nullptr) > kLdsBudget) return WQ_ERR_UNSUPPORTED;
    if (silu) {
        if (M <= 1) return launch_stream<BITS, 1, 2, 2, 1, true, true>(x, packed, scales, zeros, perm, y, M, N, K, gs, s, act_scale, bias);
        if (M <= 2) return launch_stream<BITS, 2, 2, 2, 1, true, true>(x, packed, scales, zeros, perm, y, M, N, K, gs, s, act_scale, bias);
        return launch_stream<BITS, 4, 2, 2, 1, true, true>(x, packed, scales, zeros, perm, y, M, N, K, gs, s, act_scale, bias);
    }
    constexpr int R = 2, D = 2;
    if (M <= 1) return launch_stream<BITS, 1, R, D, 1, false, true>(x, packed, scales, zeros, perm, y, M, N, K, gs, s, act_scale, bias);
    if (M <= 2) return launch_stream<BITS, 2, R, D, 1, false, true>(x, packed, scales, zeros, perm, y, M, N, K, gs, s, act_scale, bias);
    return launch_stream<BITS, 4, R, D, 1, false, true>(x, packed, scales, zeros, perm, y, M, N, K, gs, s, act_scale, bias);
}

}  // namespace

#ifndef WQ_SKINNY_MIN_M
#define WQ_SKINNY_MIN_M 2
#endif

namespace wqh {
wq_status skinny_gemv(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                      const int32_t* perm, uint16_t* y, int M, int N, int K, int bits, int gs, hipStream_t s,
                      const uint16_t* act_scale, const uint16_t* bias, void* workspace, size_t ws_bytes);
wq_status check_linear_args(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint16_t* y,
                            int M, int N, int K, int bits, int group_size, int* gs_out);
}

extern "C" wq_status wq_gemv(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                             const int32_t* perm, uint16_t* y, int32_t M, int32_t N, int32_t K, int32_t bits,
                             int32_t group_size, void* workspace, size_t workspace_bytes, void* stream) {
    int gs = 0;
    const wq_status st = wqh::check_linear_args(x, packed, scales, y, M, N, K, bits, group_size, &gs);
    if (st != WQ_OK) return st;
    if (perm && !wqh::aligned16(perm)) return WQ_ERR_ARG;  // read 16 bytes at a time
    if (workspace && !wqh::aligned16(workspace)) return WQ_ERR_ARG;
    if (M > 32) return WQ_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return WQ_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (M >= WQ_SKINNY_MIN_M) {
        const wq_status st2 =
            wqh::skinny_gemv(x, packed, scales, zeros, perm, y, M, N, K, bits, gs, s, nullptr, nullptr, workspace,
                             workspace ? workspace_bytes : 0);
        // the vector-ALU kernels below take at most 16 rows
        if (st2 != WQ_ERR_UNSUPPORTED || M > 16) return st2;
    }
    switch (bits) {
        case 2: return launch_bits<2>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
        case 3: return launch_bits<3>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
        case 4: return launch_bits<4>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
        default: return launch_bits<8>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
    }
}

extern "C" wq_status wq_gemv_silu_mul(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                                      const uint8_t* zeros, const int32_t* perm, uint16_t* y, int32_t M, int32_t N,
                                      int32_t K, int32_t bits, int32_t group_size, void* stream) {
    int gs = 0;
    const wq_status st = wqh::check_linear_args(x, packed, scales, y, M, N, K, bits, group_size, &gs);
    if (st != WQ_OK) return st;
    if (perm && !wqh::aligned16(perm)) return WQ_ERR_ARG;  // read 16 bytes at a time
    if (N % 2) return WQ_ERR_ARG;
    if (M > 4) return WQ_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return WQ_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (bits) {
        case 2: return launch_silu<2>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
        case 3: return launch_silu<3>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
        case 4: return launch_silu<4>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
        default: return launch_silu<8>(x, packed, scales, zeros, perm, y, M, N, K, gs, s);
    }
}

extern "C" wq_status wq_gemv_ex(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                                const uint8_t* zeros, const int32_t* perm, const uint16_t* act_scale,
                                const uint16_t* bias, uint16_t* y, int32_t M, int32_t N, int32_t K, int32_t bits,
                                int32_t group_size, int32_t silu, void* stream) {
    int gs = 0;
    const wq_status st = wqh::check_linear_args(x, packed, scales, y, M, N, K, bits, group_size, &gs);
    if (st != WQ_OK) return st;
    if (perm && !wqh::aligned16(perm)) return WQ_ERR_ARG;  // read 16 bytes at a time
    if (silu && N % 2) return WQ_ERR_ARG;
    if (act_scale && !wqh::aligned16(act_scale)) return WQ_ERR_ARG;
    const bool sl = silu != 0;
    if (M > 32 || (sl && M > 4)) return WQ_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return WQ_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!sl && M >= WQ_SKINNY_MIN_M) {  // the kernel wq_gemv uses for this M
        const wq_status st2 =
            wqh::skinny_gemv(x, packed, scales, zeros, perm, y, M, N, K, bits, gs, s, act_scale, bias, nullptr, 0);
        if (st2 != WQ_ERR_UNSUPPORTED || M > 4) return st2;
    }
    switch (bits) {
        case 2: return launch_ex<2>(x, packed, scales, zeros, perm, act_scale, bias, y, M, N, K, gs, sl, s);
        case 3: return launch_ex<3>(x, packed, scales, zeros, perm, act_scale, bias, y, M, N, K, gs, sl, s);
        case 4: return launch_ex<4>(x, packed, scales, zeros, perm, act_scale, bias, y, M, N, K, gs, sl, s);
        default: return launch_ex<8>(x, packed, scales, zeros, perm, act_scale, bias, y, M, N, K, gs, sl, s);
    }
}
