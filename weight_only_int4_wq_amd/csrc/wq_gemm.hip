// Prefill GEMM: y[M][N] = x[M][K] . dequant(Wq)^T on fp16 matrix cores.
//
// Batched inference is the one place the layer is a dense contraction, so
// the weight tiles are dequantized to fp16 and fed to MFMA instructions
// with fp32 accumulators ("AutoAWQ vs The Stack v2" and "AutoAWQ vs Unsloth",
// WQLinear_* paragraphs: a GEMM kernel for batches, dequantizing on the fly
// without materializing fp16 weights in memory).
//
// Tiling: a 256-thread block owns a BM x BN output tile, split over a
// WAVES_M x WAVES_N grid of wavefronts; K advances in stages of BK = 128.
//  - A (activations): each stage's BM x 128 fp16 tile is copied from global
//    memory straight into LDS by global_load_lds_dwordx4 (no registers),
//    double buffered, one barrier per stage: the copy of stage s + 1 is in
//    flight while stage s is multiplied.  In LDS a row is 16 units of 16
//    bytes and unit u of row r is stored at position u ^ (r mod 16), so the
//    sixteen rows a fragment read touches fall on distinct banks.
//  - B (weights): for v_mfma_f32_16x16x32_f16 a lane holds 8 consecutive k
//    of one output column, which is exactly one 8-code block of the packed
//    row.  Each lane therefore loads its own packed chunk (32 codes: 4
//    blocks = the 4 MFMA k-steps of the stage), dequantizes it in registers
//    with the exact (q - z) * s arithmetic, and uses the result directly as B
//    fragments: the dequantized tile lives in registers rather than LDS.
//    Lane group g (lanes 16g..16g+15) takes chunk g of the stage, and the A
//    fragments are read with the same k mapping, so the k sum is unchanged.
//  - Tiles are dealt to the XCDs in contiguous ranges and ordered in strips
//    of 4 M-tiles, so the blocks resident on one XCD cover a compact
//    rectangle of the output and reuse activations and weights from its L2.
#include <algorithm>

#include <type_traits>

#include "wq_gemm_common.h"

namespace {

using namespace wq;

template <int BITS, int BM, int BN, int WAVES_M, int NST, bool HAS_Z, bool PART>
__global__ void __launch_bounds__(256) gemm_kernel(const uint16_t* __restrict__ x,
                                                   const uint32_t* __restrict__ packed,
                                                   const uint16_t* __restrict__ scales,
                                                   const uint8_t* __restrict__ zeros, uint16_t* __restrict__ y,
                                                   int M, int N, int K, GroupDiv gd, int m_tiles, int n_tiles,
                                                   int tiles, int sps, float* __restrict__ part) {
    constexpr int GM = 4;  // M-tiles per strip of the tile order
    constexpr int WAVES_N = 4 / WAVES_M;
    constexpr int BK = 128;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int ROW_BYTES = BK * 2;          // 16 units of 16 bytes
    constexpr int A_INSTR = BM / 16;           // 1 KB copies per wavefront per stage
    static_assert(TM >= 1 && TN >= 1 && A_INSTR >= 1, "tile shape");
    // NST activation buffers and weight register sets: stage s lives in
    // buffer and set s % NST, and its loads are issued NST - 1 stages ahead
    // (indices are compile-time after unrolling, so the compiler can tell a
    // copy into one buffer from reads of another).
    constexpr int AHEAD = NST - 1;
    static_assert(NST >= 3 && NST <= 8, "pipeline depth");
    __shared__ __attribute__((aligned(1024))) uint8_t As[NST][BM * ROW_BYTES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int li = lane & 15, lg = lane >> 4;
    int m_t, n_t;
    tile_coords<GM>(blockIdx.x, tiles, m_tiles, n_tiles, m_t, n_t);
    const int m0 = m_t * BM, n0 = n_t * BN;
    const int chunks = K / 32;
    const int G = chunk_group(chunks - 1, gd) + 1;
    const size_t row_words = (size_t)chunks * BITS;
    const int n_lane0 = n0 + wn * WN + li;
    const int stages = (K + BK - 1) / BK;
    // split-K: this block's range of stages (blockIdx.y), all of K unsplit
    const int st_begin = blockIdx.y * sps;
    const int st_end = min(st_begin + sps, stages);

    // ---- A: this wavefront's share of a stage, global -> LDS directly.
    // Copy i of the wavefront fills units [64 * (wave * A_INSTR + i), +64):
    // lane l writes unit 64 * (...) + l, i.e. row (unit / 16), position l % 16,
    // which holds logical unit (l % 16) ^ (row % 16).  Rows past M and
    // columns past K read valid in-range data instead (their products only
    // reach output rows that are not stored, or meet zero weights).
    auto issue_a = [&](uint8_t* buf, int k0) {
#pragma unroll
        for (int i = 0; i < A_INSTR; ++i) {
            const int unit0 = (wave * A_INSTR + i) * 64;
            const int row = (unit0 >> 4) + (lane >> 4);
            const int u = (lane & 15) ^ (row & 15);
            const int gm = min(m0 + row, M - 1);
            const int gk = k0 + 8 * u;
            const uint16_t* src = x + (size_t)gm * K + (gk < K ? gk : 0);
            __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)(buf + unit0 * 16), 16, 0, 0);
        }
    };

    // ---- B: raw packed chunk, zero byte and scale bits of each of the TN
    // columns this lane feeds (zero scale outside the matrix).  Two register
    // sets alternate between stages, so the next stage's loads never land in
    // registers the current stage still reads.
    struct BRegs {
        uint32_t w[TN][BITS], z[TN], s[TN];
        bool ok[TN];
    };
    auto issue_b = [&](BRegs& b, int k0) {
        const int cg = k0 / 32 + lg;
        const bool kval = cg < chunks;
        const int cgc = kval ? cg : 0;
        const int g = chunk_group(cgc, gd);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = n_lane0 + j * 16;
            const bool ok = kval && n < N;
            const size_t nn = ok ? size_t(n) : 0;
            b.ok[j] = ok;
            load_chunk_b<BITS>(packed + nn * row_words + (size_t)cgc * BITS, b.w[j]);
            b.s[j] = scales[nn * G + g];
            if constexpr (HAS_Z)
                b.z[j] = zeros[nn * G + g];
            else
                b.z[j] = 1u << (BITS - 1);
        }
    };

    f4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

    // Per-lane vector-memory instructions of one issue_b (at least: a
    // 3-bit chunk may be fetched by one dwordx3 load).
    constexpr int B_OPS = TN * ((BITS == 8 ? 2 : 1) + 1 + (HAS_Z ? 1 : 0));
    static_assert((AHEAD - 1) * (B_OPS + A_INSTR) < 64, "vmcnt range");

    // One stage: wait for its data, start the loads AHEAD stages ahead,
    // multiply.  Stage s's weights and activations were issued at the top of
    // stage s - AHEAD (in that order), so only the loads issued at the tops
    // of the AHEAD - 1 stages since may still be outstanding.  Without ISSUE
    // (the stages after the unrolled loop, whose loads would all lie past
    // the range) nothing is loaded and the barrier waits for every load in
    // flight: register loads that are never read would be dropped by the
    // compiler, and the barrier's count would then let this stage's own
    // activation copies still be in flight.
    auto stage = [&](auto issue_c, int st, const BRegs& cur, BRegs& nxt, uint8_t* Ab, uint8_t* An) {
        constexpr bool ISSUE = decltype(issue_c)::value;
        copy_barrier<ISSUE ? (AHEAD - 1) * (B_OPS + A_INSTR) : 0>();
        if constexpr (ISSUE) {
            issue_b(nxt, (st + AHEAD) * BK);
            __builtin_amdgcn_sched_barrier(0);
            issue_a(An, (st + AHEAD) * BK);
            __builtin_amdgcn_sched_barrier(0);
        }

        uint32_t zz[TN], ss[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            zz[j] = zero_pair(cur.z[j]);
            ss[j] = cur.ok[j] ? scale_pair(uint16_t(cur.s[j])) : 0u;
        }
        // Software pipeline over the 4 k-steps: the A fragments (LDS reads)
        // and B fragments (decode + dequantize) of step s + 1 are produced
        // while step s's MFMAs run.
        auto load_a = [&](int s, h8 (&af)[TM]) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wm * WM + i * 16 + li;
                const int u = (4 * lg + s) ^ (row & 15);
                af[i] = *reinterpret_cast<const h8*>(Ab + row * ROW_BYTES + u * 16);
            }
        };
        auto make_b = [&](int s, h8 (&bf)[TN]) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                uint32_t hq[4], f[4];
                decode_block_nat<BITS>(cur.w[j], s, hq);
#pragma unroll
                for (int i = 0; i < 4; ++i) f[i] = as_u32(dequant_pair(hq[i], zz[j], ss[j]));
                const u4 fv = {f[0], f[1], f[2], f[3]};
                bf[j] = __builtin_bit_cast(h8, fv);
            }
        };
        h8 af[2][TM], bf[2][TN];
        load_a(0, af[0]);
        make_b(0, bf[0]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int c = s & 1;
            if (s < 3) {
                load_a(s + 1, af[c ^ 1]);
                make_b(s + 1, bf[c ^ 1]);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[c][i], bf[c][j], acc[i][j], 0, 0, 0);
        }
    };

    // Stage st_begin + i uses weight register set i % NST and activation
    // buffer i % NST (both addressed at compile time: the loop is unrolled
    // by NST).  The prologue issues the first AHEAD stages; past the range
    // the loads reread in-range data (or chunk 0 past K, with zero weight)
    // into buffers and sets that are not read again.
    BRegs b[NST];
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) {
        issue_b(b[i], (st_begin + i) * BK);
        __builtin_amdgcn_sched_barrier(0);
        issue_a(As[i], (st_begin + i) * BK);
        __builtin_amdgcn_sched_barrier(0);
    }
    int st = st_begin;
    const std::true_type loads;
    const std::false_type no_loads;
    for (; st + NST <= st_end; st += NST) {
#pragma unroll
        for (int i = 0; i < NST; ++i)
            stage(loads, st + i, b[i], b[(i + AHEAD) % NST], As[i], As[(i + AHEAD) % NST]);
    }
#pragma unroll
    for (int i = 0; i < NST - 1; ++i)
        if (st + i < st_end) stage(no_loads, st + i, b[i], b[(i + AHEAD) % NST], As[i], As[(i + AHEAD) % NST]);

    // no copy may still be writing this block's LDS when it exits
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

    // ---- epilogue: lane holds rows 4*lg + r of column li of each 16x16
    // tile; fp16 y, or this range's fp32 partial
    float* pr = PART ? part + (size_t)blockIdx.y * M * N : nullptr;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = n0 + wn * WN + j * 16 + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm * WM + i * 16 + 4 * lg + r;
                if (row < M && col < N) {
                    if constexpr (PART)
                        pr[(size_t)row * N + col] = acc[i][j][r];
                    else
                        y[(size_t)row * N + col] = __builtin_bit_cast(uint16_t, (_Float16)acc[i][j][r]);
                }
            }
        }
}

// y = fp16 of the sum of the split-K partials, ranges added in order.
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ part, int splits, long long mn,
                                                            uint16_t* __restrict__ y) {
    for (long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x; t < mn;
         t += (long long)gridDim.x * blockDim.x) {
        float v = part[t];
        for (int r = 1; r < splits; ++r) v += part[t + r * mn];
        y[t] = __builtin_bit_cast(uint16_t, (_Float16)v);
    }
}

// The same for M*N a multiple of 4: four outputs per thread, 16-byte loads
// of each range and one 8-byte store (the same additions in the same order).
__global__ void __launch_bounds__(256) splitk_reduce4_kernel(const float4* __restrict__ part, int splits,
                                                             long long mn4, uint2* __restrict__ y) {
    for (long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x; t < mn4;
         t += (long long)gridDim.x * blockDim.x) {
        float4 v = part[t];
        for (int r = 1; r < splits; ++r) {
            const float4 w = part[t + r * mn4];
            v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
        }
        const uint32_t lo = uint32_t(__builtin_bit_cast(uint16_t, (_Float16)v.x)) |
                            (uint32_t(__builtin_bit_cast(uint16_t, (_Float16)v.y)) << 16);
        const uint32_t hi = uint32_t(__builtin_bit_cast(uint16_t, (_Float16)v.z)) |
                            (uint32_t(__builtin_bit_cast(uint16_t, (_Float16)v.w)) << 16);
        y[t] = uint2{lo, hi};
    }
}

// x_out[m][k'] = x[m][perm[k']]: activations in packed column order.  A
// block takes whole rows: it copies the row into LDS with 16-byte loads, then
// every thread gathers 8 consecutive outputs through perm from LDS and writes
// them with one 16-byte store (K a multiple of 8, rows 16-byte aligned).
// (Staging up to four rows per block, so that one read of perm serves them
// all, measured the same at M = 256 and 2048.)
__global__ void __launch_bounds__(256) gather_rows_kernel(const uint16_t* __restrict__ x,
                                                          const int32_t* __restrict__ perm, int M, int K,
                                                          uint16_t* __restrict__ x_out) {
    typedef int32_t i4 __attribute__((ext_vector_type(4)));
    extern __shared__ u4 row4[];
    const uint16_t* row = reinterpret_cast<const uint16_t*>(row4);
    const int K8 = K / 8;
    for (int m = blockIdx.x; m < M; m += gridDim.x) {
        const u4* src = reinterpret_cast<const u4*>(x + size_t(m) * K);
        for (int i = threadIdx.x; i < K8; i += blockDim.x) row4[i] = src[i];
        __syncthreads();
        u4* dst = reinterpret_cast<u4*>(x_out + size_t(m) * K);
        for (int i = threadIdx.x; i < K8; i += blockDim.x) {
            const i4 p0 = reinterpret_cast<const i4*>(perm)[2 * i];
            const i4 p1 = reinterpret_cast<const i4*>(perm)[2 * i + 1];
            u4 o;
            o.x = uint32_t(row[p0.x]) | (uint32_t(row[p0.y]) << 16);
            o.y = uint32_t(row[p0.z]) | (uint32_t(row[p0.w]) << 16);
            o.z = uint32_t(row[p1.x]) | (uint32_t(row[p1.y]) << 16);
            o.w = uint32_t(row[p1.z]) | (uint32_t(row[p1.w]) << 16);
            dst[i] = o;
        }
        __syncthreads();  // the row buffer is rewritten for the next row
    }
}

// The same gather one element per thread, for rows too long for LDS.
__global__ void __launch_bounds__(256) gather_act_kernel(const uint16_t* __restrict__ x,
                                                         const int32_t* __restrict__ perm, int M, int K,
                                                         uint16_t* __restrict__ x_out) {
    const long long total = (long long)M * K;
    for (long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (long long)gridDim.x * blockDim.x) {
        const long long m = t / K;
        const int kp = int(t - m * K);
        x_out[t] = x[m * K + perm[kp]];
    }
}

// Blocks of gemm_kernel resident per CU, by tile height: the register file
// (512 per lane per SIMD, one wavefront of each block per SIMD) holds three
// 16-row, two 32-row and one 64- or 128-row block.
constexpr int small_tile_blocks_per_cu(int BM) { return BM <= 16 ? 3 : BM <= 32 ? 2 : 1; }

template <int BM, int BN>
wqh::SplitPlan tile_plan(int M, int N, int K, int bits, size_t ws_avail) {
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    return wqh::plan_split(M, N, K, bits, BM, BN, tiles, wqh::gemm_slots(small_tile_blocks_per_cu(BM)), ws_avail);
}

// With out32 the product is written unrounded as fp32 [M][N] (no split).
template <int BITS, int BM, int BN, int WAVES_M, int NST>
wq_status launch_tile(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                      uint16_t* y, int M, int N, int K, int gs, float* part, size_t part_bytes, float* out32,
                      hipStream_t s) {
    const int m_tiles = (M + BM - 1) / BM, n_tiles = (N + BN - 1) / BN;
    const int tiles = m_tiles * n_tiles;
    const GroupDiv gd = wqh::group_magic(gs);
    const wqh::SplitPlan plan = tile_plan<BM, BN>(M, N, K, BITS, (part && !out32) ? part_bytes : 0);
    const bool split = plan.splits > 1;
    const dim3 grid(tiles, plan.splits);
    float* pp = out32 ? out32 : (split ? part : nullptr);
    // PART is a template flag: the plain fp16 epilogue carries no branch
    if (zeros && pp)
        hipLaunchKernelGGL((gemm_kernel<BITS, BM, BN, WAVES_M, NST, true, true>), grid, dim3(256), 0, s, x, packed,
                           scales, zeros, y, M, N, K, gd, m_tiles, n_tiles, tiles, plan.sps, pp);
    else if (zeros)
        hipLaunchKernelGGL((gemm_kernel<BITS, BM, BN, WAVES_M, NST, true, false>), grid, dim3(256), 0, s, x, packed,
                           scales, zeros, y, M, N, K, gd, m_tiles, n_tiles, tiles, plan.sps, pp);
    else if (pp)
        hipLaunchKernelGGL((gemm_kernel<BITS, BM, BN, WAVES_M, NST, false, true>), grid, dim3(256), 0, s, x, packed,
                           scales, zeros, y, M, N, K, gd, m_tiles, n_tiles, tiles, plan.sps, pp);
    else
        hipLaunchKernelGGL((gemm_kernel<BITS, BM, BN, WAVES_M, NST, false, false>), grid, dim3(256), 0, s, x, packed,
                           scales, zeros, y, M, N, K, gd, m_tiles, n_tiles, tiles, plan.sps, pp);
    const wq_status st = wqh::launch_status();
    if (st != WQ_OK || !split) return st;
    return wqh::splitk_reduce(part, plan.splits, M, N, y, s);
}

// Small M: narrow tiles for more blocks.  Large M: 128 x 256 tiles with the
// four wavefronts side by side along N, so every packed weight column is
// dequantized by one wavefront and each activation row is re-read from L2
// once per 256 output columns.  Any of them splits K across blocks when there
// are too few tiles to fill the machine and the workspace holds the partials.
enum class TileKind { k16, k32, k64, kLarge, k128 };

// Pipeline depth (stages in flight + 1) of the small-M tiles.
#ifndef WQ_GEMM_SMALL_NST
#define WQ_GEMM_SMALL_NST 3
#endif
constexpr int kSmallNst = WQ_GEMM_SMALL_NST;

#ifndef WQ_GEMM_K64_MAX_M
#define WQ_GEMM_K64_MAX_M 64
#endif
inline TileKind tile_kind(int M, int N, int K, int bits) {
    if (M <= 16) return TileKind::k16;
    if (M <= 32) return TileKind::k32;
    if (M <= WQ_GEMM_K64_MAX_M) return TileKind::k64;
    if (wqh::gemm_large_fits(M, N, K, bits)) return TileKind::kLarge;
    return TileKind::k128;
}

// Bytes of fp32 partials the chosen kernel's split plan needs (0: no split).
inline size_t split_bytes(int M, int N, int K, int bits) {
    wqh::SplitPlan p;
    const size_t inf = ~size_t(0);
    switch (tile_kind(M, N, K, bits)) {
        case TileKind::k16: p = tile_plan<16, 64>(M, N, K, bits, inf); break;
        case TileKind::k32: p = tile_plan<32, 64>(M, N, K, bits, inf); break;
        case TileKind::k64: p = tile_plan<64, 128>(M, N, K, bits, inf); break;
        case TileKind::kLarge: p = wqh::gemm_large_plan(M, N, K, bits, inf); break;
        default: p = tile_plan<128, 256>(M, N, K, bits, inf); break;
    }
    return p.splits > 1 ? size_t(p.splits) * size_t(M) * size_t(N) * 4 : 0;
}

template <int BITS>
wq_status launch_bits(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                      uint16_t* y, int M, int N, int K, int gs, float* part, size_t part_bytes, hipStream_t s,
                      float* out32 = nullptr) {
    switch (tile_kind(M, N, K, BITS)) {
        case TileKind::k16:
            return launch_tile<BITS, 16, 64, 1, kSmallNst>(x, packed, scales, zeros, y, M, N, K, gs, part, part_bytes,
                                                            out32, s);
        case TileKind::k32:
            return launch_tile<BITS, 32, 64, 1, kSmallNst>(x, packed, scales, zeros, y, M, N, K, gs, part, part_bytes,
                                                            out32, s);
        case TileKind::k64:
            return launch_tile<BITS, 64, 128, 1, kSmallNst>(x, packed, scales, zeros, y, M, N, K, gs, part, part_bytes,
                                                            out32, s);
        case TileKind::kLarge: {
            const wqh::SplitPlan plan = wqh::gemm_large_plan(M, N, K, BITS, (part && !out32) ? part_bytes : 0);
            return wqh::gemm_large(BITS, x, packed, scales, zeros, y, M, N, K, gs, plan, part, out32, s);
        }
        default:
            return launch_tile<BITS, 128, 256, 1, 3>(x, packed, scales, zeros, y, M, N, K, gs, part, part_bytes,
                                                            out32, s);
    }
}

}  // namespace

namespace wqh {
wq_status check_linear_args(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint16_t* y,
                            int M, int N, int K, int bits, int group_size, int* gs_out);
}

namespace wqh {

int gemm_slots(int blocks_per_cu) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    return cus * blocks_per_cu;
}

wq_status splitk_reduce(const float* part, int splits, int M, int N, uint16_t* y, hipStream_t s) {
    const long long mn = (long long)M * N;
    // partials and y are 16-byte aligned (workspace and output checks)
    if (mn % 4 == 0) {
        const long long mn4 = mn / 4;
        long long blocks = (mn4 + 255) / 256;
        if (blocks > 8192) blocks = 8192;
        hipLaunchKernelGGL(splitk_reduce4_kernel, dim3(int(blocks)), dim3(256), 0, s,
                           reinterpret_cast<const float4*>(part), splits, mn4, reinterpret_cast<uint2*>(y));
        return launch_status();
    }
    long long blocks = (mn + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(int(blocks)), dim3(256), 0, s, part, splits, mn, y);
    return launch_status();
}

wq_status gemm_f32(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                   float* y32, int M, int N, int K, int bits, int gs, hipStream_t s) {
    switch (bits) {
        case 2: return launch_bits<2>(x, packed, scales, zeros, nullptr, M, N, K, gs, nullptr, 0, s, y32);
        case 3: return launch_bits<3>(x, packed, scales, zeros, nullptr, M, N, K, gs, nullptr, 0, s, y32);
        case 4: return launch_bits<4>(x, packed, scales, zeros, nullptr, M, N, K, gs, nullptr, 0, s, y32);
        default: return launch_bits<8>(x, packed, scales, zeros, nullptr, M, N, K, gs, nullptr, 0, s, y32);
    }
}

}  // namespace wqh

// Workspace layout: [gathered activations, act-order only, rounded up to 256
// bytes] [split-K fp32 partials, when the launch splits K].
static size_t gather_bytes(int M, int K, int has_perm) {
    if (!has_perm) return 0;
    return (size_t(M) * size_t(K) * 2 + 255) & ~size_t(255);
}

namespace wqh {
size_t skinny_workspace_bytes(int M, int N, int K);
}

extern "C" size_t wq_workspace_size(int32_t M, int32_t N, int32_t K, int32_t bits, int32_t has_perm) {
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    if (bits != 2 && bits != 3 && bits != 4 && bits != 8) return 0;
    const size_t gemm = gather_bytes(M, K, has_perm) + split_bytes(M, N, K, bits);
    // the decode kernel's K split (M <= 16, no act-order)
    const size_t gemv = has_perm ? 0 : wqh::skinny_workspace_bytes(M, N, K);
    return std::max(gemm, gemv);
}

extern "C" wq_status wq_gemm(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                             const int32_t* perm, uint16_t* y, int32_t M, int32_t N, int32_t K, int32_t bits,
                             int32_t group_size, void* workspace, size_t workspace_bytes, void* stream) {
    int gs = 0;
    const wq_status st = wqh::check_linear_args(x, packed, scales, y, M, N, K, bits, group_size, &gs);
    if (st != WQ_OK) return st;
    if (perm && !wqh::aligned16(perm)) return WQ_ERR_ARG;
    if (M == 0 || N == 0) return WQ_OK;
    if (workspace && !wqh::aligned16(workspace)) return WQ_ERR_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint16_t* xa = x;
    const size_t gb = gather_bytes(M, K, perm != nullptr);
    if (perm) {
        if (!workspace || workspace_bytes < size_t(M) * size_t(K) * 2) return WQ_ERR_ARG;
        uint16_t* xg = static_cast<uint16_t*>(workspace);
        if (size_t(K) * 2 <= 64 * 1024) {
            hipLaunchKernelGGL(gather_rows_kernel, dim3(std::min(M, 65535)), dim3(256), size_t(K) * 2, s, x, perm,
                               int(M), int(K), xg);
        } else {
            long long total = (long long)M * K;
            long long blocks = (total + 255) / 256;
            if (blocks > 65536) blocks = 65536;
            hipLaunchKernelGGL(gather_act_kernel, dim3(int(blocks)), dim3(256), 0, s, x, perm, int(M), int(K), xg);
        }
        const wq_status ls = wqh::launch_status();
        if (ls != WQ_OK) return ls;
        xa = xg;
    }
    // split-K partials go after the gathered activations; without room for
    // them the launch does not split
    float* part = nullptr;
    size_t part_bytes = 0;
    if (workspace && workspace_bytes > gb) {
        part = reinterpret_cast<float*>(static_cast<char*>(workspace) + gb);
        part_bytes = workspace_bytes - gb;
    }
    switch (bits) {
        case 2: return launch_bits<2>(xa, packed, scales, zeros, y, M, N, K, gs, part, part_bytes, s);
        case 3: return launch_bits<3>(xa, packed, scales, zeros, y, M, N, K, gs, part, part_bytes, s);
        case 4: return launch_bits<4>(xa, packed, scales, zeros, y, M, N, K, gs, part, part_bytes, s);
        default: return launch_bits<8>(xa, packed, scales, zeros, y, M, N, K, gs, part, part_bytes, s);
    }
}
