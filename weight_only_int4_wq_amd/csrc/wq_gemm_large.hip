// Prefill GEMM for large M: y[M][N] = x[M][K] . dequant(Wq)^T on 32x32x16
// fp16 matrix-core instructions with fp32 accumulators (the batched GEMM
// kernel of "AutoAWQ vs The Stack v2" and "AutoAWQ vs Unsloth", WQLinear_*
// paragraphs: weights dequantized on the fly, never stored as fp16).
//
// A 256-thread block owns a BM x 256 output tile (BM = 128, or 64 for a few
// hundred rows, where 128-row tiles leave too few tiles and the K split's
// fp32 partials dominate); its four wavefronts sit side by side along N,
// each with a BM x 64 tile = BM/32 x 2 instructions of 32 x 32.  K advances
// in stages of 128 (one quantization group for the usual group size), eight
// 16-deep k-steps per stage.
//
// One 32x32x16 instruction does the work of two 16x16x32 ones, so a single
// wavefront per SIMD has twice the issue slots per instruction for the LDS
// reads, the weight decode and the address arithmetic around it.
//
//  - Activations: each stage's BM x 128 fp16 tile is copied global -> LDS
//    by global_load_lds_dwordx4 (16-byte units; unit u of row r stored at
//    u ^ (r mod 16)), three stages in flight in three buffers.
//  - Weights: in a 32x32x16 instruction lane l supplies 8 consecutive k of
//    column l mod 32, i.e. one packed 8-code block.  Lane half h = l / 32
//    covers k in [64h, 64h + 64) of a stage (chunks 2h and 2h + 1 of the
//    row, two 16-byte loads for 4-bit codes), k-step t uses block t of that
//    range; the activation fragments are read with the same k mapping.
//    Packed words, scales and zeros are loaded three stages ahead into
//    rotating register sets and dequantized in registers (exact
//    (q - z) * s, one rounding), straight into the B operand.
//  - The stage barrier sits before the last k-step's matrix instructions:
//    by then every LDS read of the stage has been issued, so the next
//    stage's first fragments and the copies three stages ahead start while
//    those instructions run.
#include <type_traits>

#include "wq_gemm_common.h"

namespace {

using namespace wq;

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Natural-order pairs (codes 2i, 2i+1 of block b) as fp16 pairs that differ
// from (q_{2i}, q_{2i+1}) by the constants of zero_pair_nat.
template <int BITS>
__device__ __forceinline__ void decode_nat(const uint32_t* w, int b, uint32_t* h) {
    if constexpr (BITS == 4) {
        // Byte i of the block word holds codes 2i (low nibble) and 2i+1 (high
        // nibble).  Copy it into bytes 0 and 2, then keep the low nibble in
        // the low half under 0x6400 (1024 + q, unit step) and the high nibble
        // in bits 4..7 of the high half under 0x5400 (64 + q, step 1/16 * 16).
        const uint32_t v = w[b];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t sel = 0x0C000C00u | (uint32_t(i) << 16) | uint32_t(i);
            h[i] = and_or(__builtin_amdgcn_perm(v, v, sel), 0x00F0000Fu, 0x54006400u);
        }
    } else {
        decode_block_nat<BITS>(w, b, h);
    }
}

// The pair subtracted from decode_nat's output to leave q - z exactly.
template <int BITS>
__device__ __forceinline__ uint32_t zero_pair_nat(uint32_t z) {
    if constexpr (BITS == 4)
        return (0x6400u | z) | ((0x5400u | (z << 4)) << 16);
    else
        return zero_pair(z);
}

template <int BITS, bool HAS_Z, bool FAST, bool PART, int BM>
__global__ void __launch_bounds__(256) gemm_large_kernel(const uint16_t* __restrict__ x,
                                                         const uint32_t* __restrict__ packed,
                                                         const uint16_t* __restrict__ scales,
                                                         const uint8_t* __restrict__ zeros,
                                                         uint16_t* __restrict__ y, int M, int N, int K, GroupDiv gd,
                                                         int m_tiles, int n_tiles, int tiles, int sps,
                                                         float* __restrict__ part) {
    constexpr int GM = 4;
    static_assert(BM == 128 || BM == 64, "tile rows");
    constexpr int BN = 256, BK = 128, WN = 64;
    constexpr int TM = BM / 32, TN = WN / 32;
    constexpr int ROW_BYTES = BK * 2;
    constexpr int A_INSTR = BM / 16;      // 1 KB copies per wavefront per stage
    constexpr int CW = BITS;              // 32-bit words per 32-code chunk
    constexpr int NG = FAST ? 1 : 2;      // groups per lane, column and stage
    // Vector-memory instructions of one issue_b, counted low: the compiler
    // may merge a lane's two chunk loads (16 bytes at most per load), and a
    // low count only makes the copy barrier wait for more.
    constexpr int B_OPS = TN * ((BITS + 1) / 2 + NG * (HAS_Z ? 2 : 1));

    __shared__ __attribute__((aligned(1024))) uint8_t As0[BM * ROW_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t As1[BM * ROW_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t As2[BM * ROW_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const int c = lane & 31, hh = lane >> 5;
    int m_t, n_t;
    tile_coords<GM>(blockIdx.x, tiles, m_tiles, n_tiles, m_t, n_t);
    const int m0 = m_t * BM, n0 = n_t * BN;
    const int chunks = K / 32;
    const int G = chunk_group(chunks - 1, gd) + 1;
    const int stages = (K + BK - 1) / BK;
    // split-K: this block's range of stages (blockIdx.y), all of K unsplit
    const int st_begin = blockIdx.y * sps;
    const int st_end = min(st_begin + sps, stages);

    // ---- activation copies: byte offset of each copy's source from x + k0
    // (rows past M read row M - 1; their outputs are not stored).  With
    // FAST every stage is whole; otherwise units past K read the row's last
    // unit instead and meet zero weights.
    uint32_t a_row[A_INSTR], a_u[A_INSTR];
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i) {
        const int row = (wave * A_INSTR + i) * 4 + (lane >> 4);
        const int u = (lane & 15) ^ (row & 15);
        const int gm = min(m0 + row, M - 1);
        a_row[i] = uint32_t(gm) * uint32_t(K) * 2u;
        a_u[i] = uint32_t(u) * 8u;
    }
    auto issue_a = [&](uint8_t* buf, int k0, int i0, int i1) {
        const char* base = reinterpret_cast<const char*>(x + k0);
#pragma unroll
        for (int i = i0; i < i1; ++i) {
            const char* src;
            if constexpr (FAST) {
                src = base + (a_row[i] + 2u * a_u[i]);
            } else {
                const uint32_t gk = min(uint32_t(k0) + a_u[i], uint32_t(K - 8));
                src = reinterpret_cast<const char*>(x) + (a_row[i] + 2u * gk);
            }
            __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)(buf + (wave * A_INSTR + i) * 1024), 16, 0, 0);
        }
    };

    // ---- weights: this lane's column of each 32-column block, its chunk
    // pair of every stage, and the matching scale / zero entries
    uint32_t b_row[TN], s_row[TN];
    bool n_ok[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int n = n0 + wave * WN + 32 * j + c;
        n_ok[j] = n < N;
        const uint32_t nn = n_ok[j] ? uint32_t(n) : 0u;
        b_row[j] = nn * uint32_t(chunks * CW) * 4u + uint32_t(hh) * 2u * CW * 4u;
        s_row[j] = nn * uint32_t(G);
    }
    struct BRegs {
        uint32_t w[TN][2][CW];
        uint32_t s[TN][NG], z[TN][NG];
        bool kok[NG];
    };
    // Loads of column block j of stage st (packed chunk pair, scale, zero).
    auto issue_b = [&](BRegs& b, int st, int j) {
        if constexpr (FAST) {
            const char* base = reinterpret_cast<const char*>(packed + st * 4 * CW);
            const int g = chunk_group(4 * st, gd);
            const uint32_t* p = reinterpret_cast<const uint32_t*>(base + b_row[j]);
            load_chunk_b<BITS>(p, b.w[j][0]);
            load_chunk_b<BITS>(p + CW, b.w[j][1]);
            b.s[j][0] = scales[s_row[j] + g];
            if constexpr (HAS_Z)
                b.z[j][0] = zeros[s_row[j] + g];
            else
                b.z[j][0] = 1u << (BITS - 1);
            b.kok[0] = true;
        } else {
            const uint32_t* rowp =
                reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(packed) + b_row[j]) - hh * 2 * CW;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int cg = 4 * st + 2 * hh + e;
                b.kok[e] = cg < chunks;
                const int cgc = min(cg, chunks - 1);
                const int g = chunk_group(cgc, gd);
                load_chunk_b<BITS>(rowp + cgc * CW, b.w[j][e]);
                b.s[j][e] = scales[s_row[j] + g];
                if constexpr (HAS_Z)
                    b.z[j][e] = zeros[s_row[j] + g];
                else
                    b.z[j][e] = 1u << (BITS - 1);
            }
        }
    };
    auto issue_b_all = [&](BRegs& b, int st) {
#pragma unroll
        for (int j = 0; j < TN; ++j) issue_b(b, st, j);
    };

    struct Q {
        uint32_t zz[TN][NG], ss[TN][NG];
    };
    auto make_q = [&](const BRegs& b, Q& q) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < NG; ++e) {
                q.zz[j][e] = zero_pair_nat<BITS>(b.z[j][e]);
                q.ss[j][e] = (n_ok[j] && b.kok[e]) ? scale_pair(uint16_t(b.s[j][e])) : 0u;
            }
    };

    // A fragment of k-step t: rows 32i + c, unit 8h + t (swizzled)
    const uint32_t a_lane = uint32_t(c) * ROW_BYTES;
    auto load_a = [&](const uint8_t* buf, int t, h8 (&af)[TM]) {
        const uint32_t u = uint32_t(8 * hh + t) ^ uint32_t(c & 15);
        const uint8_t* p = buf + a_lane + u * 16u;
#pragma unroll
        for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const h8*>(p + i * 32 * ROW_BYTES);
    };
    auto make_b = [&](const BRegs& b, const Q& q, int t, h8 (&bf)[TN]) {
        const int e = t >> 2, blk = t & 3, ge = FAST ? 0 : e;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            uint32_t hq[4], f[4];
            decode_nat<BITS>(b.w[j][e], blk, hq);
#pragma unroll
            for (int p = 0; p < 4; ++p) f[p] = as_u32(dequant_pair(hq[p], q.zz[j][ge], q.ss[j][ge]));
            const u4 fv = {f[0], f[1], f[2], f[3]};
            bf[j] = __builtin_bit_cast(h8, fv);
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    h8 af[2][TM], bf[2][TN];
    Q q, qn;

    // Loads for stage st + 2 are spread over k-steps 0..6 of stage st, into
    // the register set and LDS buffer that stage st - 1 used (free since the
    // barrier that ended it): activation copies (1 KB each) over all seven
    // (BM = 128) or one at each of k-steps 0..3 (BM = 64), weight column
    // blocks at k-steps 1 and 4.
    auto a_first = [](int t) { return A_INSTR == 8 ? (t == 0 ? 0 : t + 1) : min(t, A_INSTR); };
    auto b_step = [](int j) { return 1 + 3 * j; };
    static_assert((A_INSTR == 8 || A_INSTR == 4) && TN <= 2, "load schedule");

    // Issue order within a k-step: each matrix instruction is followed by a
    // share of the LDS reads, loads and decode / dequant work of the next
    // k-step, so they run while it occupies the matrix core (in-order issue
    // would otherwise hold them behind a burst of matrix instructions).
#ifndef WQ_GEMM_L_VALU_PER_MFMA
#define WQ_GEMM_L_VALU_PER_MFMA 5
#endif
    auto interleave = [&](int n_vmem) {
#pragma unroll
        for (int m = 0; m < TM * TN; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (m < n_vmem) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            if (m < TM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, WQ_GEMM_L_VALU_PER_MFMA, 0);
        }
        // one scheduling region per k-step keeps the pattern solver cheap
        __builtin_amdgcn_sched_barrier(0);
    };

    // One stage.  On entry af[0] / bf[0] hold its k-step 0.  Its weights sit
    // in `cur`, its activations in Ab; the next stage's in `nxt` / An; the
    // loads of stage st + 2 go to `fill` / Af.  Without ISSUE (the stages
    // after the unrolled loop, where no stage st + 2 exists) nothing is
    // loaded and the barrier waits for every load in flight: the count of
    // loads a stage leaves in flight must be the one the barrier assumes, and
    // loads into registers never read again would be dropped by the compiler.
    auto stage = [&](auto issue_c, int st, const BRegs& cur, const BRegs& nxt, BRegs& fill, const uint8_t* Ab,
                     const uint8_t* An, uint8_t* Af) {
        constexpr bool ISSUE = decltype(issue_c)::value;
        const int sf = min(st + 2, st_end - 1);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int cb = t & 1;
            int n_vmem = 0;
            if (t < 7) {
                if constexpr (ISSUE) {
                const int i0 = a_first(t), i1 = a_first(t + 1);
                issue_a(Af, sf * BK, i0, i1);
                n_vmem = i1 - i0;
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    if (b_step(j) == t) {
                        issue_b(fill, sf, j);
                        n_vmem += 2 * (BITS == 8 ? 2 : 1) + NG * (HAS_Z ? 2 : 1);
                    }
                }
                load_a(Ab, t + 1, af[cb ^ 1]);
                make_b(cur, q, t + 1, bf[cb ^ 1]);
            } else {
                // stage st + 1 has landed; every read of Ab is done
                copy_barrier<ISSUE ? B_OPS + A_INSTR : 0>();
                make_q(nxt, qn);
                load_a(An, 0, af[0]);
                make_b(nxt, qn, 0, bf[0]);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[cb][i], bf[cb][j], acc[i][j], 0, 0, 0);
            interleave(n_vmem);
        }
        q = qn;
    };

    // Stage s uses register set s % 3 and buffer s % 3 (compile-time: the
    // loop is unrolled by 3).  Inside the loop, loads past the last stage
    // re-read the last stage into buffers and registers that are not used
    // again.
    BRegs b0, b1, b2;
    const int st_next = min(st_begin + 1, st_end - 1);
    issue_b_all(b0, st_begin);
    issue_a(As0, st_begin * BK, 0, A_INSTR);
    issue_b_all(b1, st_next);
    issue_a(As1, st_next * BK, 0, A_INSTR);
    copy_barrier<B_OPS + A_INSTR>();
    make_q(b0, q);
    load_a(As0, 0, af[0]);
    make_b(b0, q, 0, bf[0]);

    int st = st_begin;
    const std::true_type loads;
    const std::false_type no_loads;
    for (; st + 3 <= st_end; st += 3) {
        stage(loads, st, b0, b1, b2, As0, As1, As2);
        stage(loads, st + 1, b1, b2, b0, As1, As2, As0);
        stage(loads, st + 2, b2, b0, b1, As2, As0, As1);
    }
    if (st < st_end) stage(no_loads, st, b0, b1, b2, As0, As1, As2);
    if (st + 1 < st_end) stage(no_loads, st + 1, b1, b2, b0, As1, As2, As0);

    // no copy may still be writing this block's LDS when it exits
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

    // ---- epilogue: acc[i][j][r] is row 32i + 8(r/4) + 4h + r%4, column
    // 32j + c of the wavefront's tile; fp16 y, or this range's fp32 partial
    float* pr = PART ? part + (size_t)blockIdx.y * M * N : nullptr;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = n0 + wave * WN + 32 * j + c;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
                if (row < M && col < N) {
                    if constexpr (PART)
                        pr[(size_t)row * N + col] = acc[i][j][r];
                    else
                        y[(size_t)row * N + col] = __builtin_bit_cast(uint16_t, (_Float16)acc[i][j][r]);
                }
            }
        }
}

template <int BITS, bool HAS_Z, int BM>
wq_status launch_z(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                   uint16_t* y, int M, int N, int K, int gs, wqh::SplitPlan plan, float* part, float* out32,
                   hipStream_t s) {
    constexpr int BN = 256;
    const int m_tiles = (M + BM - 1) / BM, n_tiles = (N + BN - 1) / BN;
    const int tiles = m_tiles * n_tiles;
    const GroupDiv gd = wqh::group_magic(gs);
    const bool fast = (K % 128 == 0) && (gs % 128 == 0);
    if (out32) plan = wqh::SplitPlan{1, (K + 127) / 128};
    const bool split = plan.splits > 1;
    const dim3 grid(tiles, plan.splits);
    float* pp = out32 ? out32 : (split ? part : nullptr);
    // PART (fp32 partials or the fp32 output) is a template flag so that the
    // plain fp16 epilogue carries no per-element branch
    if (fast && pp)
        hipLaunchKernelGGL((gemm_large_kernel<BITS, HAS_Z, true, true, BM>), grid, dim3(256), 0, s, x, packed, scales,
                           zeros, y, M, N, K, gd, m_tiles, n_tiles, tiles, plan.sps, pp);
    else if (fast)
        hipLaunchKernelGGL((gemm_large_kernel<BITS, HAS_Z, true, false, BM>), grid, dim3(256), 0, s, x, packed, scales,
                           zeros, y, M, N, K, gd, m_tiles, n_tiles, tiles, plan.sps, pp);
    else if (pp)
        hipLaunchKernelGGL((gemm_large_kernel<BITS, HAS_Z, false, true, BM>), grid, dim3(256), 0, s, x, packed, scales,
                           zeros, y, M, N, K, gd, m_tiles, n_tiles, tiles, plan.sps, pp);
    else
        hipLaunchKernelGGL((gemm_large_kernel<BITS, HAS_Z, false, false, BM>), grid, dim3(256), 0, s, x, packed, scales,
                           zeros, y, M, N, K, gd, m_tiles, n_tiles, tiles, plan.sps, pp);
    const wq_status st = wqh::launch_status();
    if (st != WQ_OK || !split) return st;
    return wqh::splitk_reduce(part, plan.splits, M, N, y, s);
}

// Tile rows of the large kernel.  64-row tiles (two blocks per compute
// unit) where 128-row tiles are few and K is short, up to
// WQ_GEMM_L_BM64_MAX_M rows: measured on MI355X (4-bit, group 128) they gain
// 7-15 % on 4096 x 4096 at M = 96-256 and 3-9 % on the 2/3/8-bit 4096 x 4096
// layers at M = 256, but lose 16-25 % on the wider Llama and 70B shapes and
// on K = 11008.  Off by default (0): one GPU parity run gave a wrong sum on
// a 2-bit act-order layer at M = 256 with them, whose cause is not found.
#ifndef WQ_GEMM_L_BM64_MAX_M
#define WQ_GEMM_L_BM64_MAX_M 0
#endif
inline int large_bm(int M, int N, int K) {
    const int tiles128 = ((M + 127) / 128) * ((N + 255) / 256);
    return (M <= WQ_GEMM_L_BM64_MAX_M && K <= 4096 && tiles128 <= 32) ? 64 : 128;
}
// Resident blocks per compute unit: one 128-row block (96 KB of LDS, 128
// accumulator registers per lane), two 64-row blocks (48 KB, 64).
inline int large_blocks_per_cu(int bm) { return bm == 64 ? 2 : 1; }

template <int BITS>
wq_status launch_large(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                       uint16_t* y, int M, int N, int K, int gs, wqh::SplitPlan plan, float* part, float* out32,
                       hipStream_t s) {
    if (large_bm(M, N, K) == 64) {
        if (zeros) return launch_z<BITS, true, 64>(x, packed, scales, zeros, y, M, N, K, gs, plan, part, out32, s);
        return launch_z<BITS, false, 64>(x, packed, scales, zeros, y, M, N, K, gs, plan, part, out32, s);
    }
    if (zeros) return launch_z<BITS, true, 128>(x, packed, scales, zeros, y, M, N, K, gs, plan, part, out32, s);
    return launch_z<BITS, false, 128>(x, packed, scales, zeros, y, M, N, K, gs, plan, part, out32, s);
}

}  // namespace

namespace wqh {

bool gemm_large_fits(int M, int N, int K, int bits) {
    // byte offsets of activations, packed rows and group entries are 32-bit
    const uint64_t lim = uint64_t(1) << 32;
    return uint64_t(M) * uint64_t(K) * 2u < lim && uint64_t(N) * uint64_t(K) * uint64_t(bits) / 8u < lim &&
           uint64_t(N) * uint64_t(K / 32) < lim;
}

SplitPlan gemm_large_plan(int M, int N, int K, int bits, size_t ws_avail) {
    constexpr int BN = 256;
    const int BM = large_bm(M, N, K);
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    return plan_split(M, N, K, bits, BM, BN, tiles, gemm_slots(large_blocks_per_cu(BM)), ws_avail);
}

wq_status gemm_large(int bits, const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                     const uint8_t* zeros, uint16_t* y, int M, int N, int K, int gs, SplitPlan plan, float* part,
                     float* out32, hipStream_t s) {
    switch (bits) {
        case 2: return launch_large<2>(x, packed, scales, zeros, y, M, N, K, gs, plan, part, out32, s);
        case 3: return launch_large<3>(x, packed, scales, zeros, y, M, N, K, gs, plan, part, out32, s);
        case 4: return launch_large<4>(x, packed, scales, zeros, y, M, N, K, gs, plan, part, out32, s);
        default: return launch_large<8>(x, packed, scales, zeros, y, M, N, K, gs, plan, part, out32, s);
    }
}

}  // namespace wqh
