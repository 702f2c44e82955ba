// Device helpers shared by the prefill GEMM kernels (gfx950 only).
#pragma once

#include <algorithm>

#include "wq_common.h"

namespace wq {

template <int BITS>
__device__ __forceinline__ void load_chunk_b(const uint32_t* p, uint32_t* w) {
    if constexpr (BITS == 4) {
        const u4 v = *reinterpret_cast<const u4*>(p);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else if constexpr (BITS == 8) {
        const u4 a = reinterpret_cast<const u4*>(p)[0];
        const u4 b = reinterpret_cast<const u4*>(p)[1];
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else if constexpr (BITS == 2) {
        typedef uint32_t u2 __attribute__((ext_vector_type(2)));
        const u2 v = *reinterpret_cast<const u2*>(p);
        w[0] = v.x; w[1] = v.y;
    } else {
        w[0] = p[0]; w[1] = p[1]; w[2] = p[2];
    }
}

typedef __attribute__((address_space(1))) const void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// Tile index of block b when blocks are dealt round-robin to `parts` XCDs:
// XCD j gets the contiguous tile range [start_j, start_j + count_j).
__device__ __forceinline__ int xcd_tile(int b, int tiles, int parts) {
    const int q = tiles / parts, r = tiles % parts;
    const int xcd = b % parts, k = b / parts;
    return xcd < r ? xcd * (q + 1) + k : r * (q + 1) + (xcd - r) * q + k;
}

// vmcnt(n) with the other counters left alone (gfx9 s_waitcnt encoding).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }
// vmcnt(n) and lgkmcnt(0).
constexpr int vmcnt_lgkm0_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70; }

// Workgroup barrier for the copy pipeline: this wavefront's LDS reads are
// done (lgkmcnt(0)) and all but the newest n vector-memory operations -
// among them its global->LDS copies - have landed, then s_barrier.
// __syncthreads() would also order every outstanding LDS write, i.e. drain
// the copies that are meant to stay in flight.  The empty asm statements
// keep the compiler from moving memory accesses across the barrier.
template <int N>
__device__ __forceinline__ void copy_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(N));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Output tile of block b: tiles are dealt to the XCDs in contiguous ranges
// (xcd_tile) and a run of consecutive tile numbers covers a strip of GM
// M-tiles by several N-tiles, so the blocks resident on one XCD at a time
// reuse both their activation rows and their weight columns from its L2.
template <int GM>
__device__ __forceinline__ void tile_coords(int b, int tiles, int m_tiles, int n_tiles, int& m_t, int& n_t) {
    const int t = xcd_tile(b, tiles, 8);
    const int per_group = GM * n_tiles;
    const int group = t / per_group;
    const int first_m = group * GM;
    const int gsm = min(m_tiles - first_m, GM);
    const int r = t - group * per_group;
    m_t = first_m + r % gsm;
    n_t = r / gsm;
}

}  // namespace wq

namespace wqh {

// Split-K plan of one GEMM launch: the K stages (128 deep) are cut into
// `splits` ranges of `sps` stages; with splits > 1 every block writes its
// fp32 partial tile to the workspace and splitk_reduce sums the ranges.
struct SplitPlan {
    int splits = 1, sps = 0;
};

// Pick the split count that minimizes a simple time model: one tile over all
// of K takes `unit_us`; `tiles * S` blocks run in rounds of `slots` resident
// blocks, each doing 1/S of the work; every extra range costs writing and
// re-reading an fp32 copy of y plus the reduction launch.  Ranges keep at
// least 4 stages, and the partials must fit in `ws_avail` bytes.
inline SplitPlan plan_split(int M, int N, int K, int bits, int BM, int BN, int tiles, int slots, size_t ws_avail) {
    SplitPlan best;
    const int stages = (K + 127) / 128;
    best.sps = stages;
    if (tiles <= 0 || slots <= 0 || stages < 8) return best;
    const double flops_tile = 2.0 * BM * BN * double(K);
    const double bytes_tile = double(BN) * K * bits / 8.0;
    const double unit_us = std::max(flops_tile / 3.5e12, bytes_tile / 15e9) * 1e6;
    const double part_bytes = double(M) * N * 4.0;
    const double part_us = 2.0 * part_bytes / 4e12 * 1e6;
    double best_cost = unit_us * double((tiles + slots - 1) / slots);
    for (int S = 2; S <= 16 && S * 4 <= stages; ++S) {
        const int sps = (stages + S - 1) / S;
        const int Se = (stages + sps - 1) / sps;  // ranges actually used
        if (double(Se) * part_bytes > double(ws_avail)) break;
        const long long blocks = (long long)tiles * Se;
        const double rounds = double((blocks + slots - 1) / slots);
        const double cost = unit_us * rounds * double(sps) / stages + Se * part_us + 2.0;
        if (cost < best_cost * 0.97) {
            best_cost = cost;
            best.splits = Se;
            best.sps = sps;
        }
    }
    return best;
}

// Resident blocks of a GEMM kernel on the current device.
int gemm_slots(int blocks_per_cu);

// y[m][n] = fp16(sum over ranges r = 0..splits-1, in order, of part[r][m][n]).
wq_status splitk_reduce(const float* part, int splits, int M, int N, uint16_t* y, hipStream_t s);

// Large-M prefill GEMM (128 x 256 tiles on 32x32x16 instructions).  Its
// offsets are 32-bit: usable when gemm_large_fits().
bool gemm_large_fits(int M, int N, int K, int bits);
// Split plan of the large-M kernel for these arguments (ws_avail: bytes of
// workspace available for partials).
SplitPlan gemm_large_plan(int M, int N, int K, int bits, size_t ws_avail);
// With out32 the unrounded product goes to fp32 [M][N] instead of y (no split).
wq_status gemm_large(int bits, const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                     const uint8_t* zeros, uint16_t* y, int M, int N, int K, int gs, SplitPlan plan,
                     float* part, float* out32, hipStream_t s);

// The GEMM with the unrounded fp32 product y32 [M][N] as output (inputs
// already checked by the caller; packed column order = original order).
wq_status gemm_f32(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                   float* y32, int M, int N, int K, int bits, int gs, hipStream_t s);

// Plain fp16 product y32[m][n] = sum_k x[m][k] w[n][k] in fp32 (matrix
// cores); K a multiple of 32, rows 16-byte aligned.
wq_status dense_f32(const uint16_t* x, const uint16_t* w, float* y32, int M, int N, int K, hipStream_t s);

}  // namespace wqh
