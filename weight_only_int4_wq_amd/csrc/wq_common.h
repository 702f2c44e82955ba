// Shared host/device helpers of libwq (gfx950 only).
//
// Packed format: row n of the weight matrix is a little-endian bitstream of
// b-bit codes.  The kernels work on "chunks" of 32 consecutive packed columns
// (32*b bits = b whole words, so every chunk starts on a word boundary) and
// split a chunk into four "blocks" of 8 codes (b whole bytes each).
//
// Decoding turns the 8 codes of a block into four fp16 pairs with the
// exponent trick: the 16-bit pattern 0x6400 | q is the fp16 number 1024 + q
// for 0 <= q < 1024, so a bit-field extraction plus one OR yields exact fp16
// integers, and (1024 + q) - (1024 + z) = q - z is an exact fp16 subtraction.
// One fp16 multiply by the group scale then rounds (q - z) * s once, which is
// the dequantized weight.  Pair i (i = 0..3) of a block holds codes i and
// i + 4 of the block (low half, high half): the order in which shifts of a
// packed word expose them.  Activations are staged in the same order so that
// fp16-pair dot products and matrix-core fragments line up.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/wq.h"

namespace wq {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kMagic2 = 0x64006400u;  // fp16 pair (1024, 1024)

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// (a & mask) | magic in one v_and_or_b32.  With both constants visible the
// compiler splits it into an and and an or (the VOP3 encoding cannot carry
// two literals), so the empty asm statements hide their values: mask comes
// to sit in an SGPR, magic in a VGPR, and the compiler selects the single
// instruction itself.  The instruction must not be written as inline asm:
// the compiler does not count an asm statement as a vector-ALU instruction
// when it inserts the wait states between the vector ALU and the matrix
// cores, and a decoded word written over the accumulator input of a matrix
// instruction still in flight corrupts its result.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t magic) {
    asm("" : "+s"(mask));
    asm("" : "+v"(magic));
    return (a & mask) | magic;
}

// Number of 32-bit words in one 32-code chunk of a `bits`-wide code stream.
template <int BITS>
struct Chunk {
    static constexpr int kWords = BITS;
};

// Decode the 32 codes of one chunk (w[0..BITS-1]) into 16 fp16 pairs
// (1024 + q_a, 1024 + q_b); pair 4*b + i holds codes 8b+i and 8b+i+4.
template <int BITS>
__device__ __forceinline__ void decode_chunk(const uint32_t* w, uint32_t* h);

template <>
__device__ __forceinline__ void decode_chunk<4>(const uint32_t* w, uint32_t* h) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint32_t v = w[b];
        h[4 * b + 0] = and_or(v, 0x000F000Fu, kMagic2);
        h[4 * b + 1] = and_or(v >> 4, 0x000F000Fu, kMagic2);
        h[4 * b + 2] = and_or(v >> 8, 0x000F000Fu, kMagic2);
        h[4 * b + 3] = and_or(v >> 12, 0x000F000Fu, kMagic2);
    }
}

template <>
__device__ __forceinline__ void decode_chunk<8>(const uint32_t* w, uint32_t* h) {
    // Block b is words 2b (codes 0..3) and 2b+1 (codes 4..7), one byte each.
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint32_t lo = w[2 * b], hi = w[2 * b + 1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // byte0 <- lo.byte i, byte2 <- hi.byte i, bytes 1 and 3 <- 0
            const uint32_t sel = 0x0C000C00u | ((4u + i) << 16) | uint32_t(i);
            h[4 * b + i] = __builtin_amdgcn_perm(hi, lo, sel) | kMagic2;
        }
    }
}

template <>
__device__ __forceinline__ void decode_chunk<2>(const uint32_t* w, uint32_t* h) {
    // Block b is 16 bits: byte 2b holds codes 0..3, byte 2b+1 codes 4..7.
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint32_t v = w[b >> 1];
        const uint32_t base = (b & 1) ? 2u : 0u;
        const uint32_t sel = 0x0C000C00u | ((base + 1u) << 16) | base;
        const uint32_t t = __builtin_amdgcn_perm(0u, v, sel);
        h[4 * b + 0] = and_or(t, 0x00030003u, kMagic2);
        h[4 * b + 1] = and_or(t >> 2, 0x00030003u, kMagic2);
        h[4 * b + 2] = and_or(t >> 4, 0x00030003u, kMagic2);
        h[4 * b + 3] = and_or(t >> 6, 0x00030003u, kMagic2);
    }
}

template <>
__device__ __forceinline__ void decode_chunk<3>(const uint32_t* w, uint32_t* h) {
    // Block b is 24 bits at bit offset 24b of the 96-bit chunk.
    uint32_t v[4];
    v[0] = w[0] & 0x00FFFFFFu;
    v[1] = __builtin_amdgcn_alignbit(w[1], w[0], 24) & 0x00FFFFFFu;
    v[2] = __builtin_amdgcn_alignbit(w[2], w[1], 16) & 0x00FFFFFFu;
    v[3] = w[2] >> 8;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        // codes 0..3 (12 bits) to the low half, codes 4..7 to the high half
        const uint32_t t = (v[b] & 0x00000FFFu) | ((v[b] << 4) & 0x0FFF0000u);
        h[4 * b + 0] = and_or(t, 0x00070007u, kMagic2);
        h[4 * b + 1] = and_or(t >> 3, 0x00070007u, kMagic2);
        h[4 * b + 2] = and_or(t >> 6, 0x00070007u, kMagic2);
        h[4 * b + 3] = and_or(t >> 9, 0x00070007u, kMagic2);
    }
}

// Natural-order decode of block b (8 codes) of a chunk into four fp16 pairs
// (1024 + q_{2i}, 1024 + q_{2i+1}), i = 0..3: consecutive codes share a pair,
// so the pairs line up with activations in their stored order (the layout
// matrix-core fragments read from LDS).
template <int BITS>
__device__ __forceinline__ void decode_block_nat(const uint32_t* w, int b, uint32_t* h);

template <>
__device__ __forceinline__ void decode_block_nat<4>(const uint32_t* w, int b, uint32_t* h) {
    // byte i of v holds codes 2i (low nibble) and 2i+1 (high nibble); byte i
    // of v >> 4 has code 2i+1 in its low nibble.
    const uint32_t v = w[b], v4 = v >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t sel = 0x0C000C00u | ((4u + i) << 16) | uint32_t(i);
        h[i] = and_or(__builtin_amdgcn_perm(v4, v, sel), 0x000F000Fu, kMagic2);
    }
}

template <>
__device__ __forceinline__ void decode_block_nat<8>(const uint32_t* w, int b, uint32_t* h) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t v = w[2 * b + (i >> 1)];
        const uint32_t j = 2u * (i & 1);
        const uint32_t sel = 0x0C000C00u | ((j + 1u) << 16) | j;
        h[i] = __builtin_amdgcn_perm(v, v, sel) | kMagic2;
    }
}

template <>
__device__ __forceinline__ void decode_block_nat<2>(const uint32_t* w, int b, uint32_t* h) {
    // block b is the 16 bits at offset 16*(b&1) of word b>>1; code pair i is
    // nibble i of the block.  Byte j of v >> 2 holds code 2i+1 where byte j
    // of v holds code 2i.
    const uint32_t v = w[b >> 1], v2 = v >> 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t j = 2u * (b & 1) + (i >> 1);
        const uint32_t sel = 0x0C000C00u | ((4u + j) << 16) | j;
        const uint32_t t = __builtin_amdgcn_perm(v2, v, sel) >> (4 * (i & 1));
        h[i] = and_or(t, 0x00030003u, kMagic2);
    }
}

template <>
__device__ __forceinline__ void decode_block_nat<3>(const uint32_t* w, int b, uint32_t* h) {
    uint32_t v;
    if (b == 0) v = w[0] & 0x00FFFFFFu;
    else if (b == 1) v = __builtin_amdgcn_alignbit(w[1], w[0], 24) & 0x00FFFFFFu;
    else if (b == 2) v = __builtin_amdgcn_alignbit(w[2], w[1], 16) & 0x00FFFFFFu;
    else v = w[2] >> 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = __builtin_amdgcn_ubfe(v, 6 * i, 3);
        const uint32_t hi = __builtin_amdgcn_ubfe(v, 6 * i + 3, 3);
        h[i] = (lo | (hi << 16)) | kMagic2;
    }
}

// Group of a 32-code chunk, cg / (group_size / 32), by multiply-shift with a
// magic number from group_magic() on the host: exact for cg < 2^24 and free
// of branches (a branch around it would make the compiler drain every load
// in flight at the join).
struct GroupDiv {
    uint32_t mul;
    uint32_t shift;
    int chunks;  // d, the divisor
};

__device__ __forceinline__ int chunk_group(int cg, GroupDiv gd) {
    return int((uint64_t(uint32_t(cg)) * gd.mul) >> gd.shift);
}

// Group constants as fp16 pairs: zz = (1024 + z, 1024 + z), ss = (s, s).
__device__ __forceinline__ uint32_t zero_pair(uint32_t z) {
    const uint32_t hz = 0x6400u | z;
    return hz | (hz << 16);
}
__device__ __forceinline__ uint32_t scale_pair(uint16_t s) {
    return uint32_t(s) | (uint32_t(s) << 16);
}

// Dequantize one decoded pair: fp16((q - z) * s) for both halves.  The
// subtraction is exact; the multiply rounds once (round to nearest even).
__device__ __forceinline__ h2 dequant_pair(uint32_t hq, uint32_t zz, uint32_t ss) {
    const h2 d = as_h2(hq) - as_h2(zz);
    return d * as_h2(ss);
}

// Activation staging order inside an 8-element block: element i goes to
// position 2i (i < 4) or 2(i - 4) + 1 (i >= 4), matching decode_chunk pairs.
__host__ __device__ __forceinline__ int stage_pos(int i) { return (i < 4) ? 2 * i : 2 * (i - 4) + 1; }

// Permute 8 fp16 values (as four 32-bit words, natural order) into staging
// order: out pair i = (x_i, x_{i+4}).
__device__ __forceinline__ u4 stage_block(u4 v) {
    u4 o;
    // x0,x1 in v.x; x2,x3 in v.y; x4,x5 in v.z; x6,x7 in v.w
    o.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);  // (x0, x4)
    o.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);  // (x1, x5)
    o.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);  // (x2, x6)
    o.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);  // (x3, x7)
    return o;
}

}  // namespace wq

// Host-side helpers shared by the API translation units.
namespace wqh {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool bits_ok(int bits) { return bits == 2 || bits == 3 || bits == 4 || bits == 8; }

// Resolve group_size (-1 = all of K); returns 0 if invalid.
inline int resolve_group(int K, int group_size) {
    if (group_size == -1) return K;
    if (group_size <= 0 || group_size % 32 != 0 || K % group_size != 0) return 0;
    return group_size;
}

// Host side of chunk_group.  For d = group_size / 32 chunks per group, take
// s = 24 + ceil(log2 d) and mul = ceil(2^s / d).  Then for n < 2^24,
// n * mul / 2^s = n / d + err with 0 <= err < n / 2^s < 1 / d, which never
// reaches the next integer, so the floor is exactly n / d.
inline wq::GroupDiv group_magic(int gs) {
    const uint64_t d = uint64_t(gs / 32);
    uint32_t lg = 0;
    while ((uint64_t(1) << lg) < d) ++lg;
    const uint32_t sh = 24 + lg;
    const uint64_t mul = ((uint64_t(1) << sh) + d - 1) / d;
    return wq::GroupDiv{uint32_t(mul), sh, int(d)};
}

inline wq_status hip_status(hipError_t e) { return e == hipSuccess ? WQ_OK : WQ_ERR_HIP; }

inline wq_status launch_status() { return hip_status(hipGetLastError()); }

}  // namespace wqh
