// Status strings, shared argument checks and the batch-size dispatch.
//
// Dispatch by batch size: a GEMV kernel for single-token decode and a GEMM
// kernel for batches, picked automatically ("AutoAWQ vs Unsloth", WQLinear_*
// paragraph; "AutoAWQ vs The Stack v2", WQLinear_* paragraph).
#include "wq_common.h"

namespace {
// Largest activation row count sent to wq_gemv by wq_linear.  From M = 2 the
// decode path runs on the skinny matrix-core kernel, which streams the
// weights once for up to 16 rows.  Measured at M = 16 (MI355X, 4-bit, group
// 128): 6.3-17.5 us on the Llama-7B decode projections against 11.2-26.1 us
// for the tiled GEMM, 20.8-54.1 us against 28.0-64.6 us on the Llama-70B
// ones; at M = 4 the gap is wider.  Act-order layers take the skinny kernel's
// vector-ALU fallback, whose cost grows with M, so from M = 5 they go to the
// GEMM, whose activation copy applies the gather.
#ifndef WQ_GEMV_MAX_M
#define WQ_GEMV_MAX_M 16
#endif
constexpr int kGemvMaxM = WQ_GEMV_MAX_M;
constexpr int kGemvMaxMActOrder = 4;
// From 17 rows the skinny kernel feeds every decoded weight fragment to two
// matrix instructions and reads twice the activation fragments from LDS,
// and M rows of K activations need more K-slabs.  Measured against the
// tiled GEMM (MI355X, 4-bit, group 128, the seven Llama decode and 70B
// shapes): faster at 17 and 24 rows while M * K <= 24 * 8192 (1.02-1.32x),
// slower past that (24 x 11008: 0.94x, 17 x 28672: 0.91x) and at 32 rows on
// every shape (0.44-0.85x).
constexpr int kSkinnyWideMaxM = 24;
constexpr long long kSkinnyWideMaxMK = 24LL * 8192;
}  // namespace

namespace wqh {

bool linear_uses_gemv(int M, int K, bool act_order) {
    if (M <= (act_order ? kGemvMaxMActOrder : kGemvMaxM)) return true;
    return !act_order && M <= kSkinnyWideMaxM && K >= 256 && (long long)M * K <= kSkinnyWideMaxMK;
}

wq_status check_linear_args(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, const uint16_t* y,
                            int M, int N, int K, int bits, int group_size, int* gs_out) {
    if (M < 0 || N < 0 || K <= 0 || K % 32) return WQ_ERR_ARG;
    if (!wqh::bits_ok(bits)) return WQ_ERR_UNSUPPORTED;
    const int gs = resolve_group(K, group_size);
    if (!gs) return WQ_ERR_ARG;
    *gs_out = gs;
    if (M == 0 || N == 0) return WQ_OK;  // empty problem: no pointer is read
    if (!x || !packed || !scales || !y) return WQ_ERR_ARG;
    if (!aligned16(x) || !aligned16(packed) || !aligned16(y)) return WQ_ERR_ARG;
    *gs_out = gs;
    return WQ_OK;
}

}  // namespace wqh

extern "C" const char* wq_status_str(wq_status s) {
    switch (s) {
        case WQ_OK: return "ok";
        case WQ_ERR_ARG: return "invalid argument (null or misaligned pointer, bad shape, group size or group map)";
        case WQ_ERR_UNSUPPORTED: return "unsupported configuration (bit width or row count)";
        case WQ_ERR_HIP: return "HIP runtime call failed";
        case WQ_ERR_TOO_LARGE:
            return "problem needs more scratch memory than wq_linear_noalloc's static buffer holds "
                   "(act-order gather of M*K fp16 values over WQ_NOALLOC_SCRATCH_BYTES)";
    }
    return "unknown status";
}

extern "C" const char* wq_version(void) { return "0.1.0"; }

extern "C" int32_t wq_gemv_max_m(void) { return kGemvMaxM; }

extern "C" wq_status wq_linear(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                               const uint8_t* zeros, const int32_t* perm, uint16_t* y, int32_t M, int32_t N,
                               int32_t K, int32_t bits, int32_t group_size, void* workspace,
                               size_t workspace_bytes, void* stream) {
    if (wqh::linear_uses_gemv(M, K, perm != nullptr))
        return wq_gemv(x, packed, scales, zeros, perm, y, M, N, K, bits, group_size, workspace, workspace_bytes,
                       stream);
    return wq_gemm(x, packed, scales, zeros, perm, y, M, N, K, bits, group_size, workspace, workspace_bytes, stream);
}
