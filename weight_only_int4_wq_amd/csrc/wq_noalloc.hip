// wq_linear_noalloc: the batch-size dispatch of wq_linear with its scratch
// memory (the act-order activation gather and the split-K fp32 partials of
// the matrix-core GEMM, the K-slab partials of the decode kernel) in a
// static device array instead of a caller workspace, for callers that
// cannot allocate device memory.
//
// The array `scratch` is a file-scope __device__ variable: each GPU the
// library runs on holds its own copy, at its own address, from the first
// use until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in symbol); on the first call on a
// device the entry point looks up that device's address with
// hipGetSymbolAddress, keeps it, and passes that pointer as the workspace.
// Nothing here allocates: no hipMalloc, hipFree or allocating library call.
#include <mutex>

#include "wq_common.h"

namespace {

constexpr size_t kScratchBytes = size_t(WQ_NOALLOC_SCRATCH_BYTES);
static_assert(kScratchBytes % 256 == 0, "scratch size keeps 256-byte alignment");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (the current device);
// nullptr if the lookup fails.
void* device_scratch(int dev) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

// Bytes of the act-order gather, the one scratch part that cannot shrink.
size_t gather_need(int32_t M, int32_t K, const int32_t* perm) {
    if (!perm) return 0;
    return (size_t(M) * size_t(K) * 2 + 255) & ~size_t(255);
}

}  // namespace

namespace wqh {
bool linear_uses_gemv(int M, int K, bool act_order);
}

extern "C" wq_status wq_linear_noalloc(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                                       const uint8_t* zeros, const int32_t* perm, uint16_t* y, int32_t M, int32_t N,
                                       int32_t K, int32_t bits, int32_t group_size, void* stream) {
    const bool decode = wqh::linear_uses_gemv(M, K, perm != nullptr);
    if (decode && perm)  // the act-order decode kernel uses no scratch
        return wq_linear(x, packed, scales, zeros, perm, y, M, N, K, bits, group_size, nullptr, 0, stream);
    if (!decode && M > 0 && K > 0 && gather_need(M, K, perm) > kScratchBytes) return WQ_ERR_TOO_LARGE;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return WQ_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return WQ_ERR_UNSUPPORTED;
    void* ws = device_scratch(dev);
    if (!ws) return WQ_ERR_HIP;
    // the GEMM's split-K part takes what the gather leaves (with less room
    // it splits K fewer ways); the decode kernel puts its K-slab partials
    // there (with too little room each block walks the slabs); either way
    // the same result up to fp32 summation order
    return wq_linear(x, packed, scales, zeros, perm, y, M, N, K, bits, group_size, ws, kScratchBytes, stream);
}
