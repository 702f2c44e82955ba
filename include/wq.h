/*
 * wq.h - C ABI of libwq: weight-only quantized linear layers on gfx950.
 *
 * The layer computes y = x . dequant(Wq)^T with fp16 activations x [M][K],
 * b-bit weight codes (b in {2,3,4,8}) packed into 32-bit words, and one fp16
 * scale s and one integer zero-point z per (group of input channels, output
 * column); a code q dequantizes to (q - z) * s.  Sources: 2/3/4/8-bit codes,
 * per-group scales and zero-points with group size typically 128, optional
 * desc_act ("AutoGPTQ vs The Stack v2", first capability paragraph); weights
 * stay packed and are dequantized on the fly inside fused GEMM (batch) and
 * GEMV (single token) kernels chosen by batch size ("AutoAWQ vs The Stack
 * v2" and "AutoAWQ vs Unsloth", the WQLinear_* paragraphs).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - fp16 values travel as uint16_t bit patterns (IEEE binary16).
 *  - Every array argument is a DEVICE pointer to caller-owned, contiguous,
 *    row-major memory (last index fastest).  Inputs and outputs must not
 *    overlap unless an entry point says so.  The library allocates no device
 *    memory and keeps no state between calls; it is thread-safe.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    All work is enqueued asynchronously on it, except where stated.
 *  - Shapes: K = input channels (a multiple of 32), N = output columns,
 *    M = activation rows.  In wq_scale_act, wq_gemv, wq_gemm and wq_linear
 *    M = 0 or N = 0 is an empty problem: the call succeeds and does nothing.
 *    group_size is a multiple of 32 dividing K, or -1 for one group spanning
 *    all of K (one scale per output column).
 *    G = K / group_size groups (G = 1 for -1).
 *  - Packed weights: uint32 [N][K*bits/32].  Row n is a little-endian
 *    bitstream: packed column k' occupies bits [k'*bits, k'*bits + bits)
 *    counted from the least significant bit of the row's first word; a field
 *    that crosses a word boundary continues in the low bits of the next word.
 *  - Act-order (desc_act): g_idx[k] (int32 [K]) names the group of original
 *    input channel k.  Groups must all hold exactly group_size channels.
 *    Packing stores channels in the order perm = stable sort of k by
 *    g_idx[k]: packed column k' holds original channel perm[k'] and belongs
 *    to group k' / group_size.  Kernels take perm (int32 [K]) and read
 *    x[m][perm[k']]; perm = NULL means the identity (contiguous groups).
 *  - scales: fp16 [N][G]; zeros: uint8 [N][G], or NULL for the symmetric
 *    zero-point 2^(bits-1).
 *  - Errors: every argument is checked on the host before any device work;
 *    a failed check returns a status and enqueues nothing.  No entry point
 *    throws or aborts.  WQ_ERR_HIP reports a failed HIP call (launch or
 *    copy); the stream's earlier work is unaffected.
 *  - Alignment: x, y, packed, perm and workspace pointers must be 16-byte
 *    aligned.
 */
#ifndef WQ_H
#define WQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    WQ_OK = 0,
    WQ_ERR_ARG = 1,          /* null/misaligned pointer, bad shape or group map */
    WQ_ERR_UNSUPPORTED = 2,  /* bit width or M outside what the kernel handles  */
    WQ_ERR_HIP = 3,          /* a HIP runtime call failed                        */
    WQ_ERR_TOO_LARGE = 4     /* needs more than wq_linear_noalloc's static scratch */
} wq_status;

/* Static, NUL-terminated description of a status code. */
const char* wq_status_str(wq_status s);

/* Library version as "major.minor.patch". */
const char* wq_version(void);

/* ---------------------------------------------------------------- set-up --
 * Round-to-nearest group quantization of fp16 weights w [N][K] (the
 * baseline quantizer of "GPTQ, AWQ and the rules of post-training
 * quantization", section "The problem both methods solve"; group scales and
 * zero-points as in "AutoGPTQ vs The Stack v2").  For every output column n
 * and group j, over the group's member channels:
 *   asymmetric (symmetric = 0): s32 = (max - min) / (2^bits - 1) in fp32;
 *   symmetric  (symmetric = 1): s32 = 2 * max|w| / (2^bits - 1) in fp32;
 *   s = fp16(s32) (round to nearest even), 2^-14 if that is zero;
 *   z = clip(rint(-min / s), 0, 2^bits - 1) (asymmetric) or 2^(bits-1);
 *   q = clip(rint(w / s) + z, 0, 2^bits - 1), IEEE fp32 division,
 *   ties to even.
 * perm (nullable, int32 [K]): group j is channels perm[j*gs .. j*gs+gs-1];
 * NULL means channels j*gs .. j*gs+gs-1.
 * Outputs: codes uint8 [N][K] in original channel order, scales fp16 [N][G],
 * zeros uint8 [N][G] (must be NULL when symmetric, non-NULL otherwise).
 */
wq_status wq_quantize_rtn(const uint16_t* w, const int32_t* perm, int32_t N, int32_t K,
                          int32_t bits, int32_t group_size, int32_t symmetric,
                          uint8_t* codes, uint16_t* scales, uint8_t* zeros, void* stream);

/* AWQ per-input-channel scale ("GPTQ, AWQ and the rules of post-training
 * quantization", section "AWQ: find the one percent that matters"):
 * a_k = mean over the M rows of |x[m][k]| in float64, s_k = a_k^alpha
 * (alpha = 0.5 is an exact square root), s_out[k] = fp16(s_k) with one
 * float64 -> fp16 round-to-nearest-even; 2^-14 if that is zero.
 * x fp16 [M][K] -> s_out fp16 [K].  alpha must lie in [0, 1]. */
wq_status wq_awq_scales(const uint16_t* x, int32_t M, int32_t K, double alpha,
                        uint16_t* s_out, void* stream);

/* AWQ fold: w_out[n][k] = fp16(fp32(w[n][k]) * fp32(s[k])) - input channel
 * k of the weights multiplied by s_k (the weight side of AWQ's equivalent
 * rescaling, "GPTQ, AWQ and the rules of post-training quantization",
 * section "AWQ: find the one percent that matters").  w_out may equal w (in
 * place).  Asynchronous; WQ_ERR_ARG for null or misaligned pointers. */
wq_status wq_awq_fold(const uint16_t* w, const uint16_t* s, int32_t N, int32_t K,
                      uint16_t* w_out, void* stream);

/* AWQ's search for the scaling exponent ("GPTQ, AWQ and the rules of
 * post-training quantization", section "AWQ: find the one percent that
 * matters": s = (mean |x|)^alpha per input channel, alpha from a grid of
 * 20 points on [0, 1]).  For alpha_i = i / (n_grid - 1), i = 0..n_grid-1:
 * s = wq_awq_scales(x, alpha_i), W' = wq_awq_fold(w, s),
 * x' = wq_scale_act(x, s), W' RTN-quantized (wq_quantize_rtn, bits,
 * group_size, symmetric) and packed, and
 *   losses[i] = sum over m, n of (x' . dequant(W')^T - x . w^T)[m][n]^2,
 * each product accumulated in fp32 by the matrix cores, the squares summed
 * in float64 in a fixed order (deterministic).  *best (nullable) = the first
 * index of the smallest loss.
 * x fp16 [M][K] (calibration activations), w fp16 [N][K]; losses: HOST
 * memory, n_grid doubles; workspace: device memory of at least
 * wq_awq_search_workspace_size(...) bytes, 16-byte aligned.  2 <= n_grid
 * <= 4096; group_size as for wq_quantize_rtn (-1 = one group per row).
 * Set-up time: this call SYNCHRONIZES `stream` (it copies the losses back).
 * Returns WQ_ERR_ARG for null/misaligned pointers, bad sizes or a short
 * workspace, WQ_ERR_UNSUPPORTED for other bit widths. */
wq_status wq_awq_search(const uint16_t* x, const uint16_t* w, int32_t M, int32_t N, int32_t K,
                        int32_t bits, int32_t group_size, int32_t symmetric, int32_t n_grid,
                        double* losses, int32_t* best, void* workspace, size_t workspace_bytes,
                        void* stream);

/* Bytes of device workspace wq_awq_search needs (0 for invalid arguments). */
size_t wq_awq_search_workspace_size(int32_t M, int32_t N, int32_t K, int32_t bits,
                                    int32_t group_size, int32_t n_grid);

/* AWQ's clipping-threshold search ("AutoAWQ vs The Stack v2", paragraph on
 * per-channel scaling factors and clipping thresholds: a threshold per group
 * computed from the calibration activations, symmetric clipping).  For every
 * output row n, group g and ratio r_i = fp32(1 - i / n_grid), i = 0 ..
 * n_ratios - 1 (AWQ: n_grid = 20, n_ratios = 10, r = 1 .. 0.55):
 *   t = fp16(r_i * max over the group of |w[n][k]|)  (fp32 multiply),
 *   w_c = clip(w, -t, t), w_hat = w_c RTN-quantized and dequantized with
 *   wq_quantize_rtn's rule (bits, symmetric; the group as one RTN group),
 *   loss[n][g][i] = sum over m of (sum over k in g of x[m][k] (w - w_hat)[n][k])^2,
 * with w - w_hat rounded to fp16 and the products accumulated in fp32 by
 * the matrix cores; best[n][g] = the first index of the smallest loss, and
 * w_out = w clipped at each group's best threshold (fp16).
 * x fp16 [M][K] (calibration activations, M >= 1), w fp16 [N][K], w_out
 * fp16 [N][K] (may equal w); best int32 [N][G] and losses fp32
 * [N][G][n_ratios] are optional outputs (NULL to skip).  group_size: 32,
 * 64, 128 or 256 (or -1 with K one of these); 1 <= n_ratios <= n_grid,
 * n_ratios <= 1024.  x, w and w_out 16-byte aligned.  Asynchronous on
 * `stream`.  Returns WQ_ERR_ARG for null/misaligned pointers or bad sizes,
 * WQ_ERR_UNSUPPORTED for other bit widths or group sizes. */
wq_status wq_awq_clip(const uint16_t* x, const uint16_t* w, int32_t M, int32_t N, int32_t K,
                      int32_t bits, int32_t group_size, int32_t symmetric, int32_t n_grid,
                      int32_t n_ratios, uint16_t* w_out, int32_t* best, float* losses,
                      void* stream);

/* GPTQ ("GPTQ, AWQ and the rules of post-training quantization", section
 * "GPTQ: pay for the error with the other weights"): quantize w fp16 [N][K]
 * one input column at a time in index order, compensating each column's
 * rounding error on the columns not yet quantized.  H = x^T x (fp32 sums of
 * exact fp16 products); a channel with H[k][k] = 0 gets H[k][k] = 1 and a
 * zero weight column; H += damp * mean(diag H) * I; U = the upper Cholesky
 * factor of H^-1.  For column i: at the first column of a group, scale and
 * zero by wq_quantize_rtn's rule from the group's running weights; the
 * column's codes and w_hat by that rule; err = (w - w_hat) / U[i][i]; the
 * later columns -= err * U[i][later], applied in blocks of 64 columns.
 * All in fp32 (the float64 reference agrees in error, not bit for bit).
 * x fp16 [M][K] (calibration activations, M a multiple of 32); outputs as
 * wq_quantize_rtn's: codes uint8 [N][K], scales fp16 [N][G], zeros uint8
 * [N][G] (NULL when symmetric, required otherwise), ready for wq_pack.
 * act_order (desc_act, "AutoGPTQ vs The Stack v2", first capability
 * paragraph): the columns are processed in descending order of the Hessian
 * diagonal (after the dead-channel rule, before damping; ties by channel
 * index), groups are formed in that order, and g_idx int32 [K] (required
 * with act_order, ignored otherwise) receives each channel's group, the
 * group map wq_act_order_perm and wq_pack take; codes stay in channel order.
 * group_size: -1 (one group per row, any K) or a multiple of 32 dividing K
 * that divides 64 or is a multiple of 64.  0 <= damp < 1 (0.01 is usual).
 * workspace: device memory of at least wq_gptq_workspace_size(M, N, K)
 * bytes, 16-byte aligned (about 5 K^2 floats plus 5 N*K bytes); codes 16-byte
 * aligned.  The workspace must be ordinary (coarse-grained) device memory,
 * as hipMalloc returns: the lazy updates add into it with floating-point
 * atomics, which fine-grained or host memory does not support.
 * Asynchronous on `stream`.  Returns WQ_ERR_ARG for null/misaligned
 * pointers, bad sizes or a short workspace, WQ_ERR_UNSUPPORTED for other
 * bit widths. */
wq_status wq_gptq_quantize(const uint16_t* x, const uint16_t* w, int32_t M, int32_t N, int32_t K,
                           int32_t bits, int32_t group_size, int32_t symmetric, double damp,
                           int32_t act_order, uint8_t* codes, uint16_t* scales, uint8_t* zeros,
                           int32_t* g_idx, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace wq_gptq_quantize needs (0 for invalid sizes). */
size_t wq_gptq_workspace_size(int32_t M, int32_t N, int32_t K);

/* Act-order packing order (desc_act: groups formed in a permuted channel
 * order, "AutoGPTQ vs The Stack v2", first capability paragraph):
 * perm = stable sort of k by g_idx[k].  Checks that
 * every g_idx lies in [0, K/group_size) and every group holds exactly
 * group_size channels; returns WQ_ERR_ARG otherwise.  This call SYNCHRONIZES
 * `stream`: it copies g_idx and the computed perm back to the host to check
 * them. */
wq_status wq_act_order_perm(const int32_t* g_idx, int32_t K, int32_t group_size,
                            int32_t* perm, void* stream);

/* Pack codes uint8 [N][K] (original channel order, each < 2^bits; higher bits
 * are ignored) into packed uint32 [N][K*bits/32] (weights stay packed in
 * memory at 2/3/4/8 bits: "AutoGPTQ vs The Stack v2", first capability
 * paragraph; "AutoAWQ vs The Stack v2", WQLinear_* paragraph).  With g_idx
 * (nullable) the
 * packing order is first computed into perm (int32 [K], caller-allocated,
 * required when g_idx is given) as by wq_act_order_perm, and this call then
 * synchronizes `stream`; without g_idx, perm is ignored and the call is
 * asynchronous. */
wq_status wq_pack(const uint8_t* codes, const int32_t* g_idx, int32_t K, int32_t N,
                  int32_t bits, int32_t group_size, uint32_t* packed, int32_t* perm,
                  void* stream);

/* Inverse of wq_pack: codes uint8 [N][K] in original channel order (the
 * unpack step of the on-the-fly dequantization, "AutoAWQ vs The Stack v2",
 * WQLinear_* paragraph).  perm: as returned by wq_pack (NULL without
 * act-order).  Asynchronous; WQ_ERR_ARG for null or misaligned pointers or
 * bad sizes, WQ_ERR_UNSUPPORTED for other bit widths. */
wq_status wq_unpack(const uint32_t* packed, const int32_t* perm, int32_t K, int32_t N,
                    int32_t bits, uint8_t* codes, void* stream);

/* Materialize the dequantized weights w fp16 [N][K] (original channel
 * order): w[n][perm[k']] = fp16((q - z) * s), q the code at packed column k',
 * with one round-to-nearest-even (the group-wise affine dequantization of
 * "GPTQ, AWQ and the rules of post-training quantization", section "The
 * problem both methods solve").  Same dequantization arithmetic as the
 * GEMV/GEMM kernels; used to check it bit for bit.  Asynchronous;
 * WQ_ERR_ARG / WQ_ERR_UNSUPPORTED as wq_unpack. */
wq_status wq_dequant(const uint32_t* packed, const uint16_t* scales, const uint8_t* zeros,
                     const int32_t* perm, int32_t K, int32_t N, int32_t bits,
                     int32_t group_size, uint16_t* w, void* stream);

/* ------------------------------------------------------------- hot path --
 * AWQ input scaling: x_out[m][k] = fp16(fp32(x[m][k]) / fp32(s[k])), IEEE
 * fp32 division then one round-to-nearest-even (the activation side of the
 * AWQ rescaling: the weights' input channel k is multiplied by s_k, the
 * matching activation divided by it, "GPTQ, AWQ and the rules of
 * post-training quantization", section "AWQ: find the one percent that
 * matters").  x, s, x_out fp16, 16-byte aligned; x_out may equal x.
 * Asynchronous; WQ_ERR_ARG for null or misaligned pointers or bad sizes. */
wq_status wq_scale_act(const uint16_t* x, const uint16_t* s, int32_t M, int32_t K,
                       uint16_t* x_out, void* stream);

/* Bytes of device workspace wq_gemv, wq_gemm and wq_linear use for these
 * arguments on the current device (the largest of their needs); 0 when
 * none.  wq_gemm layout: with act-order (has_perm != 0) the gathered
 * activations x[:, perm], M*K fp16 values rounded up to 256 bytes; then,
 * when the launch has too few output tiles to fill the GPU, fp32 partial
 * outputs of a K split (splits*M*N floats; the split count is chosen on the
 * host from the shape and the number of compute units).  wq_gemv at
 * 2 <= M <= 32 without act-order, when M rows of K activations do not fit
 * in LDS at once: fp32 partial outputs of its K slabs (slabs*M*N floats,
 * sized here for the group size with the most groups).  The act-order part
 * is required; the split parts are optional: with less workspace the
 * kernels do not split K across blocks (same result up to fp32 summation
 * order, slower).  Returns 0 for non-positive sizes or unsupported bit
 * widths. */
size_t wq_workspace_size(int32_t M, int32_t N, int32_t K, int32_t bits, int32_t has_perm);

/* y fp16 [M][N] = x fp16 [M][K] . dequant(packed)^T with fp32 accumulation
 * and one rounding of the sum to fp16: the weight-only quantized linear
 * layer, weights kept packed and dequantized on the fly, a GEMV kernel for
 * single-token decode and a GEMM kernel for batches chosen by batch size
 * ("AutoAWQ vs The Stack v2" and "AutoAWQ vs Unsloth", WQLinear_*
 * paragraphs).
 *
 * wq_gemv: the decode kernels for M <= 16, and for 17 <= M <= 32 without
 *   act-order and with K >= 256 (returns WQ_ERR_UNSUPPORTED otherwise).
 *   M = 1 (and act-order layers): streams the packed words with
 *   128-bit loads, unpacks in registers, accumulates with fp16-pair dot
 *   products into fp32 and reduces the split-K partial sums across the
 *   wavefront.  2 <= M <= 32 without act-order: one pass over the weights
 *   with the products on fp16 matrix-core instructions (16 x 16 x 32; two
 *   per weight fragment from 17 rows), the
 *   activations staged in LDS; when M rows of K do not fit, K is cut into
 *   slabs, one group of blocks per slab with the workspace (then a second
 *   kernel adds the slabs' fp32 partials in slab order), or each block
 *   walking the slabs in turn without it.
 * wq_gemm: the prefill kernel for any M: dequantizes weight tiles to
 *   fp16 and feeds fp16 matrix-core (MFMA) instructions with fp32
 *   accumulators.
 * wq_linear: picks wq_gemv for M <= wq_gemv_max_m() (16; with act-order,
 *   M <= 4), and for 17 <= M <= 24 without act-order when M * K <= 24 * 8192
 *   and K >= 256, and wq_gemm otherwise (the batch-size dispatch).
 *
 * workspace: device memory of wq_workspace_size(M, N, K, bits, perm != NULL)
 * bytes (16-byte aligned), or NULL when that size is 0; WQ_ERR_ARG if
 * act-order needs it and it is missing or short, or if it is misaligned.  Split-K partials are
 * summed in a fixed order, so results are deterministic.  Calls that share
 * a workspace must be ordered on one stream.  y must not overlap any input
 * or the workspace. */
wq_status wq_gemv(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                  const uint8_t* zeros, const int32_t* perm, uint16_t* y,
                  int32_t M, int32_t N, int32_t K, int32_t bits, int32_t group_size,
                  void* workspace, size_t workspace_bytes, void* stream);

wq_status wq_gemm(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                  const uint8_t* zeros, const int32_t* perm, uint16_t* y,
                  int32_t M, int32_t N, int32_t K, int32_t bits, int32_t group_size,
                  void* workspace, size_t workspace_bytes, void* stream);

wq_status wq_linear(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                    const uint8_t* zeros, const int32_t* perm, uint16_t* y,
                    int32_t M, int32_t N, int32_t K, int32_t bits, int32_t group_size,
                    void* workspace, size_t workspace_bytes, void* stream);

/* wq_linear for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same dispatch and kernels as wq_linear, with their scratch (the
 * GEMM's act-order activation gather, then split-K fp32 partials; the
 * decode kernel's K-slab fp32 partials) in a static device array of
 * WQ_NOALLOC_SCRATCH_BYTES bytes inside the library instead of a caller
 * workspace.  Each GPU holds its own copy of the array from the
 * first call on it until the process ends; the call looks up the current
 * device's copy (hipGetSymbolAddress) on its first use there and allocates
 * nothing.  The array keeps the last call's contents and nothing in it
 * needs clearing (every byte read is first written by the same call).
 * Every call on one GPU shares the array, so calls on one GPU must be
 * ordered (one stream, or synchronized): overlapping calls race.  The
 * current device must be the stream's device.  Returns WQ_ERR_TOO_LARGE
 * when act-order needs a gather of more than WQ_NOALLOC_SCRATCH_BYTES
 * (M*K*2 bytes, rounded up to 256); with too little room for the split-K
 * partials the GEMM splits K fewer ways, and the decode kernel walks its
 * K-slabs in each block.  Otherwise as wq_linear. */
#define WQ_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)
wq_status wq_linear_noalloc(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                            const uint8_t* zeros, const int32_t* perm, uint16_t* y,
                            int32_t M, int32_t N, int32_t K, int32_t bits, int32_t group_size,
                            void* stream);

/* Fused gate/up projection with its activation, for decode batches
 * (1 <= M <= 4): the N rows of packed/scales/zeros are a gate projection
 * (rows 0 .. N/2-1) stacked over an up projection (rows N/2 .. N-1), and
 *   y fp16 [M][N/2]: y[m][j] = fp16(silu(g) * u),  silu(v) = v / (1 + e^-v),
 * with g, u the fp32-accumulated rows j and j + N/2 of x . dequant(packed)^T.
 * One launch of the decode GEMV with a fused epilogue instead of a GEMV
 * writing both halves plus an elementwise pass ("AutoAWQ vs The Stack v2",
 * paragraph on fused transformer blocks: fewer launches, no intermediate
 * tensor; SiLU as the gate activation is the gated MLP of LLaMA-shaped
 * layers).  Same argument rules as wq_gemv; N must be even (WQ_ERR_ARG),
 * WQ_ERR_UNSUPPORTED for M > 4 or when x's rows do not fit the kernel's
 * 64 KB activation stage (K up to about 16k at M = 1). */
wq_status wq_gemv_silu_mul(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                           const uint8_t* zeros, const int32_t* perm, uint16_t* y,
                           int32_t M, int32_t N, int32_t K, int32_t bits, int32_t group_size,
                           void* stream);

/* The decode GEMV with its neighbours fused (fusing a block's operations
 * into single kernels saves launches and intermediate tensors, "AutoAWQ vs
 * The Stack v2", paragraph on fused attention and transformer blocks).  act_scale (nullable, fp16 [K], 16-byte aligned): the AWQ
 * activation scaling x' = fp16(fp32(x) / fp32(act_scale[k])), done while the
 * activations are staged, bit-identical to wq_scale_act followed by
 * wq_gemv.  bias (nullable, fp16 [N]): added to the fp32 sum of each output
 * before its rounding.  silu = 0: y fp16 [M][N] = x' . dequant(Wq)^T + bias.
 * silu = 1: the stacked gate/up layout of wq_gemv_silu_mul (N even), y fp16
 * [M][N/2] = silu(g + bias[j]) * (u + bias[j + N/2]).  Other arguments as
 * wq_gemv.  silu = 0: 1 <= M <= 16 (act-order: M <= 4), and up to 32
 * without act-order for K >= 256 (the matrix-core kernel); silu = 1:
 * 1 <= M <= 4 and fp16 x of K within the 64 KB staging budget (K <= 16384
 * at M = 1); else WQ_ERR_UNSUPPORTED. */
wq_status wq_gemv_ex(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                     const uint8_t* zeros, const int32_t* perm, const uint16_t* act_scale,
                     const uint16_t* bias, uint16_t* y, int32_t M, int32_t N, int32_t K,
                     int32_t bits, int32_t group_size, int32_t silu, void* stream);

/* Measurement reference, not part of the layer: reads `bytes` bytes (a
 * multiple of 16) from device memory src (16-byte aligned) with coalesced
 * 16-byte non-temporal loads, grid-stride, and writes to the device word
 * sink only in the astronomically unlikely case that the XOR of the data
 * equals a fixed constant (so the loads cannot be optimized away).  It is
 * the achievable streaming-read bandwidth the decode kernels are compared
 * with, launched and timed the same way.  WQ_ERR_ARG for null or misaligned
 * pointers or a size that is not a multiple of 16; asynchronous. */
wq_status wq_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Largest M that wq_linear always sends to wq_gemv (16; layers with
 * act-order go to wq_gemm from M = 5; 17 <= M <= 24 go to wq_gemv too when
 * M * K <= 24 * 8192, K >= 256 and there is no act-order). */
int32_t wq_gemv_max_m(void);

#ifdef __cplusplus
}
#endif

#endif /* WQ_H */
