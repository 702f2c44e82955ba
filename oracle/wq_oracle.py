"""Plain, slow, obviously correct CPU oracle for weight-only quantized linear layers.

TEST INFRASTRUCTURE.  This module is the yardstick the HIP library is checked
against; it shares no code with that library and must never be imported by
it.  Only the tests, the smoke check and the CPU-baseline leg of the benchmark
use it.

What it computes, and where each step comes from:

* Round-to-nearest (RTN) group quantization of fp16 weights to b-bit codes
  with one fp16 scale and one integer zero-point per (group of input
  channels, output column).  Round-to-nearest as the baseline quantizer:
  "GPTQ, AWQ and the rules of post-training quantization", section "The
  problem both methods solve".  Per-group scales and zero-points, group size
  typically 128, bit widths 2/3/4/8 and the optional desc_act (act-order)
  group map: "AutoGPTQ vs The Stack v2", first capability paragraph (GPTQ
  quantization).  The `w_bit` / `q_group_size` parameter pair: "When to Use
  AWQ vs GPTQ", section "Practical Usage".
* AWQ equivalence rescaling: scale input channel k of the weights by s_k and
  divide the matching activation by s_k, with s_k the channel's mean
  activation magnitude raised to alpha; the layer output is unchanged in exact
  arithmetic.  "GPTQ, AWQ and the rules of post-training quantization",
  section "AWQ: find the one percent that matters".
* AWQ's search for alpha: a 20-point grid on [0, 1], each point scored by
  the squared output error of the rescaled, quantized layer against the
  original layer on the calibration activations (same section).
* AWQ's clipping-threshold search: per group, a symmetric threshold from a
  grid of shrink ratios of the group's largest magnitude, scored by the
  group's output error on the calibration activations ("AutoAWQ vs The
  Stack v2", paragraph on scaling factors and clipping thresholds).
* GPTQ: columns quantized in a fixed order, each rounding error compensated
  on the remaining columns through the upper Cholesky factor of the
  inverse Hessian of the layer's reconstruction loss ("GPTQ, AWQ and the
  rules of post-training quantization", section "GPTQ: pay for the error
  with the other weights"); optionally in act-order (descending Hessian
  diagonal, the desc_act option of "AutoGPTQ vs The Stack v2").
* Packing of codes into 32-bit words, dequantization (q - z) * s and the
  product y = x . dequant(Wq)^T (+ an optional bias; the gated form
  silu(x . Wg^T) * (x . Wu^T) of a fused epilogue).  Weights stay packed
  and are dequantized on the fly inside the product: "AutoAWQ vs The Stack v2", paragraph on the
  WQLinear_* GEMM/GEMV modules, and "AutoAWQ vs Unsloth", the matching
  paragraph.  The product is defined exactly, so the oracle writes that
  definition out in float64.

The pages fix none of the following; the reading taken for each is stated
where it is used:
  scale = (max - min) / (2^b - 1) in fp32, rounded to fp16, and the codes are
  derived from the stored fp16 scale; zero = clip(rint(-min / s), 0, 2^b - 1);
  symmetric mode uses scale = 2 * max|w| / (2^b - 1) and zero = 2^(b-1);
  rounding is IEEE round-half-to-even; a zero scale becomes 2^-14;
  little-endian LSB-first bitstream packing; act-order packs columns in the
  stable-sorted order of the group map; AWQ statistics in float64 over the
  rows of the activation batch, s rounded once to fp16.
"""

from __future__ import annotations

import numpy as np

F16 = np.float16
F32 = np.float32
F64 = np.float64

#: Bit widths the GPTQ capability lists (2/3/4/8-bit integer weights).
SUPPORTED_BITS = (2, 3, 4, 8)

#: Smallest normal fp16, used in place of a scale that rounds to zero.
_SCALE_FLOOR = F16(2.0 ** -14)


def _check_bits(bits: int) -> int:
    if bits not in SUPPORTED_BITS:
        raise ValueError(f"bits must be one of {SUPPORTED_BITS}, got {bits}")
    return (1 << bits) - 1


def group_of_channel(K: int, group_size: int, g_idx=None) -> np.ndarray:
    """Group index of every input channel k (int64 [K]).

    Without act-order, channels are grouped contiguously: g(k) = k // group_size.
    group_size == -1 means one group spanning all K channels (per-channel, i.e.
    one scale per output column).  With act-order the caller's g_idx map gives
    the group of each channel directly (GPTQ desc_act, "AutoGPTQ vs The Stack
    v2", first capability).
    """
    if g_idx is not None:
        g = np.asarray(g_idx, dtype=np.int64)
        if g.shape != (K,):
            raise ValueError("g_idx must have shape [K]")
        return g
    gs = K if group_size == -1 else group_size
    if gs <= 0 or K % gs:
        raise ValueError("group_size must divide K")
    return np.arange(K, dtype=np.int64) // gs


def act_order_perm(g_idx) -> np.ndarray:
    """Packed column order for act-order: the stable sort of k by g_idx[k].

    Column k' of the packed matrix holds original channel perm[k'], so the
    members of each group sit next to each other and the group of packed
    column k' is k' // group_size when all groups have equal size.
    """
    return np.argsort(np.asarray(g_idx, dtype=np.int64), kind="stable")


def rtn_quantize(w, bits: int, group_size: int, g_idx=None, symmetric: bool = False):
    """Round-to-nearest group quantization of fp16 weights w[N][K].

    Returns (codes uint8 [N][K] in original channel order,
             scales fp16 [N][G], zeros uint8 [N][G] or None when symmetric).

    Per (output column n, group j), over the member channels of group j:
      asymmetric: s32 = (max - min) / qmax          (fp32 subtract, fp32 divide)
      symmetric:  s32 = (2 * max|w|) / qmax         (fp32)
      s = fp16(s32), replaced by 2^-14 if it rounds to zero
      asymmetric: z = clip(rint(-min / s), 0, qmax) (fp32 divide)
      symmetric:  z = 2^(b-1)
      q = clip(rint(w / s) + z, 0, qmax)            (fp32 divide, half-even)
    """
    qmax = _check_bits(bits)
    w = np.asarray(w)
    if w.dtype != F16 or w.ndim != 2:
        raise ValueError("w must be a 2-D float16 array [N][K]")
    N, K = w.shape
    gk = group_of_channel(K, group_size, g_idx)
    G = int(gk.max()) + 1 if K else 0
    w32 = w.astype(F32)
    codes = np.zeros((N, K), dtype=np.uint8)
    scales = np.zeros((N, G), dtype=F16)
    zeros = None if symmetric else np.zeros((N, G), dtype=np.uint8)
    for j in range(G):
        members = np.nonzero(gk == j)[0]
        if members.size == 0:
            raise ValueError(f"group {j} has no members")
        wg = w32[:, members]                                   # [N][|group|]
        if symmetric:
            amax = np.max(np.abs(wg), axis=1)
            s32 = (F32(2.0) * amax) / F32(qmax)
        else:
            mn = np.min(wg, axis=1)
            mx = np.max(wg, axis=1)
            s32 = (mx - mn) / F32(qmax)
        s_h = s32.astype(F16)
        s_h[s_h == 0] = _SCALE_FLOOR
        s_f = s_h.astype(F32)
        if symmetric:
            z = np.full(N, F32(1 << (bits - 1)), dtype=F32)
        else:
            z = np.clip(np.rint((-mn) / s_f), F32(0), F32(qmax))
            zeros[:, j] = z.astype(np.uint8)
        q = np.clip(np.rint(wg / s_f[:, None]) + z[:, None], F32(0), F32(qmax))
        codes[:, members] = q.astype(np.uint8)
        scales[:, j] = s_h
    return codes, scales, zeros


def pack(codes, bits: int) -> np.ndarray:
    """Pack b-bit codes[N][K] into uint32 words[N][K*b/32].

    Convention (the pages give no layout): each row is a little-endian
    bitstream; code k occupies bits [k*b, k*b + b) counted from the least
    significant bit of word 0, and a field that crosses a word boundary
    continues in the low bits of the next word.
    """
    qmax = _check_bits(bits)
    c = np.asarray(codes)
    if c.ndim != 2:
        raise ValueError("codes must be 2-D [N][K]")
    N, K = c.shape
    if (K * bits) % 32:
        raise ValueError("K * bits must be a multiple of 32")
    if c.size and int(c.max()) > qmax:
        raise ValueError("code out of range")
    # bit plane i of code k lands on stream bit k*bits + i
    stream = np.zeros((N, K * bits), dtype=np.uint8)
    for i in range(bits):
        stream[:, i::bits] = (c >> i) & 1
    # numpy packs stream bit 8j + t into bit t of byte j (bitorder="little"),
    # and four consecutive bytes read as a little-endian uint32 form one word
    return np.packbits(stream, axis=1, bitorder="little").view("<u4").astype(np.uint32)


def unpack(packed, bits: int, K: int) -> np.ndarray:
    """Exact inverse of `pack`: uint32 words[N][K*b/32] -> uint8 codes[N][K]."""
    _check_bits(bits)
    p = np.asarray(packed, dtype=np.uint32)
    N, W = p.shape
    if W * 32 != K * bits:
        raise ValueError("packed width does not match K * bits / 32")
    stream = np.unpackbits(p.astype("<u4").view(np.uint8), axis=1, bitorder="little")
    codes = np.zeros((N, K), dtype=np.uint8)
    for i in range(bits):
        codes |= stream[:, i::bits] << i
    return codes


def _zero_matrix(zeros, bits, shape):
    if zeros is None:
        return np.full(shape, 1 << (bits - 1), dtype=np.int64)
    return np.asarray(zeros).astype(np.int64)


def dequant(codes, scales, zeros, bits: int, group_size: int, g_idx=None) -> np.ndarray:
    """w_hat[n][k] = fp16( fp32(q - z) * fp32(s) ) for the group of channel k.

    (q - z) is an exact small integer and the fp32 product of it with an fp16
    scale is exact, so there is a single round-to-nearest-even, to fp16.
    zeros=None means the symmetric zero 2^(b-1).
    """
    _check_bits(bits)
    q = np.asarray(codes).astype(np.int64)
    N, K = q.shape
    gk = group_of_channel(K, group_size, g_idx)
    s = np.asarray(scales, dtype=F16)
    z = _zero_matrix(zeros, bits, s.shape)
    diff = (q - z[:, gk]).astype(F32)
    return (diff * s[:, gk].astype(F32)).astype(F16)


def dequant_fp64_path(codes, scales, zeros, bits: int, group_size: int, g_idx=None) -> np.ndarray:
    """Second formulation of `dequant`: exact product in float64, one direct
    float64 -> fp16 rounding.  Must agree bit for bit with `dequant`."""
    q = np.asarray(codes).astype(np.int64)
    N, K = q.shape
    gk = group_of_channel(K, group_size, g_idx)
    s = np.asarray(scales, dtype=F16).astype(F64)
    z = _zero_matrix(zeros, bits, s.shape)
    return ((q - z[:, gk]).astype(F64) * s[:, gk]).astype(F16)


def awq_channel_scales(x, alpha: float = 0.5):
    """AWQ per-input-channel scale from activation statistics.

    a_k = mean over rows m of |x[m][k]| (float64), s_k = a_k ** alpha, then
    s_h = fp16(s) by one direct float64 -> fp16 rounding ("GPTQ, AWQ and the
    rules of post-training quantization", section "AWQ: find the one percent
    that matters": average activation magnitude raised to a power alpha).
    A channel whose scale rounds to zero gets 2^-14 (the pages are silent on
    dead channels).  Returns (s float64 [K], s_h fp16 [K]).
    """
    x64 = np.asarray(x, dtype=F16).astype(F64)
    a = np.mean(np.abs(x64), axis=0)
    s = np.sqrt(a) if alpha == 0.5 else np.power(a, F64(alpha))
    s_h = s.astype(F16)
    s_h[s_h == 0] = _SCALE_FLOOR
    return s, s_h


def awq_fold_weight(w, s_h) -> np.ndarray:
    """W'[n][k] = fp16( fp32(W[n][k]) * fp32(s_h[k]) ): input channel k of the
    weights is multiplied by s_k (the product of two fp16 values is exact in
    fp32, so this is one rounding)."""
    w = np.asarray(w, dtype=F16)
    s = np.asarray(s_h, dtype=F16).astype(F32)
    return (w.astype(F32) * s[None, :]).astype(F16)


def awq_scale_act(x, s_h) -> np.ndarray:
    """x'[m][k] = fp16( fp32(x[m][k]) / fp32(s_h[k]) ): the matching
    activation is divided by s_k (IEEE fp32 division, then one rounding to
    fp16)."""
    x = np.asarray(x, dtype=F16)
    s = np.asarray(s_h, dtype=F16).astype(F32)
    return (x.astype(F32) / s[None, :]).astype(F16)


def linear_ref(x, w_hat, chunk: int = 8192, bias=None) -> np.ndarray:
    """y[m][n] = sum_k x[m][k] * w_hat[n][k] (+ bias[n]) in float64 (exact
    definition of the layer output from the dequantized weights; the
    optional fp16 bias of a fused epilogue is added to the exact sum).
    Chunked over n only to bound memory."""
    x64 = np.asarray(x, dtype=F16).astype(F64)
    w = np.asarray(w_hat, dtype=F16)
    N = w.shape[0]
    y = np.empty((x64.shape[0], N), dtype=F64)
    for n0 in range(0, N, chunk):
        y[:, n0:n0 + chunk] = x64 @ w[n0:n0 + chunk].astype(F64).T
    if bias is not None:
        y += np.asarray(bias, dtype=F16).astype(F64)[None, :]
    return y


def silu_mul_ref(x, w_hat, bias=None) -> np.ndarray:
    """Fused gate/up projection with its activation, in float64.

    w_hat holds the two projections stacked, 2I rows: rows [0, I) the gate,
    rows [I, 2I) the up projection.  With g = x . W_gate^T and u = x . W_up^T
    (exact float64 sums), y = silu(g) * u, silu(v) = v / (1 + e^-v).  The
    pages describe fusing several of a block's operations into one kernel to
    cut launches and intermediate tensors ("AutoAWQ vs The Stack v2",
    paragraph on fused transformer blocks); which operations, and SiLU as
    the gate's activation, is the reading taken (the gated MLP of the
    LLaMA-shaped layers the workloads use).  An optional bias [2I] is added
    to g and u before the activation.
    """
    y = linear_ref(x, w_hat, bias=bias)
    two_i = y.shape[1]
    if two_i % 2:
        raise ValueError("the stacked gate/up weight needs an even row count")
    half = two_i // 2
    g, u = y[:, :half], y[:, half:]
    return g / (1.0 + np.exp(-g)) * u


def quantize_linear_layer(w, bits: int, group_size: int, g_idx=None, symmetric: bool = False):
    """RTN-quantize w[N][K] and pack it the way the packed format stores it.

    Returns a dict with codes (original order), scales, zeros, perm (None
    without act-order), packed words (packed column order) and w_hat (the
    dequantized fp16 weights in original channel order).
    """
    N, K = np.asarray(w).shape
    codes, scales, zeros = rtn_quantize(w, bits, group_size, g_idx, symmetric)
    perm = None
    packed_codes = codes
    if g_idx is not None:
        perm = act_order_perm(g_idx)
        packed_codes = codes[:, perm]
    return dict(
        codes=codes, scales=scales, zeros=zeros, perm=perm,
        packed=pack(packed_codes, bits),
        w_hat=dequant(codes, scales, zeros, bits, group_size, g_idx),
    )


def awq_alpha_grid(n_grid: int = 20) -> np.ndarray:
    """The AWQ exponent grid: n_grid evenly spaced points on [0, 1], both
    ends included ("GPTQ, AWQ and the rules of post-training quantization",
    section "AWQ: find the one percent that matters": a grid search of 20
    points on the interval from 0 to 1; the pages do not say whether the
    ends are included, and the plain reading of points on the closed
    interval is taken)."""
    if n_grid < 2:
        raise ValueError("the grid needs at least 2 points")
    return np.arange(n_grid, dtype=F64) / F64(n_grid - 1)


def awq_search(x, w, bits: int, group_size: int, n_grid: int = 20, symmetric: bool = False):
    """AWQ's grid search for the scaling exponent alpha (same section).

    For every alpha on awq_alpha_grid(n_grid): s_h = AWQ channel scales of
    x with that alpha, W' = W folded by s_h, x' = x divided by s_h, W'
    RTN-quantized and dequantized to w_hat', and the loss is the squared
    output error of the quantized layer against the original one,
        loss = sum over m, n of (x' . w_hat'^T - x . W^T)[m][n]^2,
    both products exact in float64 from the fp16 operands.  The pages say
    the rescaling reduces the quantization error and that alpha comes from a
    20-point search; they do not state the search objective, and the layer
    output error on the calibration activations is the reading taken.
    Returns (alphas float64 [n_grid], losses float64 [n_grid], best index =
    first minimum).
    """
    x = np.asarray(x, dtype=F16)
    w = np.asarray(w, dtype=F16)
    alphas = awq_alpha_grid(n_grid)
    y_ref = linear_ref(x, w)
    losses = np.empty(n_grid, dtype=F64)
    for i, a in enumerate(alphas):
        _, s_h = awq_channel_scales(x, float(a))
        w_f = awq_fold_weight(w, s_h)
        x_f = awq_scale_act(x, s_h)
        q = quantize_linear_layer(w_f, bits, group_size, symmetric=symmetric)
        d = linear_ref(x_f, q["w_hat"]) - y_ref
        losses[i] = np.sum(d * d)
    return alphas, losses, int(np.argmin(losses))


def awq_clip_ratios(n_grid: int = 20, n_ratios: int = 10) -> np.ndarray:
    """Shrink ratios of AWQ's clipping search: r_i = fp32(1 - i / n_grid),
    i = 0 .. n_ratios - 1 (1.0, 0.95, ..., 0.55 by default).  The pages say
    AWQ computes clipping thresholds from the calibration data and clips
    symmetrically; the grid (the published method's: shrink the group's
    largest magnitude by up to one half in steps of 1/20) is the plain
    reading taken."""
    if n_grid < 1 or not 1 <= n_ratios <= n_grid:
        raise ValueError("need 1 <= n_ratios <= n_grid")
    return np.array([1.0 - i / n_grid for i in range(n_ratios)], dtype=F32)


def awq_clip_search(x, w, bits: int, group_size: int, n_grid: int = 20, n_ratios: int = 10,
                    symmetric: bool = False):
    """AWQ's clipping-threshold search ("AutoAWQ vs The Stack v2", the
    paragraph on per-channel scaling factors and clipping thresholds: a
    threshold per weight group from the calibration activations, symmetric
    clipping).  For every output row n, group g and ratio r_i:
        t = fp16(fp32(r_i) * max over the group of |w|)   (fp32 multiply)
        w_c = clip(w, -t, t)                               (exact in fp16)
        w_hat = RTN-dequantized w_c (the group as one RTN group)
        loss[n][g][i] = sum over m of (sum over k in g of x[m][k] (w - w_hat)[n][k])^2
    in float64 from the fp16 values; best[n][g] = the first index of the
    smallest loss; w_clip = w clipped at the best threshold (fp16).
    The objective, the group's own output error on the calibration
    activations, is the reading taken where the pages name none.
    Returns dict(ratios, losses float64 [N][G][R], best int [N][G], w_clip)."""
    x = np.asarray(x, dtype=F16)
    w = np.asarray(w, dtype=F16)
    N, K = w.shape
    gs = K if group_size == -1 else int(group_size)
    if gs <= 0 or K % gs:
        raise ValueError("group_size must divide K")
    G = K // gs
    ratios = awq_clip_ratios(n_grid, n_ratios)
    X = x.astype(F64)
    losses = np.zeros((N, G, len(ratios)), dtype=F64)
    thresholds = np.zeros((N, G, len(ratios)), dtype=F16)
    for g in range(G):
        cols = slice(g * gs, (g + 1) * gs)
        wg = w[:, cols]
        amax = np.max(np.abs(wg.astype(F32)), axis=1)
        for i, r in enumerate(ratios):
            t = (r * amax).astype(F16)
            thresholds[:, g, i] = t
            tf = t.astype(F32)[:, None]
            wc = np.clip(wg.astype(F32), -tf, tf).astype(F16)
            codes, scales, zeros = rtn_quantize(wc, bits, -1, symmetric=symmetric)
            w_hat = dequant(codes, scales, zeros, bits, -1)
            p = X[:, cols] @ (wg.astype(F64) - w_hat.astype(F64)).T       # [M][N]
            losses[:, g, i] = np.sum(p * p, axis=0)
    best = np.argmin(losses, axis=2)
    w_clip = w.copy()
    for g in range(G):
        cols = slice(g * gs, (g + 1) * gs)
        t = thresholds[np.arange(N), g, best[:, g]].astype(F32)[:, None]
        w_clip[:, cols] = np.clip(w[:, cols].astype(F32), -t, t).astype(F16)
    return dict(ratios=ratios, losses=losses, best=best, w_clip=w_clip)


def _group_params_f32(wg, bits: int, symmetric: bool):
    """The RTN rule of rtn_quantize for one group per row, on float32 values
    wg [N][n]: returns (s_h fp16 [N], z float32 [N])."""
    qmax = F32((1 << bits) - 1)
    if symmetric:
        s32 = (F32(2.0) * np.max(np.abs(wg), axis=1)) / qmax
    else:
        mn = np.min(wg, axis=1)
        s32 = (np.max(wg, axis=1) - mn) / qmax
    s_h = s32.astype(F16)
    s_h[s_h == 0] = _SCALE_FLOOR
    if symmetric:
        z = np.full(wg.shape[0], F32(1 << (bits - 1)), dtype=F32)
    else:
        z = np.clip(np.rint((-mn) / s_h.astype(F32)), F32(0), qmax)
    return s_h, z


def gptq_quantize(w, x, bits: int, group_size: int, symmetric: bool = False, damp: float = 0.01,
                  act_order: bool = False):
    """GPTQ ("GPTQ, AWQ and the rules of post-training quantization",
    section "GPTQ: pay for the error with the other weights"): columns are
    quantized one at a time in a fixed order (index order), and each
    column's rounding error is compensated on the columns not yet quantized
    through the inverse Hessian of the layer's reconstruction loss, written
    with a Cholesky factor.

    H = x^T x (float64; the loss's Hessian up to a factor 2 that cancels).
    A channel with H[k][k] = 0 gets H[k][k] = 1 and W[:, k] = 0; then
    H += damp * mean(diag H) * I.  U = the upper Cholesky factor of H^-1
    (H^-1 = U^T U).  For i = 0 .. K-1: at the first column of a group, its
    scale and zero come from the group's current weights by the RTN rule;
    the column's codes q and dequantized weights w_hat are taken with that
    rule (decisions on the float32 value of the running weights);
    err = (W[:, i] - w_hat) / U[i][i];  W[:, i+1:] -= err U[i, i+1:].
    The lazy batching of the updates is an ordering of the same arithmetic
    and is left out here.  The pages outline the method; the damping (1 %
    of the mean diagonal), the dead-channel rule and groups taken from the
    running weights at their first column are the published method's
    choices, read as the plain ones.
    act_order (the pages' desc_act option for GPTQ, "AutoGPTQ vs The Stack
    v2", first capability paragraph): the columns are processed in
    descending order of diag(H) after the dead-channel rule (stable for
    ties), groups are formed in that processing order, and g_idx[k] = (the
    position of channel k in that order) // group_size maps each channel to
    its group; the reading taken is the published method's.
    Returns a dict like quantize_linear_layer's (codes in original channel
    order, scales and zeros [N][G] by group, w_hat), plus g_idx int32 [K]
    (act_order only, else None).
    """
    qmax = _check_bits(bits)
    W = np.asarray(w, dtype=F16).astype(F64).copy()
    X = np.asarray(x, dtype=F16).astype(F64)
    N, K = W.shape
    gs = K if group_size == -1 else int(group_size)
    if gs <= 0 or K % gs:
        raise ValueError("group_size must divide K")
    H = X.T @ X
    dead = np.diag(H) == 0
    H[dead, dead] = 1.0
    W[:, dead] = 0.0
    perm = np.arange(K)
    if act_order:
        perm = np.argsort(-np.diag(H), kind="stable")
        W = W[:, perm]
        H = H[np.ix_(perm, perm)]
    H[np.diag_indices(K)] += damp * np.mean(np.diag(H))
    U = np.linalg.cholesky(np.linalg.inv(H)).T
    G = K // gs
    codes = np.zeros((N, K), dtype=np.uint8)
    scales = np.zeros((N, G), dtype=F16)
    zeros = None if symmetric else np.zeros((N, G), dtype=np.uint8)
    w_hat = np.zeros((N, K), dtype=F16)
    s_f = z = None
    for i in range(K):
        if i % gs == 0:
            s_h, z = _group_params_f32(W[:, i:i + gs].astype(F32), bits, symmetric)
            scales[:, i // gs] = s_h
            if not symmetric:
                zeros[:, i // gs] = z.astype(np.uint8)
            s_f = s_h.astype(F32)
        col = W[:, i].astype(F32)
        q = np.clip(np.rint(col / s_f) + z, F32(0), qmax)
        codes[:, i] = q.astype(np.uint8)
        wq = ((q - z) * s_f).astype(F16)
        w_hat[:, i] = wq
        err = (W[:, i] - wq.astype(F64)) / U[i, i]
        W[:, i + 1:] -= np.outer(err, U[i, i + 1:])
    if not act_order:
        return dict(codes=codes, scales=scales, zeros=zeros, w_hat=w_hat, g_idx=None)
    # back to the original channel order
    codes_o = np.empty_like(codes)
    w_hat_o = np.empty_like(w_hat)
    codes_o[:, perm] = codes
    w_hat_o[:, perm] = w_hat
    g_idx = np.empty(K, dtype=np.int32)
    g_idx[perm] = np.arange(K) // gs
    return dict(codes=codes_o, scales=scales, zeros=zeros, w_hat=w_hat_o, g_idx=g_idx)


def f64_to_f16_nearest(v: float) -> np.float16:
    """Nearest fp16 to a float64 value by exhaustive search over all finite
    fp16 values (ties to the even bit pattern).  Only used to pin numpy's
    float64 -> fp16 conversion; far too slow for anything else."""
    allh = np.arange(0, 0x7C00, dtype=np.uint16).view(F16).astype(F64)
    a = abs(float(v))
    d = np.abs(allh - a)
    best = np.nonzero(d == d.min())[0]
    if best.size > 1:
        best = best[best % 2 == 0]
    h = np.uint16(best[0])
    if v < 0:
        h = np.uint16(h | 0x8000)
    return np.array([h], dtype=np.uint16).view(F16)[0]
