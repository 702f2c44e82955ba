"""Edge cases of the quantizer, the packed format and both product kernels on
the GPU, through the C ABI.

The hand-worked fixtures under tests/golden/ (groups on the quantization
grid, round-half-to-even ties with even and odd zero-points, codes taken
from the stored fp16 scale) go through the whole path: GPU quantization,
packing, unpacking, dequantization, the GEMV and the GEMM.  Their expected
codes, scales, zeros and dequantized weights are the fixtures' own values.
With integer activations every product and partial sum of those weights is
exact in fp32, so the layer output must equal fp16 of the exact product bit
for bit, whatever the kernel's summation order.

Round-to-nearest as the baseline quantizer: "GPTQ, AWQ and the rules of
post-training quantization", section "The problem both methods solve".
Degenerate groups (max == min, or an all-zero group when symmetric) take
the smallest normal fp16 scale 2^-14; zero activations give a zero output.
"""

import numpy as np
import pytest

import oracle as O
import wq_inputs as I
from fixtures import read_fixture

torch = pytest.importorskip("torch")
import weight_only_int4_wq_amd as wq  # noqa: E402

pytestmark = pytest.mark.gpu

REL_L2 = 1e-3
MAX_ABS = 5e-2
SCALE_FLOOR_BITS = 0x0400  # fp16 2^-14


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wq.lib()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.cpu().numpy()


def bits16(a):
    return np.ascontiguousarray(a).view(np.uint16)


def check_y(y_gpu, y_ref, tag=""):
    y = host(y_gpu).astype(np.float64)
    assert y.shape == y_ref.shape, tag
    assert np.all(np.isfinite(y)), tag
    err = y - y_ref
    denom = np.linalg.norm(y_ref)
    rel = np.linalg.norm(err) / denom if denom > 0 else np.linalg.norm(err)
    mx = np.max(np.abs(err)) if err.size else 0.0
    assert rel <= REL_L2 and mx <= MAX_ABS, f"{tag}: rel_l2={rel:.3e} max_abs={mx:.3e}"


def gpu_layer(w, bits, gs, g_idx=None, sym=False):
    wd = dev(w)
    perm = None if g_idx is None else wq.act_order_perm(dev(g_idx), gs)
    codes, scales, zeros = wq.quantize_rtn(wd, bits, gs, perm=perm, symmetric=sym)
    packed, perm2 = wq.pack(codes, bits, gs, g_idx=None if g_idx is None else dev(g_idx))
    return dict(codes=codes, scales=scales, zeros=zeros, packed=packed, perm=perm2)


def int_activations(seed, M, K, lo=-4, hi=4):
    """Small integer activations: every product with a weight that is a
    multiple of 2^-k stays exact in fp32 accumulation."""
    g = np.random.default_rng(list(seed))
    return g.integers(lo, hi + 1, size=(M, K)).astype(np.float16)


GEMV_MS = (1, 2, 3, 4, 8, 16, 32)
GEMM_MS = (1, 17, 64, 130)


def products(x_ms, L, bits, gs):
    """(kernel, M, y) for every kernel and row count that applies."""
    out = []
    for M, x in x_ms.items():
        # the decode kernels take up to 16 rows, and up to 32 on the
        # matrix-core kernel (no act-order, K of at least 256)
        skinny = L["perm"] is None and x.shape[1] >= 256
        kernels = (["gemv"] if M <= 16 or (M <= 32 and skinny) else []) + ["gemm", "linear"]
        for k in kernels:
            fn = {"gemv": wq.gemv, "gemm": wq.gemm, "linear": wq.linear}[k]
            out.append((k, M, fn(dev(x), L["packed"], L["scales"], L["zeros"], bits, gs, perm=L["perm"])))
    return out


# --------------------------------------------- on-grid groups and ties ----

def _grid_rows(N, K):
    """Weight rows built from the on-grid fixture: every 128-wide group is the
    even-zero or odd-zero grid in a seeded order, and some groups carry one
    of the fixture's tie values at a position that holds neither the
    minimum nor the maximum.  Returns w and, from the fixture alone, the
    expected zeros, codes and dequantized weights."""
    rows = read_fixture("rtn_on_grid.txt")
    fx = {r[0]: r[1:] for r in rows if r[0] not in ("tie",)}
    ties = [(float(v), int(c), float(d)) for _, v, c, d in (r for r in rows if r[0] == "tie")]
    gsz = int(fx["group"][0])
    step = float(fx["step"][0])
    grids = [(float(fx["base"][0]), int(fx["zero"][0]), ties),
             (float(fx["odd_base"][0]), int(fx["odd_zero"][0]),
              [(float(fx["odd_tie"][0]), int(fx["odd_tie"][1]), float(fx["odd_tie"][2]))])]
    G = K // gsz
    g = np.random.default_rng([200, N, K])
    w = np.zeros((N, K), np.float16)
    codes = np.zeros((N, K), np.uint8)
    w_hat = np.zeros((N, K), np.float16)
    zeros = np.zeros((N, G), np.uint8)
    for n in range(N):
        for j in range(G):
            base, zero, tie_list = grids[(n + j) % 2]
            order = g.permutation(gsz)
            q = (order % 16).astype(np.int64)          # grid index of each member
            vals = base + step * q
            cds = q.copy()
            deq = vals.copy()
            kind = (n * G + j) % (len(tie_list) + 1)
            if kind < len(tie_list):
                # a member whose grid index is neither 0 (min) nor 15 (max)
                pos = int(np.nonzero((q != 0) & (q != 15))[0][g.integers(0, 100)])
                v, c, d = tie_list[kind]
                vals[pos], cds[pos], deq[pos] = v, c, d
            sl = slice(j * gsz, (j + 1) * gsz)
            w[n, sl] = vals.astype(np.float16)
            codes[n, sl] = cds
            w_hat[n, sl] = deq.astype(np.float16)
            zeros[n, j] = zero
    return w, float(fx["scale"][0]), zeros, codes, w_hat


@pytest.mark.parametrize("N,K", [(70, 384), (9, 1024)])
def test_golden_on_grid_and_ties_through_gpu_path(N, K):
    bits, gs = 4, 128
    w, scale, zeros, codes, w_hat = _grid_rows(N, K)
    L = gpu_layer(w, bits, gs)
    assert np.all(host(L["scales"]) == np.float16(scale))
    assert np.array_equal(host(L["zeros"]), zeros)
    assert np.array_equal(host(L["codes"]), codes)
    assert np.array_equal(host(wq.unpack(L["packed"], bits, K)), codes)
    wd = wq.dequant(L["packed"], L["scales"], L["zeros"], bits, gs, K)
    assert np.array_equal(bits16(host(wd)), bits16(w_hat))
    # the fixture's weights also agree with the oracle's packed words
    assert np.array_equal(host(L["packed"]).view(np.uint32), O.pack(codes, bits))
    xs = {M: int_activations((201, M, K), M, K) for M in GEMV_MS + GEMM_MS}
    for kernel, M, y in products(xs, L, bits, gs):
        exact = xs[M].astype(np.float64) @ w_hat.astype(np.float64).T
        want = exact.astype(np.float16)
        assert np.array_equal(bits16(host(y)), bits16(want)), (kernel, M)


def test_golden_on_grid_through_act_order_path():
    # the same rows under an act-order group map: the fixture's groups are
    # placed on the channels the map assigns to them
    bits, gs, N, K = 4, 128, 40, 512
    w_grid, scale, zeros, codes_grid, w_hat_grid = _grid_rows(N, K)
    g_idx = I.act_order_gidx((202,), K, gs)
    perm = O.act_order_perm(g_idx)            # packed column k' holds channel perm[k']
    w = np.empty_like(w_grid)
    w_hat = np.empty_like(w_hat_grid)
    codes = np.empty_like(codes_grid)
    w[:, perm], w_hat[:, perm], codes[:, perm] = w_grid, w_hat_grid, codes_grid
    L = gpu_layer(w, bits, gs, g_idx=g_idx)
    assert np.all(host(L["scales"]) == np.float16(scale))
    assert np.array_equal(host(L["zeros"]), zeros)
    assert np.array_equal(host(L["codes"]), codes)
    assert np.array_equal(host(wq.unpack(L["packed"], bits, K, perm=L["perm"])), codes)
    wd = wq.dequant(L["packed"], L["scales"], L["zeros"], bits, gs, K, perm=L["perm"])
    assert np.array_equal(bits16(host(wd)), bits16(w_hat))
    xs = {M: int_activations((203, M, K), M, K) for M in (1, 4, 16, 64)}
    for kernel, M, y in products(xs, L, bits, gs):
        want = (xs[M].astype(np.float64) @ w_hat.astype(np.float64).T).astype(np.float16)
        assert np.array_equal(bits16(host(y)), bits16(want)), (kernel, M)


def test_golden_stored_fp16_scale_through_gpu_path():
    # one 32-wide group per row carries the fixture's values in a seeded
    # order; the row's other groups are ordinary weights checked against the
    # oracle
    rows = read_fixture("rtn_scale_rounding.txt")
    fx = {r[0]: r[1] for r in rows if len(r) == 2}
    cases = [(float(v), int(c), float(d)) for v, c, d in (r for r in rows if len(r) == 3)]
    bits, gs, N, K = 4, 32, 48, 256
    G = K // gs
    w = I.weights((204,), N, K, 0.02)
    g = np.random.default_rng([204])
    want = {}
    for n in range(N):
        j = n % G
        vals = np.zeros(gs, np.float64)
        cds = np.full(gs, int(fx["zero"]), np.int64)       # the zeros code to the zero-point
        deq = np.zeros(gs, np.float64)
        for i, (v, c, d) in enumerate(cases):
            vals[i], cds[i], deq[i] = v, c, d
        order = g.permutation(gs)
        w[n, j * gs:(j + 1) * gs] = vals[order].astype(np.float16)
        want[n] = (j, cds[order], deq[order])
    ref = O.quantize_linear_layer(w, bits, gs)
    L = gpu_layer(w, bits, gs)
    scales, zeros, codes = host(L["scales"]), host(L["zeros"]), host(L["codes"])
    wd = host(wq.dequant(L["packed"], L["scales"], L["zeros"], bits, gs, K))
    for n, (j, cds, deq) in want.items():
        sl = slice(j * gs, (j + 1) * gs)
        assert scales[n, j] == np.float16(float(fx["scale"])), n
        assert zeros[n, j] == int(fx["zero"]), n
        assert np.array_equal(codes[n, sl], cds.astype(np.uint8)), n
        assert np.array_equal(wd[n, sl].astype(np.float64), deq), n
    assert np.array_equal(codes, ref["codes"])
    assert np.array_equal(bits16(scales), bits16(ref["scales"]))
    assert np.array_equal(zeros, ref["zeros"])
    assert np.array_equal(bits16(wd), bits16(ref["w_hat"]))
    for M in (1, 4, 16, 64):
        x = I.activations((205, M), M, K)
        y_ref = O.linear_ref(x, ref["w_hat"])
        for kernel in (("gemv",) if M <= 16 else ()) + ("gemm",):
            fn = {"gemv": wq.gemv, "gemm": wq.gemm}[kernel]
            check_y(fn(dev(x), L["packed"], L["scales"], L["zeros"], bits, gs), y_ref, f"{kernel} M={M}")


# ------------------------------------------------------ degenerate groups ----

def _degenerate_weights(seed, N, K, gs):
    """Rows of ordinary weights with constant rows (positive, negative, zero)
    and single constant or all-zero groups mixed in."""
    gsz = K if gs == -1 else gs
    w = I.weights(seed, N, K, 0.02)
    consts = [0.25, -0.5, 0.0, 1e-3, -3e-5]
    for n in range(0, N, 3):
        c = consts[(n // 3) % len(consts)]
        if (n // 3) % 2 == 0:
            w[n, :] = np.float16(c)                          # constant row
        else:
            j = (n // 3) % (K // gsz)
            w[n, j * gsz:(j + 1) * gsz] = np.float16(c)      # one constant group
    return w


DEGENERATE_CASES = [(b, g, s) for b in (2, 3, 4, 8) for g in (32, 128, -1) for s in (False, True)]


@pytest.mark.parametrize("bits,gs,sym", DEGENERATE_CASES)
def test_degenerate_groups_bit_exact_and_through_products(bits, gs, sym):
    N, K = 45, 256
    w = _degenerate_weights((206, bits, gs % 997, int(sym)), N, K, gs)
    ref = O.quantize_linear_layer(w, bits, gs, symmetric=sym)
    L = gpu_layer(w, bits, gs, sym=sym)
    scales = host(L["scales"])
    assert np.array_equal(host(L["codes"]), ref["codes"])
    assert np.array_equal(bits16(scales), bits16(ref["scales"]))
    if not sym:
        assert np.array_equal(host(L["zeros"]), ref["zeros"])
    assert np.array_equal(host(L["packed"]).view(np.uint32), ref["packed"])
    wd = wq.dequant(L["packed"], L["scales"], L["zeros"], bits, gs, K)
    assert np.array_equal(bits16(host(wd)), bits16(ref["w_hat"]))
    # the floor itself: a constant group (and an all-zero group when
    # symmetric) has scale 2^-14; symmetric all-zero groups code to 2^(b-1)
    gsz = K if gs == -1 else gs
    wg = w.astype(np.float64).reshape(N, K // gsz, gsz)
    flat = (wg.max(axis=2) == wg.min(axis=2)) if not sym else (np.abs(wg).max(axis=2) == 0)
    assert flat.any()
    assert np.all(bits16(scales)[flat] == SCALE_FLOOR_BITS)
    if sym:
        zero_codes = host(L["codes"]).reshape(N, K // gsz, gsz)[flat]
        assert np.all(zero_codes == (1 << (bits - 1)))
    xs = {M: I.activations((207, M), M, K) for M in (1, 4, 16, 64)}
    for kernel, M, y in products(xs, L, bits, gs):
        check_y(y, O.linear_ref(xs[M], ref["w_hat"]), f"{kernel} M={M}")


def test_constant_rows_through_act_order_path():
    bits, gs, N, K = 4, 64, 30, 512
    w = _degenerate_weights((208,), N, K, gs)
    g_idx = I.act_order_gidx((208,), K, gs)
    ref = O.quantize_linear_layer(w, bits, gs, g_idx=g_idx)
    L = gpu_layer(w, bits, gs, g_idx=g_idx)
    assert np.array_equal(host(L["codes"]), ref["codes"])
    assert np.array_equal(bits16(host(L["scales"])), bits16(ref["scales"]))
    assert np.array_equal(host(L["zeros"]), ref["zeros"])
    assert np.array_equal(host(L["packed"]).view(np.uint32), ref["packed"])
    xs = {M: I.activations((209, M), M, K) for M in (1, 3, 16, 100)}
    for kernel, M, y in products(xs, L, bits, gs):
        check_y(y, O.linear_ref(xs[M], ref["w_hat"]), f"{kernel} M={M}")


# ------------------------------------------------------ zero activations ----

@pytest.mark.parametrize("bits,gs,sym,act", [(4, 128, False, False), (4, 128, False, True), (2, 32, True, False),
                                             (3, 32, True, True), (8, -1, True, False), (3, 128, False, False)])
def test_zero_activations_give_zero_output(bits, gs, sym, act):
    N, K = 300, 1024
    seed = (210, bits, gs % 997, int(act))
    w = I.weights(seed, N, K, 0.02)
    g_idx = I.act_order_gidx(seed, K, gs) if act else None
    L = gpu_layer(w, bits, gs, g_idx=g_idx, sym=sym)
    for M in (1, 2, 4, 8, 16, 17, 64, 300):
        x = torch.zeros((M, K), dtype=torch.float16, device="cuda")
        kernels = ((wq.gemv,) if M <= 16 else ()) + (wq.gemm, wq.linear)
        for fn in kernels:
            y = host(fn(x, L["packed"], L["scales"], L["zeros"], bits, gs, perm=L["perm"]))
            assert np.all(bits16(y) == 0), (fn.__name__, M)      # +0.0, bit for bit
    s = dev(np.full(K, 0.75, np.float16))
    for M in (1, 4):
        x = torch.zeros((M, K), dtype=torch.float16, device="cuda")
        y = host(wq.gemv_ex(x, L["packed"], L["scales"], L["zeros"], bits, gs, perm=L["perm"], act_scale=s))
        assert np.all(bits16(y) == 0), M
        y = host(wq.gemv_silu_mul(x, L["packed"], L["scales"], L["zeros"], bits, gs, perm=L["perm"]))
        assert np.all(bits16(y) == 0), M


# --------------------------------------- scale floors of the other quantizers ----

@pytest.mark.parametrize("bits,gs,sym", [(4, 128, False), (3, 32, True), (8, -1, True), (2, 64, False)])
def test_gptq_zero_and_constant_rows(bits, gs, sym):
    # On correlated calibration data a zero weight row stays zero through the
    # compensation (its rounding error is zero): every group degenerates to
    # the 2^-14 scale.  With a diagonal Hessian nothing is carried, so the
    # constant rows equal plain RTN's bit for bit as well.
    N, K, M = 40, 256, 128
    seed = (211, bits, gs % 997)
    w = _degenerate_weights(seed, N, K, gs)
    w[1, :] = 0
    x = I.correlated_activations(seed, M, K)
    codes, scales, zeros, _ = wq.gptq_quantize(dev(w), dev(x), bits, gs, symmetric=sym)
    G = scales.shape[1]
    assert np.all(bits16(host(scales))[1] == SCALE_FLOOR_BITS)
    want = (1 << (bits - 1)) if sym else 0
    assert np.all(host(codes)[1] == want)
    if not sym:
        assert np.all(host(zeros)[1] == 0)
    ref = O.gptq_quantize(w, x, bits, gs, symmetric=sym)
    assert np.array_equal(host(codes)[1], ref["codes"][1])
    xd = (3.0 * np.eye(K)).astype(np.float16)
    codes, scales, zeros, _ = wq.gptq_quantize(dev(w), dev(xd), bits, gs, symmetric=sym)
    rc, rs, rz = O.rtn_quantize(w, bits, gs, symmetric=sym)
    assert np.array_equal(host(codes), rc)
    assert np.array_equal(bits16(host(scales)), bits16(rs))
    if not sym:
        assert np.array_equal(host(zeros), rz)
    assert G == (1 if gs == -1 else K // gs)


@pytest.mark.parametrize("bits,gs,sym", [(4, 128, False), (3, 32, True), (8, -1, False)])
def test_awq_clip_degenerate_groups(bits, gs, sym):
    # all-zero and constant groups: every ratio clips to a constant group,
    # RTN takes the scale floor, and the oracle fixes losses, the chosen
    # ratio (the first minimum) and the clipped weights
    M, N, K = 64, 36, 256
    seed = (212, bits, gs % 997)
    w = _degenerate_weights(seed, N, K, gs)
    x = I.with_outliers(I.activations(seed, M, K), I.outlier_channels(seed, K, 0.05))
    ref = O.awq_clip_search(x, w, bits, gs, symmetric=sym)
    w_clip, best, losses = wq.awq_clip(dev(x), dev(w), bits, gs, symmetric=sym, with_losses=True)
    L = ref["losses"]
    lg = host(losses).astype(np.float64)
    scale = np.max(L)
    assert np.all(np.abs(lg - L) <= 5e-3 * L + 1e-9 * scale)
    b = host(best)
    gsz = K if gs == -1 else gs
    wg = w.astype(np.float64).reshape(N, K // gsz, gsz)
    zero_group = np.abs(wg).max(axis=2) == 0
    assert zero_group.any()
    assert np.all(b[zero_group] == 0) and np.all(ref["best"][zero_group] == 0)
    assert np.mean(b == ref["best"]) >= 0.99
    same = np.repeat(b == ref["best"], gsz, axis=1)
    assert np.array_equal(bits16(host(w_clip))[same], bits16(ref["w_clip"])[same])


def test_gptq_act_order_with_non_finite_calibration_data():
    # A NaN in the calibration activations makes a Hessian diagonal entry
    # NaN.  The act-order ranking is a total order with NaN last, so the
    # processing order is still a permutation: the call completes, the group
    # map has equal groups and the codes stay in range (their values are
    # meaningless for such input).
    M, N, K, bits, gs = 64, 40, 256, 4, 32
    seed = (213,)
    x = I.correlated_activations(seed, M, K)
    x[3, 17] = np.float16(np.nan)
    x[5, 90] = np.float16(np.inf)
    w = I.weights(seed, N, K, 0.02)
    codes, scales, zeros, g_idx = wq.gptq_quantize(dev(w), dev(x), bits, gs, act_order=True)
    torch.cuda.synchronize()
    gi = host(g_idx)
    assert np.array_equal(np.bincount(gi, minlength=K // gs), np.full(K // gs, gs))
    assert host(codes).max() <= (1 << bits) - 1
    perm = host(wq.act_order_perm(g_idx, gs))
    assert np.array_equal(np.sort(perm), np.arange(K))


def test_quantized_linear_awq_act_order_long_rows():
    # act-order with an AWQ input scale on 28672-channel rows at M = 1: the
    # fused decode kernel either takes it or declines, and the layer's
    # output meets the tolerance either way
    K, N, bits, gs = 28672, 48, 4, 128
    seed = (214,)
    x = I.with_outliers(I.activations(seed, 4, K), I.outlier_channels(seed, K))
    w = I.weights(seed, N, K, 0.015)
    g_idx = I.act_order_gidx(seed, K, gs)
    _, s_h = O.awq_channel_scales(x, 0.5)
    layer = wq.QuantizedLinear.from_float(dev(w), bits=bits, group_size=gs, g_idx=dev(g_idx), act_scale=dev(s_h))
    ref = O.quantize_linear_layer(O.awq_fold_weight(w, s_h), bits, gs, g_idx=g_idx)
    for M in (1, 4):
        y = layer(dev(x[:M]))
        check_y(y, O.linear_ref(O.awq_scale_act(x[:M], s_h), ref["w_hat"]), f"M={M}")
