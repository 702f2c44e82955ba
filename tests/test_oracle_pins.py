"""Pins of the CPU oracle against things fixed outside the oracle itself:
hand-worked fixtures, closed forms, invariants, brute force and textbook
special cases.  CPU only."""

import itertools
import os

import numpy as np
import pytest

import oracle as O
import wq_inputs as I

from fixtures import read_fixture as _read_fixture


# ----------------------------------------------------------------- packing

def test_pack_golden_words():
    rows = _read_fixture("pack_words.txt")
    assert len(rows) == 5
    for row in rows:
        bits, K, pattern = int(row[0]), int(row[1]), row[2]
        want = np.array([int(v, 16) for v in row[3:]], dtype=np.uint32)
        k = np.arange(K)
        codes = (k % (1 << bits)) if pattern == "mod" else np.full(K, (1 << bits) - 1)
        codes = codes.astype(np.uint8)[None, :]
        got = O.pack(codes, bits)
        assert got.shape == (1, len(want))
        assert np.array_equal(got[0], want), (bits, [hex(v) for v in got[0]])
        assert np.array_equal(O.unpack(got, bits, K), codes)


def _bits_of_stream(words, start, nbits):
    # Brute-force read of a bit field from a little-endian word stream using
    # Python integers.
    value = 0
    for i in range(nbits):
        pos = start + i
        bit = (int(words[pos // 32]) >> (pos % 32)) & 1
        value |= bit << i
    return value


@pytest.mark.parametrize("bits", O.SUPPORTED_BITS)
def test_pack_bruteforce_bit_reads(bits):
    K = 96 if bits == 3 else 64
    codes = I.random_codes((11, bits), 3, K, bits)
    packed = O.pack(codes, bits)
    assert packed.shape == (3, K * bits // 32)
    for n in range(3):
        for k in range(K):
            assert _bits_of_stream(packed[n], k * bits, bits) == codes[n, k]


@pytest.mark.parametrize("bits", O.SUPPORTED_BITS)
def test_pack_roundtrip(bits):
    for K in (32, 128, 4096 // bits * bits if bits != 3 else 384):
        codes = I.random_codes((12, bits, K), 7, K, bits)
        assert np.array_equal(O.unpack(O.pack(codes, bits), bits, K), codes)


def test_pack_rejects_bad_input():
    with pytest.raises(ValueError):
        O.pack(np.zeros((1, 8), np.uint8), 3)          # 24 bits: not whole words
    with pytest.raises(ValueError):
        O.pack(np.full((1, 32), 16, np.uint8), 4)      # code out of range
    with pytest.raises(ValueError):
        O.pack(np.zeros((1, 32), np.uint8), 5)         # unsupported width


# ------------------------------------------------------------- quantizer

def _on_grid_group():
    fx = {r[0]: r[1:] for r in _read_fixture("rtn_on_grid.txt") if r[0] != "tie"}
    ties = [r[1:] for r in _read_fixture("rtn_on_grid.txt") if r[0] == "tie"]
    base, step = float(fx["base"][0]), float(fx["step"][0])
    j = np.arange(int(fx["group"][0]))
    w = (base + step * (j % 16)).astype(np.float16)[None, :]
    return fx, ties, w


def test_rtn_on_grid_is_exact():
    fx, _, w = _on_grid_group()
    bits = int(fx["bits"][0])
    codes, scales, zeros = O.rtn_quantize(w, bits, 128)
    assert scales[0, 0] == np.float16(float(fx["scale"][0]))
    assert zeros[0, 0] == int(fx["zero"][0])
    assert np.array_equal(codes[0], (np.arange(128) % 16).astype(np.uint8))
    w_hat = O.dequant(codes, scales, zeros, bits, 128)
    assert np.array_equal(w_hat.view(np.uint16), w.view(np.uint16))


def test_rtn_tie_break_half_even():
    fx, ties, w = _on_grid_group()
    bits = int(fx["bits"][0])
    for value, code, deq in ties:
        w2 = w.copy()
        w2[0, 7] = np.float16(float(value))   # j=7 holds 0.375: not an extreme
        codes, scales, zeros = O.rtn_quantize(w2, bits, 128)
        assert scales[0, 0] == np.float16(0.125) and zeros[0, 0] == 4
        assert codes[0, 7] == int(code), value
        w_hat = O.dequant(codes, scales, zeros, bits, 128)
        assert w_hat[0, 7] == np.float16(float(deq))


def test_rtn_tie_with_odd_zero():
    fx = {r[0]: r[1:] for r in _read_fixture("rtn_on_grid.txt")}
    base, step = float(fx["odd_base"][0]), float(fx["step"][0])
    w = (base + step * (np.arange(128) % 16)).astype(np.float16)[None, :]
    value, code, deq = fx["odd_tie"]
    w[0, 7] = np.float16(float(value))
    codes, scales, zeros = O.rtn_quantize(w, 4, 128)
    assert zeros[0, 0] == int(fx["odd_zero"][0]) and scales[0, 0] == np.float16(step)
    assert codes[0, 7] == int(code)
    assert O.dequant(codes, scales, zeros, 4, 128)[0, 7] == np.float16(float(deq))


def test_rtn_codes_use_stored_fp16_scale():
    rows = _read_fixture("rtn_scale_rounding.txt")
    fx = {r[0]: r[1] for r in rows if len(r) == 2}
    cases = [r for r in rows if len(r) == 3]
    w = np.zeros((1, 32), np.float16)
    for i, (v, _, _) in enumerate(cases):
        w[0, i] = np.float16(float(v))
    codes, scales, zeros = O.rtn_quantize(w, 4, 32)
    assert scales[0, 0] == np.float16(float(fx["scale"])) and zeros[0, 0] == int(fx["zero"])
    w_hat = O.dequant(codes, scales, zeros, 4, 32)
    for i, (v, c, d) in enumerate(cases):
        assert codes[0, i] == int(c), v
        assert float(w_hat[0, i]) == float(d), v


def test_rtn_groups_are_indexed_per_group():
    # Two groups of 32 with very different ranges: a wrong group index (or
    # swapped axis) gives the wrong scale for one of them.
    K = 64
    w = np.zeros((2, K), np.float16)
    w[0, :32] = np.linspace(-1, 1, 32)     # range 2
    w[0, 32:] = np.linspace(-4, 4, 32)     # range 8
    w[1, :32] = np.linspace(0, 0.5, 32) - 0.25
    w[1, 32:] = np.linspace(-2, 2, 32)
    codes, scales, zeros = O.rtn_quantize(w, 4, 32)
    want = np.array([[2 / 15, 8 / 15], [0.5 / 15, 4 / 15]])
    assert np.allclose(scales.astype(np.float64), want, rtol=1e-3)
    # Per-channel (group_size = -1) is one group over all of K.
    c2, s2, z2 = O.rtn_quantize(w, 4, -1)
    assert s2.shape == (2, 1)
    assert np.isclose(float(s2[0, 0]), 8 / 15, rtol=1e-3)


@pytest.mark.parametrize("bits,gs,sym", [(4, 128, False), (2, 32, True), (3, 128, True),
                                         (8, -1, True), (3, 32, False), (8, 128, False)])
def test_rtn_code_range_and_error_bound(bits, gs, sym):
    N, K = 64, 512
    w = I.weights((21, bits, gs % 1000), N, K, 0.02)
    codes, scales, zeros = O.rtn_quantize(w, bits, gs, symmetric=sym)
    qmax = (1 << bits) - 1
    assert codes.max() <= qmax
    if sym:
        assert zeros is None
    else:
        assert zeros.max() <= qmax
    w_hat = O.dequant(codes, scales, zeros, bits, gs)
    gk = O.group_of_channel(K, gs)
    s_h = scales.astype(np.float64)[:, gk]
    # recompute the unrounded fp32 scale to bound the edge clipping
    w64 = w.astype(np.float64)
    G = scales.shape[1]
    s32 = np.zeros((N, G))
    for j in range(G):
        wg = w64[:, gk == j]
        s32[:, j] = (2 * np.abs(wg).max(1) if sym else wg.max(1) - wg.min(1)) / qmax
    clip = qmax * np.abs(s32 - scales.astype(np.float64))[:, gk]
    bound = 0.5 * s_h + clip + 2.0 ** -11 * np.abs(w_hat.astype(np.float64)) + 1e-7
    if sym:
        bound = bound + 0.5 * s_h  # the positive end of the symmetric grid is one step short
    err = np.abs(w64 - w_hat.astype(np.float64))
    assert np.all(err <= bound)


def test_rtn_symmetric_closed_form():
    # max|w| = 1.5 (taken by the negative end), 4-bit: scale = 3/15 = 0.2 ->
    # fp16(0.2) = 0.199951171875; zero = 8.  -1.5/s = -7.5018 -> -8 -> code 0;
    # 1.0/s = 5.0012 -> 5 -> code 13.
    w = np.array([[-1.5, -0.2, 0.0, 0.2, 1.0] + [0.0] * 27], np.float16)
    codes, scales, zeros = O.rtn_quantize(w, 4, 32, symmetric=True)
    s = np.float16(0.2)
    assert zeros is None and scales[0, 0] == s
    s32 = np.float32(s)
    want = np.clip(np.rint(w.astype(np.float32) / s32) + 8, 0, 15)
    assert np.array_equal(codes[0], want[0].astype(np.uint8))
    assert codes[0, 0] == 0 and codes[0, 2] == 8 and codes[0, 4] == 13


def test_rtn_degenerate_group_scale_floor():
    w = np.full((1, 32), 0.25, np.float16)      # max == min
    codes, scales, zeros = O.rtn_quantize(w, 4, 32)
    assert scales[0, 0] == np.float16(2.0 ** -14)
    assert zeros[0, 0] == 0                     # -0.25/s < 0 clips to 0
    assert np.all(codes == 15)                  # 0.25/s is far above the top code


# ----------------------------------------------------------------- dequant

@pytest.mark.parametrize("bits,sym", [(2, True), (3, False), (4, False), (8, True)])
def test_dequant_formulations_agree(bits, sym):
    w = I.weights((31, bits), 16, 256, 0.05)
    codes, scales, zeros = O.rtn_quantize(w, bits, 64, symmetric=sym)
    a = O.dequant(codes, scales, zeros, bits, 64)
    b = O.dequant_fp64_path(codes, scales, zeros, bits, 64)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_numpy_f64_to_f16_is_correctly_rounded():
    # The AWQ scale is rounded float64 -> fp16 in one step; pin numpy's
    # conversion against an exhaustive nearest-value search, including
    # values just either side of rounding midpoints.
    g = np.random.default_rng(5)
    vals = list(g.uniform(0.01, 30.0, 40))
    for h in g.integers(0x1000, 0x7000, 20):
        lo = float(np.array([h], np.uint16).view(np.float16)[0])
        hi = float(np.array([h + 1], np.uint16).view(np.float16)[0])
        mid = 0.5 * (lo + hi)
        vals += [mid, np.nextafter(mid, 0), np.nextafter(mid, 100)]
    for v in vals:
        got = np.float64(v).astype(np.float16)
        want = O.f64_to_f16_nearest(v)
        assert got.view(np.uint16) == want.view(np.uint16), v


# --------------------------------------------------------------------- AWQ

def test_awq_scale_closed_form():
    # Column k alternates +a_k and -b_k: mean |x| = c_k = (a_k + b_k) / 2 (the
    # mean, not the max, of the magnitudes), so s = c_k ** alpha.
    a = np.array([0.25, 1.0, 2.0, 1.0] * 8, dtype=np.float64)
    b = np.array([0.25, 7.0, 6.0, 17.0] * 8, dtype=np.float64)
    c = (a + b) / 2                                    # 0.25, 4, 4, 9
    rows = np.arange(6)[:, None] % 2 == 0
    x = np.where(rows, a[None, :], -b[None, :]).astype(np.float16)
    s, s_h = O.awq_channel_scales(x, 0.5)
    assert np.allclose(s, np.sqrt(c), rtol=0, atol=1e-15)
    assert np.array_equal(s_h, np.sqrt(c).astype(np.float16))
    s0, _ = O.awq_channel_scales(x, 0.0)
    assert np.all(s0 == 1.0)
    s1, _ = O.awq_channel_scales(x, 1.0)
    assert np.allclose(s1, c)


def test_awq_scale_rounds_once_to_fp16():
    # mean |x| = 0.5 + 2^-12 + 2^-26 lies just above the midpoint between
    # fp16 0.5 and 0.5 + 2^-11; one direct rounding gives the upper value
    # (rounding through fp32 first would land on the midpoint and tie down).
    x = np.array([[1.0], [1.0 + 2.0 ** -10], [2.0 ** -24], [0.0]], dtype=np.float16)
    s, s_h = O.awq_channel_scales(x, 1.0)
    assert s[0] == 0.5 + 2.0 ** -12 + 2.0 ** -26
    assert float(s_h[0]) == 0.5 + 2.0 ** -11


def test_awq_invariance_exact_with_power_of_two_scales():
    # With s_k a power of two, folding and dividing are exact, so the layer
    # computes the same function bit for bit (the equivalence the rescaling
    # rests on).
    K, M, N = 64, 4, 5
    mags = 4.0 ** (np.arange(K) % 5 - 2)              # mean|x| = 4^j -> s = 2^j
    signs = np.where((np.arange(M)[:, None] + np.arange(K)[None, :]) % 2, 1.0, -1.0)
    x = (signs * mags[None, :]).astype(np.float16)
    w = I.weights((41,), N, K, 0.5)
    s, s_h = O.awq_channel_scales(x, 0.5)
    assert np.all(s_h.astype(np.float64) == 2.0 ** (np.arange(K) % 5 - 2))
    xs, ws = O.awq_scale_act(x, s_h), O.awq_fold_weight(w, s_h)
    assert np.array_equal(O.linear_ref(xs, ws), O.linear_ref(x, w))


def test_awq_invariance_with_rounding():
    # Generic scales: only the fp16 roundings of x' and W' separate the two
    # products.  Scaling the wrong axis would break this by O(1).
    K, M, N = 256, 64, 96
    x = I.with_outliers(I.activations((42,), M, K), I.outlier_channels((42,), K, 0.05))
    w = I.weights((42,), N, K, 0.02)
    _, s_h = O.awq_channel_scales(x, 0.5)
    y0 = O.linear_ref(x, w)
    y1 = O.linear_ref(O.awq_scale_act(x, s_h), O.awq_fold_weight(w, s_h))
    rel = np.linalg.norm(y1 - y0) / np.linalg.norm(y0)
    assert rel < 2e-3
    # a fold along the wrong axis is far off
    bad = (w.astype(np.float32) * s_h.astype(np.float32)[:N, None]).astype(np.float16)
    relbad = np.linalg.norm(O.linear_ref(O.awq_scale_act(x, s_h), bad) - y0) / np.linalg.norm(y0)
    assert relbad > 0.1


def test_awq_reduces_error_on_outlier_channels():
    # Activation-aware rescaling protects the weights on high-magnitude input
    # channels, so the quantized layer's output error drops relative to plain
    # RTN on the same weights ("AWQ: find the one percent that matters").
    K, M, N = 1024, 256, 256
    seed = (43,)
    x = I.with_outliers(I.activations(seed, M, K), I.outlier_channels(seed, K))
    w = I.weights(seed, N, K, 0.02)
    y_true = O.linear_ref(x, w)
    plain = O.quantize_linear_layer(w, 4, 128)
    e_plain = np.linalg.norm(O.linear_ref(x, plain["w_hat"]) - y_true)
    _, s_h = O.awq_channel_scales(x, 0.5)
    awq = O.quantize_linear_layer(O.awq_fold_weight(w, s_h), 4, 128)
    e_awq = np.linalg.norm(O.linear_ref(O.awq_scale_act(x, s_h), awq["w_hat"]) - y_true)
    assert e_awq < 0.8 * e_plain


# ------------------------------------------------------------ AWQ search

def test_awq_alpha_grid_closed_form():
    # twenty evenly spaced points on the closed interval [0, 1]
    g = O.awq_alpha_grid(20)
    assert g.shape == (20,)
    assert g[0] == 0.0 and g[-1] == 1.0
    assert np.allclose(np.diff(g), 1.0 / 19.0, rtol=0, atol=1e-15)


def test_awq_search_at_alpha_zero_is_plain_rtn():
    # alpha = 0 gives s = a^0 = 1 for every channel: the fold and the
    # division are identities, so the first loss is the plain RTN output
    # error, computed here without any AWQ step.
    M, K, N = 16, 256, 24
    seed = (44,)
    x = I.with_outliers(I.activations(seed, M, K), I.outlier_channels(seed, K))
    w = I.weights(seed, N, K, 0.02)
    _, losses, _ = O.awq_search(x, w, 4, 128, n_grid=4)
    q = O.quantize_linear_layer(w, 4, 128)
    d = x.astype(np.float64) @ (q["w_hat"].astype(np.float64) - w.astype(np.float64)).T
    assert np.isclose(losses[0], np.sum(d * d), rtol=1e-12, atol=0)


def test_awq_search_bruteforce_tiny():
    # Every step written out with scalar loops on a tiny layer (one group):
    # channel statistics, scale rounding, fold, division, quantization by
    # the pinned RTN, and the squared output error against the original.
    M, K, N = 3, 32, 2
    seed = (45,)
    x = I.activations(seed, M, K)
    w = I.weights(seed, N, K, 0.05)
    alphas, losses, best = O.awq_search(x, w, 4, 32, n_grid=3)
    assert list(alphas) == [0.0, 0.5, 1.0]
    for i, a in enumerate(alphas):
        s_h = np.zeros(K, dtype=np.float16)
        for k in range(K):
            mean = sum(abs(float(x[m, k])) for m in range(M)) / M
            s_h[k] = np.float16(mean ** a)
        wf = np.zeros((N, K), dtype=np.float16)
        xf = np.zeros((M, K), dtype=np.float16)
        for k in range(K):
            for n in range(N):
                wf[n, k] = np.float16(np.float32(w[n, k]) * np.float32(s_h[k]))
            for m in range(M):
                xf[m, k] = np.float16(np.float32(x[m, k]) / np.float32(s_h[k]))
        codes, scales, zeros = O.rtn_quantize(wf, 4, 32)
        loss = 0.0
        for m in range(M):
            for n in range(N):
                yq = sum(float(xf[m, k]) * float(np.float16(np.float32(int(codes[n, k]) - int(zeros[n, 0]))
                                                             * np.float32(scales[n, 0])))
                         for k in range(K))
                yr = sum(float(x[m, k]) * float(w[n, k]) for k in range(K))
                loss += (yq - yr) ** 2
        assert np.isclose(losses[i], loss, rtol=1e-10, atol=0), (i, losses[i], loss)
    assert best == int(np.argmin(losses))


def test_awq_search_prefers_rescaling_on_outlier_channels():
    # With a few high-magnitude input channels the search settles on a
    # positive alpha whose output error is clearly below plain RTN's
    # (the rescaling claim of "AWQ: find the one percent that matters").
    M, K, N = 128, 1024, 128
    seed = (46,)
    x = I.with_outliers(I.activations(seed, M, K), I.outlier_channels(seed, K))
    w = I.weights(seed, N, K, 0.02)
    alphas, losses, best = O.awq_search(x, w, 4, 128, n_grid=20)
    assert alphas[best] > 0.0
    assert losses[best] < 0.8 * losses[0]


# ------------------------------------------------------------------ GPTQ

def test_gptq_with_uncorrelated_inputs_is_rtn():
    # x = c * I makes H a multiple of the identity: every off-diagonal entry
    # of the inverse Hessian's Cholesky factor is 0, no error is carried to
    # other columns, and GPTQ must return plain RTN's codes, scales, zeros.
    K, N = 256, 40
    seed = (48,)
    w = I.weights(seed, N, K, 0.02)
    x = (np.eye(K) * 3.0).astype(np.float16)
    for bits, gs, sym in ((4, 128, False), (3, 32, True), (8, -1, True)):
        g = O.gptq_quantize(w, x, bits, gs, symmetric=sym)
        codes, scales, zeros = O.rtn_quantize(w, bits, gs, symmetric=sym)
        assert np.array_equal(g["codes"], codes), (bits, gs)
        assert np.array_equal(g["scales"].view(np.uint16), scales.view(np.uint16)), (bits, gs)
        if not sym:
            assert np.array_equal(g["zeros"], zeros)


def _obs_reference(w, x, bits, gs, damp=0.01):
    # The same column-by-column compensation written with the explicit
    # inverse Hessian (Optimal Brain Surgeon form): after quantizing column
    # i, W[:, j] -= err_i * Hinv[i][j] / Hinv[i][i] for the remaining j, and
    # column i is eliminated from Hinv.  Mathematically the Cholesky form's
    # update; written independently with scalar loops.
    W = w.astype(np.float64).copy()
    X = x.astype(np.float64)
    N, K = W.shape
    H = X.T @ X
    for k in range(K):
        if H[k, k] == 0:
            H[k, k] = 1.0
            W[:, k] = 0.0
    mean_diag = sum(H[k, k] for k in range(K)) / K
    for k in range(K):
        H[k, k] += damp * mean_diag
    Hinv = np.linalg.inv(H)
    qmax = (1 << bits) - 1
    codes = np.zeros((N, K), dtype=np.int64)
    for i in range(K):
        if i % gs == 0:
            grp = W[:, i:i + gs].astype(np.float32)
            mn, mx = grp.min(axis=1), grp.max(axis=1)
            s_h = ((mx - mn) / np.float32(qmax)).astype(np.float16)
            s_f = s_h.astype(np.float32)
            z = np.clip(np.rint(-mn / s_f), 0, qmax).astype(np.float32)
        for n in range(N):
            v = np.float32(W[n, i])
            q = min(max(np.rint(v / s_f[n]) + z[n], 0), qmax)
            codes[n, i] = int(q)
            what = float(np.float16(np.float32(q - z[n]) * s_f[n]))
            e = (W[n, i] - what) / Hinv[i, i]
            for j in range(i + 1, K):
                W[n, j] -= e * Hinv[i, j]
        # eliminate column i from the inverse Hessian
        Hinv = Hinv - np.outer(Hinv[:, i], Hinv[i, :]) / Hinv[i, i]
    return codes


def test_gptq_cholesky_form_matches_inverse_hessian_form():
    K, N, M = 16, 5, 64
    seed = (49,)
    rng = np.random.default_rng(list(seed))
    x = (rng.standard_normal((M, K)) @ rng.standard_normal((K, K)) * 0.3).astype(np.float16)
    w = I.weights(seed, N, K, 0.05)
    g = O.gptq_quantize(w, x, 4, 8)
    assert np.array_equal(g["codes"].astype(np.int64), _obs_reference(w, x, 4, 8))


def test_gptq_beats_rtn_on_correlated_inputs():
    # compensation lowers the layer's output error below plain rounding's
    K, N, M = 256, 64, 512
    seed = (50,)
    rng = np.random.default_rng(list(seed))
    mix = np.eye(K) + 0.3 * rng.standard_normal((K, K)) / np.sqrt(K)
    x = (rng.standard_normal((M, K)) @ mix).astype(np.float16)
    w = I.weights(seed, N, K, 0.02)
    y = O.linear_ref(x, w)
    g = O.gptq_quantize(w, x, 4, 128)
    r = O.quantize_linear_layer(w, 4, 128)
    e_g = np.linalg.norm(O.linear_ref(x, g["w_hat"]) - y)
    e_r = np.linalg.norm(O.linear_ref(x, r["w_hat"]) - y)
    assert e_g < 0.9 * e_r, (e_g, e_r)


# ------------------------------------------------------- fused gate / up

def test_silu_mul_closed_forms():
    # y = silu(g) * u with g, u the two halves of one stacked product: pick
    # x and w so that g and u are known numbers.  silu(0) = 0, silu(1) =
    # 1 / (1 + 1/e), silu(-1) = -1 / (1 + e), and u scales the result.
    K = 32
    x = np.zeros((1, K), dtype=np.float16)
    x[0, 0] = 1.0
    w = np.zeros((6, K), dtype=np.float16)
    w[0, 0], w[1, 0], w[2, 0] = 0.0, 1.0, -1.0     # gate values 0, 1, -1
    w[3, 0], w[4, 0], w[5, 0] = 5.0, 2.0, 3.0      # up values
    y = O.silu_mul_ref(x, w)
    e = np.e
    assert y.shape == (1, 3)
    assert y[0, 0] == 0.0
    assert np.isclose(y[0, 1], 2.0 / (1.0 + 1.0 / e), rtol=1e-15)
    assert np.isclose(y[0, 2], -3.0 / (1.0 + e), rtol=1e-15)


def test_silu_mul_halves_follow_the_stacking():
    # swapping the gate and up halves changes the result (the gate goes
    # through silu, the up projection does not)
    seed = (47,)
    x = I.activations(seed, 2, 64)
    w = I.weights(seed, 8, 64, 0.5)
    y = O.silu_mul_ref(x, w)
    g = x.astype(np.float64) @ w[:4].astype(np.float64).T
    u = x.astype(np.float64) @ w[4:].astype(np.float64).T
    assert np.allclose(y, g * u / (1 + np.exp(-g)), rtol=1e-12, atol=0)
    swapped = O.silu_mul_ref(x, np.concatenate([w[4:], w[:4]]))
    assert not np.allclose(swapped, y)
    with pytest.raises(ValueError):
        O.silu_mul_ref(x, w[:7])


# ------------------------------------------------------------------ matmul

def test_linear_matches_bruteforce_triple_loop():
    M, K, N = 3, 64, 5
    seed = (51,)
    x = I.activations(seed, M, K)
    q = O.quantize_linear_layer(I.weights(seed, N, K, 0.02), 4, 32)
    y = O.linear_ref(x, q["w_hat"])
    assert y.shape == (M, N)
    for m, n in itertools.product(range(M), range(N)):
        acc = 0.0
        for k in range(K):
            zq = 8 if q["zeros"] is None else int(q["zeros"][n, k // 32])
            w_nk = (int(q["codes"][n, k]) - zq) * float(q["scales"][n, k // 32])
            acc += float(x[m, k]) * float(np.float16(w_nk))
        assert abs(y[m, n] - acc) <= 1e-12 * max(1.0, abs(acc))


def test_linear_integer_special_case_is_exact():
    # Scale 1, zero 0 and integer activations: the layer is an integer
    # matrix product, which numpy's int64 matmul computes exactly.
    M, K, N, bits = 4, 128, 6, 4
    g = np.random.default_rng(52)
    codes = g.integers(0, 16, (N, K), dtype=np.uint8)
    xi = g.integers(-8, 9, (M, K))
    scales = np.ones((N, K // 32), np.float16)
    zeros = np.zeros((N, K // 32), np.uint8)
    w_hat = O.dequant(codes, scales, zeros, bits, 32)
    y = O.linear_ref(xi.astype(np.float16), w_hat)
    assert np.array_equal(y, (xi @ codes.astype(np.int64).T).astype(np.float64))


# --------------------------------------------------------------- act-order

def test_act_order_perm_hand_example():
    g_idx = np.array([1, 0, 0, 1, 2, 2, 0, 1, 2], np.int32)
    perm = O.act_order_perm(g_idx)
    assert list(perm) == [1, 2, 6, 0, 3, 7, 4, 5, 8]
    assert list(g_idx[perm]) == [0, 0, 0, 1, 1, 1, 2, 2, 2]


def test_act_order_group_scales_follow_gidx():
    # Group 0 = the channels g_idx maps to 0 (wherever they are).
    K = 64
    g_idx = np.array([k % 2 for k in range(K)], np.int32)   # even -> 0, odd -> 1
    w = np.zeros((1, K), np.float16)
    w[0, 0::2] = np.linspace(-1, 1, 32)
    w[0, 1::2] = np.linspace(-3, 3, 32)
    _, scales, _ = O.rtn_quantize(w, 4, 32, g_idx=g_idx)
    assert np.allclose(scales[0].astype(np.float64), [2 / 15, 6 / 15], rtol=1e-3)


def test_act_order_permutation_invariance():
    # Relabelling input channels consistently in x, W and g_idx leaves the
    # output unchanged, and the packed words only depend on the packed order.
    M, N, K, gs, bits = 3, 8, 256, 32, 3
    seed = (61,)
    x = I.activations(seed, M, K)
    w = I.weights(seed, N, K, 0.02)
    g_idx = I.act_order_gidx(seed, K, gs)
    q = O.quantize_linear_layer(w, bits, gs, g_idx=g_idx, symmetric=True)
    y = O.linear_ref(x, q["w_hat"])
    sigma = np.random.default_rng(62).permutation(K)
    q2 = O.quantize_linear_layer(w[:, sigma], bits, gs, g_idx=g_idx[sigma], symmetric=True)
    y2 = O.linear_ref(x[:, sigma], q2["w_hat"])
    assert np.max(np.abs(y - y2)) <= 1e-12 * np.max(np.abs(y))
    # unpacking the packed words and undoing perm gives the original codes
    unp = O.unpack(q["packed"], bits, K)
    back = np.empty_like(unp)
    back[:, q["perm"]] = unp
    assert np.array_equal(back, q["codes"])
    # groups are contiguous in packed order
    assert np.array_equal(g_idx[q["perm"]], np.arange(K) // gs)


# ------------------------------------------------------- AWQ clip search --

def test_awq_clip_ratio_grid_closed_form():
    r = O.awq_clip_ratios(20, 10)
    assert r.dtype == np.float32
    assert np.array_equal(r, np.array([1.0, 0.95, 0.9, 0.85, 0.8, 0.75, 0.7, 0.65, 0.6, 0.55], dtype=np.float32))
    with pytest.raises(ValueError):
        O.awq_clip_ratios(20, 21)


def test_awq_clip_on_grid_weights_keep_full_range():
    # Weights on the RTN grid of their own range (asymmetric, 4 bits:
    # values -1 .. 0.875 in steps of 0.125) quantize exactly at ratio 1,
    # so the loss there is exactly 0 and any clipping can only add error.
    vals = (np.arange(16) - 8) * 0.125
    w = np.tile(vals, 4).reshape(2, 32).astype(np.float16)
    w[1] = w[1][::-1]
    x = I.activations((60,), 8, 32)
    r = O.awq_clip_search(x, w, 4, 32)
    assert np.all(r["losses"][:, :, 0] == 0.0)
    assert np.all(r["losses"][:, :, 1:] > 0.0)
    assert np.all(r["best"] == 0)
    assert np.array_equal(r["w_clip"].view(np.uint16), w.view(np.uint16))


def test_awq_clip_zero_activations_pick_first_ratio():
    w = I.weights((61,), 3, 64, 0.02)
    x = np.zeros((4, 64), dtype=np.float16)
    r = O.awq_clip_search(x, w, 3, 32, symmetric=True)
    assert np.all(r["losses"] == 0.0) and np.all(r["best"] == 0)


def test_awq_clip_outlier_prefers_a_threshold():
    # One weight far out in a group of small ones, on an input channel whose
    # activations are tiny: at ratio 1 the step is set by the outlier and
    # every other weight rounds coarsely; clipping costs little on that
    # channel and gives all others a finer step.
    g = np.random.default_rng([62])
    w = (0.01 * g.standard_normal((4, 128))).astype(np.float16)
    w[:, 17] = np.float16(0.3)
    x = I.activations((62,), 64, 128)
    x[:, 17] = (x[:, 17].astype(np.float32) * 0.01).astype(np.float16)
    r = O.awq_clip_search(x, w, 3, 128)
    assert np.all(r["best"] > 0)
    L = r["losses"][:, 0, :]
    assert np.all(L[np.arange(4), r["best"][:, 0]] < 0.8 * L[:, 0])
    t = np.abs(r["w_clip"].astype(np.float32)).max(axis=1)
    assert np.all(t < 0.3)


def _clip_loss_brute(x, w, bits, gs, ratio_idx, n_grid, symmetric):
    # scalar loops, the RTN rule written out for one group at a time
    qmax = (1 << bits) - 1
    M, K = x.shape
    N = w.shape[0]
    out = np.zeros((N, K // gs))
    r = np.float32(1.0 - ratio_idx / n_grid)
    for n in range(N):
        for g in range(K // gs):
            ks = range(g * gs, (g + 1) * gs)
            amax = max(abs(float(w[n, k])) for k in ks)
            t = float(np.float16(np.float32(r) * np.float32(amax)))
            wc = [min(max(float(w[n, k]), -t), t) for k in ks]
            if symmetric:
                s = float(np.float16(np.float32(2.0) * np.float32(max(abs(v) for v in wc)) / np.float32(qmax)))
                z = float(1 << (bits - 1))
            else:
                lo, hi = min(wc), max(wc)
                s = float(np.float16((np.float32(hi) - np.float32(lo)) / np.float32(qmax)))
            if s == 0.0:
                s = 2.0 ** -14
            if not symmetric:
                z = min(max(float(np.rint(np.float32(-lo) / np.float32(s))), 0.0), float(qmax))
            d = []
            for k, v in zip(ks, wc):
                q = min(max(float(np.rint(np.float32(v) / np.float32(s))) + z, 0.0), float(qmax))
                wh = float(np.float16(np.float32(q - z) * np.float32(s)))
                d.append(float(w[n, k]) - wh)
            tot = 0.0
            for m in range(M):
                acc = 0.0
                for j, k in enumerate(ks):
                    acc += float(x[m, k]) * d[j]
                tot += acc * acc
            out[n, g] = tot
    return out


@pytest.mark.parametrize("bits,sym", [(4, False), (3, True), (2, False)])
def test_awq_clip_losses_match_brute_force(bits, sym):
    seed = (63, bits)
    x = I.activations(seed, 3, 64)
    w = I.weights(seed, 2, 64, 0.02)
    w[0, 5] = np.float16(0.12)
    r = O.awq_clip_search(x, w, bits, 32, n_grid=20, n_ratios=10, symmetric=sym)
    for i in (0, 3, 9):
        b = _clip_loss_brute(x, w, bits, 32, i, 20, sym)
        assert np.allclose(r["losses"][:, :, i], b, rtol=1e-12, atol=1e-18)


def test_bias_closed_forms():
    # zero activations give the bias itself; a unit activation on channel j
    # gives column j of w_hat plus the bias; silu(b_g) * b_u for x = 0
    w_hat = np.array([[0.5, -1.0], [2.0, 0.25], [0.0, 1.5], [-0.75, 1.0]], dtype=np.float16)
    b = np.array([0.125, -2.0, 1.0, 3.0], dtype=np.float16)
    assert np.array_equal(O.linear_ref(np.zeros((1, 2), np.float16), w_hat, bias=b)[0], b.astype(np.float64))
    y = O.linear_ref(np.array([[0.0, 1.0]], np.float16), w_hat, bias=b)[0]
    assert np.array_equal(y, np.array([-1.0 + 0.125, 0.25 - 2.0, 1.5 + 1.0, 1.0 + 3.0]))
    z = O.silu_mul_ref(np.zeros((1, 2), np.float16), w_hat, bias=b)[0]
    assert np.allclose(z, [0.125 / (1 + np.exp(-0.125)) * 1.0, -2.0 / (1 + np.exp(2.0)) * 3.0], rtol=1e-15)


def test_gptq_act_order_with_diagonal_hessian_is_rtn_in_rank_groups():
    # x = diag(c) with distinct c: H is diagonal, nothing is carried, the
    # processing order is c descending, and the result is plain RTN with the
    # groups given by that order
    K, N, gs = 128, 24, 32
    seed = (51,)
    w = I.weights(seed, N, K, 0.02)
    c = 1.0 + np.random.default_rng([51]).permutation(K) / 16.0      # distinct, exact in fp16
    x = np.diag(c).astype(np.float16)
    r = O.gptq_quantize(w, x, 4, gs, act_order=True)
    order = np.argsort(-c, kind="stable")
    want_g = np.empty(K, dtype=np.int32)
    want_g[order] = np.arange(K) // gs
    assert np.array_equal(r["g_idx"], want_g)
    rc, rs, rz = O.rtn_quantize(w, 4, gs, g_idx=want_g)
    assert np.array_equal(r["codes"], rc)
    assert np.array_equal(r["scales"].view(np.uint16), rs.view(np.uint16))
    assert np.array_equal(r["zeros"], rz)


def test_gptq_act_order_is_fixed_order_on_the_permuted_problem():
    # act-order GPTQ equals fixed-order GPTQ run on the inputs permuted into
    # descending diag(H), mapped back to the original channels
    K, N, M, gs = 96, 16, 256, 32
    seed = (52,)
    g = np.random.default_rng([52])
    x = (I.correlated_activations(seed, M, K).astype(np.float32) * (0.5 + g.random(K))).astype(np.float16)
    w = I.weights(seed, N, K, 0.02)
    r = O.gptq_quantize(w, x, 3, gs, act_order=True)
    d = np.sum(x.astype(np.float64) ** 2, axis=0)
    order = np.argsort(-d, kind="stable")
    f = O.gptq_quantize(w[:, order], x[:, order], 3, gs)
    assert np.array_equal(r["codes"][:, order], f["codes"])
    assert np.array_equal(r["scales"].view(np.uint16), f["scales"].view(np.uint16))
    assert np.array_equal(r["g_idx"][order], np.arange(K) // gs)
    assert not np.array_equal(order, np.arange(K))
