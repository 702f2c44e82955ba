"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random tensors and builds the workload's structure
(weights, activations, outlier channels, the act-order group map).  It holds
none of the quantization or matmul arithmetic: the CPU oracle and the HIP
library each take these arrays as plain inputs.

Every generator takes an explicit integer seed tuple; numpy's PCG64
`default_rng(seed)` keeps the streams independent, so the weights of a shape
do not change when the number of activation rows does.
"""

from __future__ import annotations

import numpy as np

# Stream identifiers inside a seed tuple.
STREAM_W = 0
STREAM_X = 1
STREAM_AUX = 2


def rng(*seed: int) -> np.random.Generator:
    return np.random.default_rng(list(seed))


def weights(seed: tuple, N: int, K: int, sigma: float) -> np.ndarray:
    """fp16 W[N][K] with entries fp16(sigma * N(0,1)), drawn in fp32."""
    g = rng(*seed, STREAM_W)
    w = g.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(sigma)
    return w.astype(np.float16)


def activations(seed: tuple, M: int, K: int) -> np.ndarray:
    """fp16 x[M][K] with entries fp16(N(0,1)), drawn in fp32."""
    g = rng(*seed, STREAM_X)
    return g.standard_normal((M, K), dtype=np.float32).astype(np.float16)


def outlier_channels(seed: tuple, K: int, fraction: float = 0.01) -> np.ndarray:
    """Sorted indices of round(fraction * K) distinct input channels."""
    g = rng(*seed, STREAM_AUX)
    n_out = int(round(fraction * K))
    return np.sort(g.choice(K, size=n_out, replace=False))


def with_outliers(x: np.ndarray, channels: np.ndarray, factor: float = 20.0) -> np.ndarray:
    """Copy of x with the given input channels multiplied by `factor`
    (computed in fp32, stored as fp16): the salient-channel activation
    pattern of the prefill workload."""
    y = x.copy()
    y[:, channels] = (x[:, channels].astype(np.float32) * np.float32(factor)).astype(np.float16)
    return y


def correlated_activations(seed: tuple, M: int, K: int, rank: int = 16, strength: float = 1.0) -> np.ndarray:
    """fp16 x[M][K] = z + strength * f . V with z, f, V standard normal (z
    [M][K], f [M][rank], V [rank][K] / sqrt(rank)), drawn and summed in
    fp32: input channels correlated through a shared low-rank component, so
    the calibration Hessian x^T x has large off-diagonal entries."""
    g = rng(*seed, STREAM_X, 1)
    z = g.standard_normal((M, K), dtype=np.float32)
    f = g.standard_normal((M, rank), dtype=np.float32)
    v = g.standard_normal((rank, K), dtype=np.float32) / np.float32(np.sqrt(rank))
    return (z + np.float32(strength) * (f @ v)).astype(np.float16)


def act_order_gidx(seed: tuple, K: int, group_size: int) -> np.ndarray:
    """Act-order group map: g_idx[k] = pi[k] // group_size for a seeded random
    permutation pi of the K input channels (equal-size groups)."""
    g = rng(*seed, STREAM_AUX)
    pi = g.permutation(K)
    return (pi // group_size).astype(np.int32)


def random_codes(seed: tuple, N: int, K: int, bits: int) -> np.ndarray:
    """Uniform random b-bit codes, for packing tests."""
    g = rng(*seed, STREAM_AUX)
    return g.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
