"""Seeded synthetic inputs for the MX workloads.

This module holds random-number recipes only -- no quantization arithmetic --
so that both the HIP path (tests, bench) and the CPU oracle (tests) can be fed
the very same arrays.  Every array is NumPy, generated on the host with PCG64
(``numpy.random.default_rng(seed)``).

Recipe (shared by every workload):
  * values  ``rng.standard_normal(size, dtype=float32) * float32(sigma)``
  * outliers: exactly ``round(p * n)`` distinct flat indices drawn with
    ``rng.choice(n, k, replace=False)``, multiplied in place by ``factor``.
  * weights are generated directly in the B^T [N, K] orientation.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def normal_with_outliers(rng: np.random.Generator, shape, sigma: float,
                         outlier_frac: float = 0.0, factor: float = 1.0) -> np.ndarray:
    """N(0, sigma^2) float32 with a fraction of entries scaled by ``factor``."""
    x = rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)
    n = x.size
    k = int(round(outlier_frac * n))
    if k:
        idx = rng.choice(n, k, replace=False)
        x.reshape(-1)[idx] *= np.float32(factor)
    return x


@dataclass
class RoundTripCase:
    """MXFP4 round trip, fp32 256x1024 (seed 1001).

    N(0,1), 1% outliers x100, 4 rows zeroed, and 2 blocks (outside the zero
    rows) whose scale byte is set to 0xFF in the copy used for decoding.
    """
    x: np.ndarray
    zero_rows: np.ndarray
    ff_blocks: np.ndarray      # flat block indices into scales.reshape(-1)


def roundtrip_case(rows: int = 256, cols: int = 1024, seed: int = 1001) -> RoundTripCase:
    rng = np.random.default_rng(seed)
    x = normal_with_outliers(rng, (rows, cols), 1.0, 0.01, 100.0)
    zero_rows = rng.choice(rows, 4, replace=False)
    x[zero_rows] = 0.0
    nb = cols // 32
    allowed = np.array([b for b in range(rows * nb) if (b // nb) not in set(zero_rows.tolist())])
    ff = rng.choice(allowed, 2, replace=False)
    return RoundTripCase(x=x, zero_rows=np.sort(zero_rows), ff_blocks=np.sort(ff))


def weight_codec_case(rows: int = 8192, cols: int = 8192, seed: int = 1002) -> np.ndarray:
    """MXFP4 weight quantize + dequantize: N(0, 0.02), 0.1% outliers x50."""
    rng = np.random.default_rng(seed)
    return normal_with_outliers(rng, (rows, cols), 0.02, 0.001, 50.0)


def decode_matmul_case(M: int = 16, N: int = 4096, K: int = 4096, seed: int = 1003):
    """Decode-shaped MXFP4 x MXFP4: A [M, K] and B^T [N, K], both N(0,1)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((M, K), dtype=np.float32)
    bt = rng.standard_normal((N, K), dtype=np.float32)
    return a, bt


def square_fp8_case(M: int = 8192, N: int = 8192, K: int = 8192, seed: int = 1004):
    """MXFP8 x MXFP8: A [M, K] and B^T [N, K], both N(0,1)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((M, K), dtype=np.float32)
    bt = rng.standard_normal((N, K), dtype=np.float32)
    return a, bt


def prefill_linear_case(M: int = 2048, N: int = 28672, K: int = 8192, seed: int = 1005):
    """LLM linear layer, prefill-shaped: activations A [M, K] N(0,1) with 0.5%
    outliers x20 (quantized on the fly to E4M3) and weights B^T [N, K]
    N(0, 0.02) (pre-quantized to E2M1)."""
    rng = np.random.default_rng(seed)
    a = normal_with_outliers(rng, (M, K), 1.0, 0.005, 20.0)
    bt = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    return a, bt


def f32b_decode_case(M: int = 4096, N: int = 16, K: int = 4096, seed: int = 1006):
    """Weight-only quantization, decode-shaped: weights A [M, K] N(0, 0.02)
    with 0.1% outliers x50 (to be quantized along K) times float32
    activations B [K, N] N(0, 1)."""
    rng = np.random.default_rng(seed)
    a = normal_with_outliers(rng, (M, K), 0.02, 0.001, 50.0)
    b = rng.standard_normal((K, N), dtype=np.float32)
    return a, b


def f32b_square_case(M: int = 4096, N: int = 4096, K: int = 4096, seed: int = 1007):
    """Weight-only quantization, square: A [M, K] N(0, 0.02) times float32
    B [K, N] N(0, 1)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((M, K), dtype=np.float32) * np.float32(0.02)
    b = rng.standard_normal((K, N), dtype=np.float32)
    return a, b
