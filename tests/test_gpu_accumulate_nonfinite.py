"""Accumulation into a C that holds NaN and infinities.

"A Dialect Is a Set of Co-Designed Decisions", section "The accumulator
operand": C is both input and output and the product is added to it, so each
output is C_in[m, n] + (A.B)[m, n].  With finite operands, a NaN in C_in gives
NaN there and an infinity stays the same infinity; every other output holds
the stated tolerance against the oracle.  Each kernel family is taken: the
skinny decode kernels, the 256x256-tile kernel in both scale-staging modes,
the general kernel (K not a multiple of 128), the three f32-B kernels and the
product with A quantized inside it.
"""
import numpy as np
import pytest

from bit_gemm_mx_amd import binding as B
from oracle import mx_oracle as O

from gpu_util import assert_matmul_close, dev, gpu_matmul, host
from test_gpu_matmul import quantized_normal

pytestmark = pytest.mark.gpu


def c_with_nonfinite(rng, M, N):
    c = (rng.standard_normal((M, N)) * 10).astype(np.float32)
    c[0, 0] = np.nan
    c[M // 2, N - 1] = np.inf
    c[M - 1, N // 2] = -np.inf
    c[:, min(1, N - 1)] = -np.inf          # a whole column
    c[M - 1, 0] = np.nan
    return c


def check(got, want, mag, cin):
    bad = ~np.isfinite(cin)
    assert np.array_equal(np.isnan(got[bad]), np.isnan(cin[bad])), "NaN of C_in not kept"
    inf = np.isinf(cin)
    assert np.array_equal(got[inf], cin[inf]), "infinity of C_in not kept"
    with np.errstate(invalid="ignore"):
        assert_matmul_close(np.where(bad, 0.0, got), np.where(bad, 0.0, want),
                            np.where(bad, 0.0, mag))


@pytest.mark.parametrize("ae,be", [(O.E2M1, O.E2M1), (O.E4M3, O.E2M1), (O.E2M1, O.E4M3)])
@pytest.mark.parametrize("M,N,K", [
    (16, 300, 1024),   # staged skinny decode kernel (M <= 32, K % 128 == 0)
    (17, 33, 160),     # register skinny kernel
    (300, 257, 1024),  # 256x256 tiles, scales per 512-K chunk
    (300, 257, 640),   # 256x256 tiles, scales per stage
    (200, 70, 1056),   # general kernel
])
def test_block_matmul(ae, be, M, N, K):
    rng = np.random.default_rng(M * 7 + N + K + 10 * ae + be)
    ac, asc = quantized_normal(rng, M, K, ae)
    bc, bsc = quantized_normal(rng, N, K, be, sigma=0.02)
    cin = c_with_nonfinite(rng, M, N)
    got = gpu_matmul(ac, asc, ae, bc, bsc, be, M, N, K, c_in=cin, accumulate=True)
    with np.errstate(invalid="ignore"):
        want, mag = O.block_matmul(ac, asc, ae, bc, bsc, be, M, N, K, c_in=cin, accumulate=True)
    check(got, want, mag, cin)


@pytest.mark.parametrize("elem", [O.E2M1, O.E4M3])
@pytest.mark.parametrize("M,N,K", [
    (70, 100, 1056),    # fp32 matrix-core kernel
    (2048, 1028, 384),  # bf16 split kernel (at least 256 tiles of 128x64)
    (33, 4, 4352),      # streamed K-split kernel
])
def test_block_matmul_f32b(elem, M, N, K):
    rng = np.random.default_rng(M + 3 * N + K + elem)
    ac, asc = quantized_normal(rng, M, K, elem)
    b = rng.standard_normal((K, N)).astype(np.float32)
    cin = c_with_nonfinite(rng, M, N)
    a = B.MXTensor(dev(ac), dev(asc), M, K, elem)
    got = host(B.block_matmul_f32b(a, dev(b), out=dev(cin), accumulate=True))
    with np.errstate(invalid="ignore"):
        want, mag = O.block_matmul_f32b(ac, asc, elem, b, M, N, K, c_in=cin, accumulate=True)
    check(got, want, mag, cin)


@pytest.mark.parametrize("ae,be", [(O.E4M3, O.E2M1), (O.E2M1, O.E2M1)])
def test_block_matmul_quantize_a(ae, be):
    rng = np.random.default_rng(41 + ae + be)
    M, N, K = 300, 257, 1024
    a = (rng.standard_normal((M, K)) * 0.5).astype(np.float32)
    bc, bsc = quantized_normal(rng, N, K, be, sigma=0.02)
    cin = c_with_nonfinite(rng, M, N)
    bt = B.MXTensor(dev(bc), dev(bsc), N, K, be)
    got = host(B.block_matmul_quantize_a(dev(a), ae, bt, out=dev(cin), accumulate=True))
    ac, asc = O.quantize(a, ae)
    with np.errstate(invalid="ignore"):
        want, mag = O.block_matmul(ac, asc, ae, bc, bsc, be, M, N, K, c_in=cin, accumulate=True)
    check(got, want, mag, cin)
