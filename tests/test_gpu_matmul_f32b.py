"""GPU parity of mx_block_matmul_f32b (block-scaled A times an ordinary
float32 B) against the oracle.

Bound, per output element: |gpu - oracle| <= 1e-5 * sum_k |a_k b_k|
(+ |C_in| when accumulating), the matmul tolerance of the quantized path,
with identical NaN positions and exact zeros where the bound is 0.  Shapes
cover every launch shape (16x16 tiles with K split over the waves, operands
loaded element-wise or streamed through LDS; 128x64 tiles on the float32
matrix cores, and on the bf16 ones with B split into exact parts, including
the values that split cannot carry), ragged M, N and
K, a B that is not 16-byte aligned, and the two measured workloads in full: decode
(MXFP4 weights 4096x4096 times float32 activations 4096x16) and the square
4096^3 product.
"""
import numpy as np
import pytest
import torch

from bit_gemm_mx_amd import binding as B
from bit_gemm_mx_amd import workloads as W
from oracle import mx_oracle as O

from gpu_util import assert_matmul_close, dev, host

pytestmark = pytest.mark.gpu

ELEMS = [O.E2M1, O.E4M3]


def rand_a(rng, M, K, elem, lo=110, hi=145):
    if elem == O.E2M1:
        codes = O.pack_nibbles(rng.integers(0, 16, (M, K), dtype=np.uint8))
    else:
        el = rng.integers(0, 256, (M, K), dtype=np.uint8)
        el[(el & 0x7F) == 0x7F] = 0x38
        codes = el
    return codes, rng.integers(lo, hi, (M, K // 32), dtype=np.uint8)


def rand_b(rng, K, N):
    b = rng.standard_normal((K, N)).astype(np.float32)
    return b * np.exp2(rng.integers(-20, 20, (1, N))).astype(np.float32)


def run(ac, asc, elem, b, M, N, K, c_in=None, accumulate=False):
    a = B.MXTensor(dev(ac), dev(asc), M, K, elem)
    out = dev(c_in.astype(np.float32)) if c_in is not None else None
    return host(B.block_matmul_f32b(a, dev(b), out=out, accumulate=accumulate))


SHAPES = [(1, 1, 32), (3, 5, 64), (16, 16, 128), (17, 33, 160), (70, 100, 1056), (5, 7, 8192),
          (300, 520, 2048), (1024, 1024, 512), (1030, 1100, 320), (64, 2048, 96),
          (2100, 1100, 320), (2048, 2048, 1024)]
# Shapes for the 128x64-tile launch on the bf16 matrix cores (at least 256
# tiles, K % 128 == 0, N % 4 == 0): N ragged within a 64-column tile (a
# wave's columns past N read the next B row), M ragged, one group of four
# blocks (K = 128) so the load ring runs past K, K not a multiple of 512.
BF16_SHAPES = [(2048, 1028, 384), (2000, 2048, 640), (4096, 1024, 128), (1100, 2052, 256)]
# Shapes for the streamed K-split launch (K % 256 == 0, N % 4 == 0, few tiles):
# one 256-K unit (15 of 16 waves idle), units not a multiple of 16, ragged M,
# N = 4 and column tiles cut short of 16, the decode shape's K at small M.
STREAM_SHAPES = [(1, 4, 256), (17, 20, 256), (33, 4, 4352), (100, 36, 8448), (5, 12, 4096),
                 (130, 68, 1280)]


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("M,N,K", SHAPES + STREAM_SHAPES + BF16_SHAPES)
def test_random_operands(elem, M, N, K):
    rng = np.random.default_rng(M * 131 + N * 7 + K + elem)
    ac, asc = rand_a(rng, M, K, elem)
    b = rand_b(rng, K, N)
    got = run(ac, asc, elem, b, M, N, K)
    want, mag = O.block_matmul_f32b(ac, asc, elem, b, M, N, K)
    assert_matmul_close(got, want, mag)


@pytest.mark.parametrize("elem", ELEMS)
def test_quantized_float_weights(elem):
    # weights quantized on the GPU (the usual producer of A), float32 activations
    rng = np.random.default_rng(3)
    M, N, K = 200, 48, 2048
    w = W.normal_with_outliers(rng, (M, K), 0.02, 0.001, 50.0)
    x = rng.standard_normal((K, N)).astype(np.float32)
    a = B.quantize(dev(w), elem)
    got = host(B.block_matmul_f32b(a, dev(x)))
    ac, asc = O.quantize(w, elem)
    want, mag = O.block_matmul_f32b(ac, asc, elem, x, M, N, K)
    assert_matmul_close(got, want, mag)


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("M,N,K", [(20, 30, 96), (1100, 300, 256), (40, 20, 1024),
                                   (2048, 1024, 256)])
def test_accumulate(elem, M, N, K):
    rng = np.random.default_rng(M + N + K)
    ac, asc = rand_a(rng, M, K, elem)
    b = rand_b(rng, K, N)
    cin = (rng.standard_normal((M, N)) * 1e5).astype(np.float32)
    got = run(ac, asc, elem, b, M, N, K, c_in=cin, accumulate=True)
    want, mag = O.block_matmul_f32b(ac, asc, elem, b, M, N, K, c_in=cin, accumulate=True)
    assert_matmul_close(got, want, mag)


def test_accumulate_zero_does_not_read_c():
    rng = np.random.default_rng(4)
    M, N, K = 33, 17, 64
    ac, asc = rand_a(rng, M, K, O.E2M1)
    b = rand_b(rng, K, N)
    got = run(ac, asc, O.E2M1, b, M, N, K, c_in=np.full((M, N), np.nan, np.float32))
    want, mag = O.block_matmul_f32b(ac, asc, O.E2M1, b, M, N, K)
    assert_matmul_close(got, want, mag)


@pytest.mark.parametrize("elem", ELEMS)
def test_nan_scales_codes_and_b(elem):
    rng = np.random.default_rng(5)
    M, N, K = 40, 36, 256
    ac, asc = rand_a(rng, M, K, elem)
    asc[3, 2] = 0xFF
    if elem == O.E4M3:
        ac[9, 100] = 0xFF
    b = rand_b(rng, K, N)
    b[17, 5] = np.nan
    got = run(ac, asc, elem, b, M, N, K)
    want, mag = O.block_matmul_f32b(ac, asc, elem, b, M, N, K)
    assert np.isnan(want).sum() > 0
    assert_matmul_close(got, want, mag)


@pytest.mark.parametrize("elem", ELEMS)
def test_square_shape_values_outside_the_bf16_split(elem):
    """The 128x64-tile launch multiplies on the bf16 matrix cores, B split
    into three exact bf16 parts; a block holding a value that split cannot
    carry exactly runs the float32 MFMAs.  Planted: A scale bytes 0, 1, 2
    (E4M3 codes there decode below the bf16 subnormals) and a NaN scale; B
    values whose last bits fall below the bf16 subnormals (a normal value
    near 2^-120 and a float32 subnormal), +Inf, -Inf and a NaN.  Every output
    against the oracle: infinities equal, NaN positions equal, the rest
    within the tolerance."""
    rng = np.random.default_rng(21 + elem)
    M, N, K = 2048, 1024, 512
    ac, asc = rand_a(rng, M, K, elem)
    asc[5, 3], asc[77, 0], asc[1500, 15] = 0, 1, 2      # rows of three different waves
    asc[900, 7] = 0xFF
    b = rand_b(rng, K, N)
    b[100, 3] = np.float32(1.2345 * 2.0 ** -120)
    b[200, 500] = np.float32(3e-41)
    b[300, 700] = np.inf
    b[301, 701] = -np.inf
    b[400, 900] = np.nan
    got = run(ac, asc, elem, b, M, N, K)
    want, mag = O.block_matmul_f32b(ac, asc, elem, b, M, N, K)
    inf = np.isinf(want)
    assert inf.sum() > 100 and np.isnan(want[900]).all() and np.isnan(want[:, 900]).all()
    np.testing.assert_array_equal(got[inf], want[inf])
    assert_matmul_close(np.where(inf, 0, got), np.where(inf, 0, want), np.where(inf, 0, mag))


@pytest.mark.parametrize("elem", ELEMS)
def test_square_shape_one_signed_operands(elem):
    """Positive A and B: every product has the same sign, so the matrix
    cores' truncation of each partial sum below its largest term (2^-24) does
    not cancel across products or K steps.  The bf16 launch keeps a tile's sum
    in the MFMA accumulator for four blocks (twelve MFMAs) before adding it in
    float32; K = 8192 gives 64 such groups per output.  Every output within
    the tolerance, and the worst one well inside it."""
    rng = np.random.default_rng(31 + elem)
    M, N, K = 2048, 1024, 8192
    if elem == O.E2M1:
        el = rng.integers(1, 8, (M, K), dtype=np.uint8)                 # positive codes
        ac = O.pack_nibbles(el)
    else:
        ac = rng.integers(1, 0x7F, (M, K), dtype=np.uint8)              # positive, no NaN
    asc = rng.integers(110, 145, (M, K // 32), dtype=np.uint8)
    b = np.abs(rand_b(rng, K, N))
    got = run(ac, asc, elem, b, M, N, K)
    want, mag = O.block_matmul_f32b(ac, asc, elem, b, M, N, K)
    worst = assert_matmul_close(got, want, mag)
    print(f"one-signed operands, elem {elem}: worst error {worst:.3g} of the tolerance")
    assert worst < 0.5, f"worst error {worst:.3g} of the tolerance"


def test_zero_rows_and_identity():
    rng = np.random.default_rng(6)
    M, K = 48, 64
    ac, asc = rand_a(rng, M, K, O.E4M3)
    ac[5] = 0
    got = run(ac, asc, O.E4M3, np.eye(K, dtype=np.float32), M, K, K)
    assert np.array_equal(got, O.dequantize(ac, asc, O.E4M3, K))     # -0.0 sums to +0.0
    assert np.all(got[5] == 0)


def exhaustive_a(elem, M, K):
    """Rows cycling through every scale byte whose decoded values stay finite
    (E2M1 up to 252: 6 * 2^125; E4M3 up to 246: 448 * 2^119) and, along K,
    every finite code (E4M3's two NaN codes replaced by zero)."""
    top = 252 if elem == O.E2M1 else 246
    scales = (np.arange(M * (K // 32)).reshape(M, K // 32) // (K // 32) % (top + 1)).astype(np.uint8)
    el = (np.arange(K) % (16 if elem == O.E2M1 else 256)).astype(np.uint8)
    if elem == O.E4M3:
        el[(el & 0x7F) == 0x7F] = 0
    el = np.tile(el, (M, 1))
    codes = O.pack_nibbles(el) if elem == O.E2M1 else el
    return codes, scales


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("M,K", [(256, 256), (2048, 1024), (2048, 1056)])
def test_identity_b_decodes_every_code_and_scale_exactly(elem, M, K):
    """C = A . I is A's exact decode (each output is one product with 1 plus
    zeros), so this pins the in-register decode -- the hardware's scaled
    converts to float32, and to bf16 on the bf16 matrix cores -- value for
    value, for every finite code at every scale byte that keeps it finite,
    subnormal results included.  256 rows take the K-split launch shape,
    2048 x 1024 the 128x64-tile shape on the bf16 matrix cores (E4M3 rows at
    scale bytes 0..2 on the float32 ones), 2048 x 1056 (K not a multiple of
    128) the 128x64-tile shape on the float32 matrix cores."""
    ac, asc = exhaustive_a(elem, M, K)
    got = run(ac, asc, elem, np.eye(K, dtype=np.float32), M, K, K)
    want = O.dequantize(ac, asc, elem, K)
    assert not np.isnan(want).any()
    np.testing.assert_array_equal(got, want)   # values: -0.0 sums to +0.0


def test_agrees_with_quantized_b_product():
    # B holding the dequantized values of a quantized B^T: both entry points
    # compute the same product
    rng = np.random.default_rng(7)
    M, N, K = 300, 260, 1024
    ac, asc = rand_a(rng, M, K, O.E2M1)
    bc, bsc = rand_a(rng, N, K, O.E4M3)
    b = np.ascontiguousarray(O.dequantize(bc, bsc, O.E4M3, K).T)
    got = run(ac, asc, O.E2M1, b, M, N, K)
    want, mag = O.block_matmul(ac, asc, O.E2M1, bc, bsc, O.E4M3, M, N, K)
    assert_matmul_close(got, want, mag)


def test_decode_weights_only_full():
    """MXFP4 weights 4096x4096 times float32 activations 4096x16, every output."""
    w, x = W.f32b_decode_case()
    a = B.quantize(dev(w), O.E2M1)
    got = host(B.block_matmul_f32b(a, dev(x)))
    ac, asc = host(a.codes), host(a.scales)
    want, mag = O.block_matmul_f32b(ac, asc, O.E2M1, x, 4096, 16, 4096)
    assert_matmul_close(got, want, mag)


def test_square_4096_full():
    """MXFP4 A 4096x4096 times float32 B 4096x4096, every output."""
    w, x = W.f32b_square_case()
    a = B.quantize(dev(w), O.E2M1)
    got = host(B.block_matmul_f32b(a, dev(x)))
    ac, asc = host(a.codes), host(a.scales)
    del a
    torch.cuda.empty_cache()
    want, mag = O.block_matmul_f32b(ac, asc, O.E2M1, x, 4096, 4096, 4096)
    assert_matmul_close(got, want, mag)


@pytest.mark.parametrize("elem", ELEMS)
def test_b_not_16_byte_aligned(elem):
    """A B that starts 4 bytes past a 16-byte boundary cannot take the streamed
    launch's 16-byte loads; the call must still give the oracle's result."""
    rng = np.random.default_rng(11)
    M, N, K = 64, 16, 1024
    ac, asc = rand_a(rng, M, K, elem)
    b = rand_b(rng, K, N)
    buf = torch.zeros(K * N + 4, dtype=torch.float32, device="cuda")
    bd = buf[1:1 + K * N].view(K, N)
    bd.copy_(dev(b))
    assert bd.data_ptr() % 16 == 4
    a = B.MXTensor(dev(ac), dev(asc), M, K, elem)
    got = host(B.block_matmul_f32b(a, bd))
    want, mag = O.block_matmul_f32b(ac, asc, elem, b, M, N, K)
    assert_matmul_close(got, want, mag)
