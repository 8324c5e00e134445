"""block_matmul at the top of the E8M0 range: outputs that round to +-Inf.

"Bit Layout", section "The E8M0 shared scale": a scale byte s is 2^(s-127),
up to 2^127.  The product's definition ("A Dialect Is a Set of Co-Designed
Decisions", section "The four ops") is the exact sum rounded to float32, so
an output whose exact value exceeds the largest float32 is +-Inf and one just
below it is finite.  Operands hold one code everywhere (every product of a
row and column pair equal, so no summation order or group truncation
matters); the scale bytes of rows and columns are chosen so that the exact
outputs fall on both sides of the overflow threshold (0.56 to 0.79 of the
largest float32 just below it, 1.1 to 1.6 times it just above), and at
ordinary magnitudes.  A last case has the product of two block scales beyond
the float32 range while the output, a product of small codes, is not.  The
f32-B product is taken with A values up to the top of the float32 range, and
past it, where it decodes A as mx_dequantize does.
"""
import numpy as np
import pytest

from bit_gemm_mx_amd import binding as B
from oracle import mx_oracle as O

from gpu_util import assert_matmul_close, dev, gpu_matmul, host

pytestmark = pytest.mark.gpu

TOP = {O.E2M1: 0x7, O.E4M3: 0x7E}      # 6.0 and 448, the largest magnitudes
# s_a + s_b at which the exact output first exceeds the largest float32, for
# K = 1024 or 1056 (32 or 33 blocks of the top code squared):
# 2^(s - 254) * blocks * 32 * top_a * top_b crosses 2^128 between s - 1 and s.
FIRST_INF = {(O.E2M1, O.E2M1): 367, (O.E4M3, O.E4M3): 355, (O.E4M3, O.E2M1): 361,
             (O.E2M1, O.E4M3): 361}


def uniform_operand(rows, K, elem, scale_bytes, negative_rows=()):
    code = np.full((rows, K), TOP[elem], np.uint8)
    code[list(negative_rows)] |= 0x8 if elem == O.E2M1 else 0x80
    codes = O.pack_nibbles(code) if elem == O.E2M1 else code
    return codes, np.repeat(np.asarray(scale_bytes, np.uint8).reshape(rows, 1), K // 32, axis=1)


def check(got, want, mag):
    inf = np.isinf(want)
    assert inf.any() and (~inf).any()
    assert np.array_equal(got[inf], want[inf]), "an overflowing output is not the same infinity"
    assert_matmul_close(np.where(inf, 0.0, got), np.where(inf, 0.0, want), np.where(inf, 0.0, mag))


@pytest.mark.parametrize("ae,be", list(FIRST_INF))
@pytest.mark.parametrize("M,N,K", [(16, 64, 1024), (17, 36, 1056), (300, 257, 1024),
                                   (200, 70, 1056)])
def test_overflow_threshold(ae, be, M, N, K):
    s = FIRST_INF[(ae, be)]
    h = s // 2
    # rows: 127, h - 1 (finite with every column but the top one), h, 254
    sa = np.array([127, h - 1, h, 254])[np.arange(M) % 4]
    # columns: 127, s - 1 - h (sum s - 1 with row h: finite, just below 2^128),
    # s - h (sum s with row h: Inf), 60 (finite even with row 254)
    sb = np.array([127, s - 1 - h, s - h, 60])[np.arange(N) % 4]
    ac, asc = uniform_operand(M, K, ae, sa)
    bc, bsc = uniform_operand(N, K, be, sb, negative_rows=range(1, N, 3))
    got = gpu_matmul(ac, asc, ae, bc, bsc, be, M, N, K)
    want, mag = O.block_matmul(ac, asc, ae, bc, bsc, be, M, N, K)
    check(got, want, mag)


# Largest scale byte at which the top code still decodes to a float32 value:
# 6 * 2^125 and 448 * 2^119 (the largest bytes mx_quantize writes).
F32_TOP_BYTE = {O.E2M1: 252, O.E4M3: 246}


@pytest.mark.parametrize("elem", [O.E2M1, O.E4M3])
def test_f32b_overflow(elem):
    """The f32-B product with A values up to the top of the float32 range
    and B values of 2^100 (outputs far past the largest float32: +-Inf) or
    2^-60 (finite); every product stays in the normal float32 range or
    beyond it (a product below it rounds to zero or a subnormal in the
    kernels' float32 arithmetic)."""
    M, N, K = 70, 100, 1056
    sa = np.array([127, 200, F32_TOP_BYTE[elem], 100])[np.arange(M) % 4]
    ac, asc = uniform_operand(M, K, elem, sa)
    b = np.full((K, N), 2.0 ** 100, np.float32)
    b[:, ::3] *= -1
    b[:, 1::5] = 2.0 ** -60
    a = B.MXTensor(dev(ac), dev(asc), M, K, elem)
    got = host(B.block_matmul_f32b(a, dev(b)))
    want, mag = O.block_matmul_f32b(ac, asc, elem, b, M, N, K)
    check(got, want, mag)


@pytest.mark.parametrize("elem", [O.E2M1, O.E4M3])
def test_f32b_a_beyond_float32_decodes_to_infinity(elem):
    """The f32-B product decodes A to float32 as mx_dequantize does, so an A
    value beyond the float32 range (the top code at a scale byte above
    F32_TOP_BYTE, which mx_quantize never writes) is +-Inf there: every
    output of its row is +-Inf or NaN, even where the exact sum with a tiny B
    is finite.  The rows below that byte hold the stated tolerance."""
    M, N, K = 70, 100, 1056
    sa = np.array([127, F32_TOP_BYTE[elem] + 1, 254, 60])[np.arange(M) % 4]
    ac, asc = uniform_operand(M, K, elem, sa)
    b = np.full((K, N), 2.0 ** -60, np.float32)
    b[:, ::3] *= -1
    a = B.MXTensor(dev(ac), dev(asc), M, K, elem)
    got = host(B.block_matmul_f32b(a, dev(b)))
    want, mag = O.block_matmul_f32b(ac, asc, elem, b, M, N, K)
    beyond = sa > F32_TOP_BYTE[elem]
    assert np.all(np.isfinite(want)), "the exact outputs are all finite"
    assert np.all(~np.isfinite(got[beyond])), "rows with A beyond float32 are +-Inf or NaN"
    assert_matmul_close(got[~beyond], want[~beyond], mag[~beyond])


@pytest.mark.parametrize("elem", [O.E2M1, O.E4M3])
@pytest.mark.parametrize("M,N,K", [(70, 100, 1056), (2048, 1028, 384), (33, 4, 4352)])
def test_f32b_products_below_the_normal_range(elem, M, N, K):
    """The three f32-B kernels (fp32 matrix cores, bf16 split, streamed
    K-split) with products far below the normal float32 range (A at scale
    byte 30 times B = 2^-60: 2^-157 and smaller) beside ordinary ones: every
    output within the stated tolerance plus the header's underflow term,
    2^-146 per product."""
    rng = np.random.default_rng(M + N + K + elem)
    sa = np.array([127, 30, 100, 30])[np.arange(M) % 4]
    ac, asc = uniform_operand(M, K, elem, sa)
    b = np.where(rng.random((K, N)) < 0.5, 2.0 ** -60, 1.0).astype(np.float32)
    b[:, ::3] *= -1
    a = B.MXTensor(dev(ac), dev(asc), M, K, elem)
    got = host(B.block_matmul_f32b(a, dev(b)))
    want, mag = O.block_matmul_f32b(ac, asc, elem, b, M, N, K)
    err = np.abs(got.astype(np.float64) - want)
    bound = 1e-5 * mag + K * 2.0 ** -146
    assert np.all(err <= bound), f"worst err / bound {np.max(err / bound):.3g}"


SMALL = {O.E2M1: (0x1, 0.5), O.E4M3: (0x01, 2.0 ** -9)}   # smallest nonzero magnitudes


@pytest.mark.parametrize("ae,be", list(FIRST_INF))
@pytest.mark.parametrize("M,N,K", [(16, 64, 1024), (300, 257, 1024), (200, 70, 1056)])
def test_scale_product_beyond_float32_with_small_codes(ae, be, M, N, K):
    """One nonzero product per output, the two smallest nonzero codes, and
    block scales whose product 2^(sa+sb-254) exceeds the largest float32
    (2^129 .. 2^145) while the output stays finite (2^127 or below); a few
    columns take a scale one step larger, so that their outputs overflow
    only by the codes' product."""
    ca, va = SMALL[ae]
    cb, vb = SMALL[be]
    e_codes = int(np.log2(va * vb))                  # -2 .. -18
    # sa + sb - 254 + e_codes = 127 exactly: the finite outputs are 2^127
    s = 254 + 127 - e_codes
    sa = np.full(M, 254)
    sb = np.full(N, s - 254)
    sb[::7] += 1                                     # 2^128: Inf
    a = np.zeros((M, K), np.uint8)
    b = np.zeros((N, K), np.uint8)
    a[:, 5] = ca
    b[:, 5] = cb
    b[1::4, 5] |= 0x8 if be == O.E2M1 else 0x80
    ac = O.pack_nibbles(a) if ae == O.E2M1 else a
    bc = O.pack_nibbles(b) if be == O.E2M1 else b
    asc = np.repeat(sa.astype(np.uint8).reshape(M, 1), K // 32, axis=1)
    bsc = np.repeat(sb.astype(np.uint8).reshape(N, 1), K // 32, axis=1)
    got = gpu_matmul(ac, asc, ae, bc, bsc, be, M, N, K)
    want, mag = O.block_matmul(ac, asc, ae, bc, bsc, be, M, N, K)
    assert np.all(np.abs(want[:, 1:7][np.isfinite(want[:, 1:7])]) == 2.0 ** 127)
    check(got, want, mag)


@pytest.mark.parametrize("ae,be", list(FIRST_INF))
@pytest.mark.parametrize("M,N,K", [(16, 64, 1024), (17, 36, 1056), (300, 257, 1024),
                                   (200, 70, 1056)])
def test_outputs_in_the_float32_subnormal_range(ae, be, M, N, K):
    """Scale bytes at the bottom of the E8M0 range: the exact outputs run
    through the float32 subnormals (from below half the smallest one, zero,
    for E2M1 x E2M1) to normal values.  Below the normal float32 range the
    matrix instruction keeps each scaled contribution only on a grid near
    the smallest subnormals (measured: at most 3.1 * 2^-149 per block of K
    beyond the stated tolerance), so the bound here adds the header's
    underflow term, 2^-146 per block.  Normal outputs hold the stated
    tolerance alone."""
    sa = 40 + 4 * (np.arange(M) % 8)
    sb = 40 + 3 * (np.arange(N) % 8)
    ac, asc = uniform_operand(M, K, ae, sa)
    bc, bsc = uniform_operand(N, K, be, sb, negative_rows=range(1, N, 3))
    got = gpu_matmul(ac, asc, ae, bc, bsc, be, M, N, K)
    want, mag = O.block_matmul(ac, asc, ae, bc, bsc, be, M, N, K)
    tiny = np.finfo(np.float32).tiny
    sub = (want != 0) & (np.abs(want) < tiny)
    assert sub.any() and (np.abs(want) >= tiny).any()
    err = np.abs(got.astype(np.float64) - want)
    bound = 1e-5 * mag + (K // 32) * 2.0 ** -146
    assert np.all(err <= bound), f"worst err / bound {np.max(err / bound):.3g}"
    nrm = np.abs(want) >= tiny
    assert_matmul_close(got[nrm], want[nrm], mag[nrm])


@pytest.mark.parametrize("ae,be", [(O.E4M3, O.E2M1), (O.E2M1, O.E2M1), (O.E4M3, O.E4M3)])
def test_quantize_in_product_at_the_ends_of_float32(ae, be):
    """mx_block_matmul_quantize_a with A rows near the largest float32
    (scale bytes 246..252 from the quantize) and rows of subnormal floats
    (scale bytes near 0), against B^T rows at scale bytes 127, 254 and 30:
    outputs past the largest float32 are the same infinity, the others hold
    the stated tolerance plus the underflow term.  (A's values span one
    binade per block, so E4M3 x E4M3 groups stay inside the instruction's
    exact window too; the subnormal rows quantize to zero codes at scale
    byte 0.)"""
    rng = np.random.default_rng(5 + ae + 3 * be)
    M, N, K = 300, 257, 1024
    fmax = float(np.finfo(np.float32).max)
    kind = np.arange(M) % 3
    a = rng.uniform(0.5, 1.0, (M, K))
    a = np.where(kind[:, None] == 0, a * fmax, np.where(kind[:, None] == 1, a * 2.0 ** -140, a))
    # one sign per output (A positive, signs from B's rows): where single
    # products overflow float32, a sum of mixed signs would be order-dependent
    a = a.astype(np.float32)
    sb = np.array([127, 254, 30])[np.arange(N) % 3]
    bc, bsc = uniform_operand(N, K, be, sb, negative_rows=range(1, N, 4))
    bt = B.MXTensor(dev(bc), dev(bsc), N, K, be)
    got = host(B.block_matmul_quantize_a(dev(a), ae, bt))
    ac, asc = O.quantize(a, ae)
    want, mag = O.block_matmul(ac, asc, ae, bc, bsc, be, M, N, K)
    inf = np.isinf(want)
    assert inf.any() and (~inf).any()
    assert np.array_equal(got[inf], want[inf]), "an overflowing output is not the same infinity"
    err = np.abs(got[~inf].astype(np.float64) - want[~inf])
    bound = 1e-5 * mag[~inf] + (K // 32) * 2.0 ** -146
    assert np.all(err <= bound), f"worst err / bound {np.max(err / bound):.3g}"
