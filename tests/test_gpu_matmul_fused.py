"""GPU parity of mx_block_matmul_quantize_a (float32 A quantized along K inside
the product, times a block-scaled B) against the oracle.

Two bars:
* the quantization is mx_quantize's, bit for bit: with B^T the identity each
  output is one product q * 1, exact, so C must equal the oracle's
  dequantize(quantize(A)) value for value (every code and scale byte of A, ties,
  saturation, subnormals, zero blocks and the exact fallback included), and
  rows whose blocks hold NaN or Inf must be the oracle's NaN rows;
* the product is mx_block_matmul's: within T1 = 1e-5 * sum_k |a_k b_k| (+ |C_in|)
  of the oracle's block_matmul of the oracle's quantized A for E2M1 x E2M1 and
  the mixed pairs (whose groups of 8 products are summed exactly), and bit for
  bit equal to quantize() followed by block_matmul() where that product runs
  the tiled kernel (same MFMA sequence per output), the prefill workload in full.
E4M3 x E4M3 shares the FP8 instruction's group truncation with mx_block_matmul:
checked for NaN positions and against T1 plus the instruction's truncation bound.
"""
import numpy as np
import pytest
import torch

from bit_gemm_mx_amd import binding as B
from bit_gemm_mx_amd import workloads as W
from oracle import mx_oracle as O

from gpu_util import (assert_bits_equal, assert_matmul_close, dev, fp8_group_truncation_bound,
                      host)

pytestmark = pytest.mark.gpu

PAIRS = [(O.E2M1, O.E2M1), (O.E4M3, O.E2M1), (O.E2M1, O.E4M3), (O.E4M3, O.E4M3)]
EXACT_GROUP_PAIRS = PAIRS[:3]

ONE = {O.E2M1: 0x2, O.E4M3: 0x38}   # the code of 1.0


def identity_bt(K, elem):
    """B^T = I [K, K] as block-scaled codes (scale byte 127)."""
    el = np.zeros((K, K), np.uint8)
    el[np.arange(K), np.arange(K)] = ONE[elem]
    codes = O.pack_nibbles(el) if elem == O.E2M1 else el
    return codes, np.full((K, K // 32), 127, np.uint8)


def fused(a, ae, bc, bsc, be, N, c_in=None, accumulate=False):
    M, K = a.shape
    bt = B.MXTensor(dev(bc), dev(bsc), N, K, be)
    out = dev(c_in.astype(np.float32)) if c_in is not None else None
    return host(B.block_matmul_quantize_a(dev(a), ae, bt, out=out, accumulate=accumulate))


def spread_rows(rng, M, K, outliers=0.01):
    x = W.normal_with_outliers(rng, (M, K), 1.0, outliers, 30.0)
    return x * np.exp2(rng.integers(-20, 20, (M, 1))).astype(np.float32)


def special_rows(rng, M, K):
    """Seeded data with the codec's special cases placed in blocks of A."""
    x = spread_rows(rng, M, K)
    x[0, :11] = [6.0, 0.75, -0.75, 1.75, 3.5, 5.0, 7.0, -0.1, -0.0, 0.25, 0.2]  # E2M1 ties
    x[1, :8] = [448.0, 464.0, -480.0, 0.0048828125, 1.0, 2.0, 3.0, 0.5]          # E4M3 top
    x[2, 32:64] = 0.0                                        # an all-zero block
    x[3, 64:96] = -0.0
    x[4, :32] = 2.0 ** -140                                  # f32 subnormal block maximum
    x[4, 32:64] = rng.standard_normal(32).astype(np.float32) * 2.0 ** -127
    x[5, :32] = np.float32(7.9999995)                        # amax 0x40FFFFFF
    x[6, 5] = np.nan
    x[7, 40] = np.inf
    x[8, 100 % K] = -np.inf
    x[9, :32] = np.finfo(np.float32).max
    # values 1..8 ulp off the E2M1 / E4M3 midpoints, never on one (fast path)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5625, 0.6875, 3.25], np.float32)
    offs = (rng.integers(1, 9, mids.size) * rng.choice([-1, 1], mids.size)).astype(np.int32)
    x[10, :10] = (mids.view(np.int32) + offs).view(np.float32)
    x[10, 10:32] = 1.0
    return x


@pytest.mark.parametrize("ae,be", PAIRS)
@pytest.mark.parametrize("M,K", [(256, 512), (200, 480), (19, 96)])
def test_quantization_is_mx_quantize(ae, be, M, K):
    rng = np.random.default_rng(M + K + 7 * ae + be)
    a = special_rows(rng, M, K)
    bc, bsc = identity_bt(K, be)
    got = fused(a, ae, bc, bsc, be, K)
    qc, qs = O.quantize(a, ae)
    want, _ = O.block_matmul(qc, qs, ae, bc, bsc, be, M, K, K)   # NaN rows where A has NaN/Inf
    assert np.array_equal(np.isnan(got), np.isnan(want)), "NaN positions differ"
    ok = ~np.isnan(want).any(axis=1)
    assert ok.sum() >= M - 3
    deq = O.dequantize(qc, qs, ae, K)
    np.testing.assert_array_equal(got[ok], deq[ok])      # values: -0.0 sums to +0.0


SHAPES = [(1, 1, 32), (3, 5, 64), (17, 33, 160), (128, 128, 128), (130, 260, 1056),
          (300, 520, 2048), (257, 129, 8192), (64, 1000, 384), (1000, 64, 640)]


@pytest.mark.parametrize("ae,be", EXACT_GROUP_PAIRS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_product_within_t1(ae, be, M, N, K):
    rng = np.random.default_rng(3 * M + 5 * N + K + 11 * ae + be)
    a = spread_rows(rng, M, K)
    bc, bsc = O.quantize(spread_rows(rng, N, K), be)
    got = fused(a, ae, bc, bsc, be, N)
    qc, qs = O.quantize(a, ae)
    want, mag = O.block_matmul(qc, qs, ae, bc, bsc, be, M, N, K)
    assert_matmul_close(got, want, mag)


@pytest.mark.parametrize("M,N,K", [(130, 260, 1056), (300, 520, 2048)])
def test_fp8_pair_nan_positions_and_truncation_bound(M, N, K):
    rng = np.random.default_rng(M + N + K)
    a = spread_rows(rng, M, K)
    a[7, 3] = np.nan
    bc, bsc = O.quantize(spread_rows(rng, N, K), O.E4M3)
    got = fused(a, O.E4M3, bc, bsc, O.E4M3, N).astype(np.float64)
    qc, qs = O.quantize(a, O.E4M3)
    want, mag = O.block_matmul(qc, qs, O.E4M3, bc, bsc, O.E4M3, M, N, K)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    rows, cols = np.nonzero(~np.isnan(want))
    bound = 1e-5 * mag[rows, cols] + fp8_group_truncation_bound(qc, qs, bc, bsc, K, rows, cols)
    assert np.all(np.abs(got[rows, cols] - want[rows, cols]) <= bound)


@pytest.mark.parametrize("ae,be", EXACT_GROUP_PAIRS)
def test_accumulate_and_nan_rows(ae, be):
    rng = np.random.default_rng(41 + ae + be)
    M, N, K = 150, 140, 1024
    a = spread_rows(rng, M, K)
    a[11, 500] = np.nan
    a[12, 0] = -np.inf
    bc, bsc = O.quantize(spread_rows(rng, N, K), be)
    cin = rng.standard_normal((M, N)).astype(np.float32)
    got = fused(a, ae, bc, bsc, be, N, c_in=cin, accumulate=True)
    qc, qs = O.quantize(a, ae)
    want, mag = O.block_matmul(qc, qs, ae, bc, bsc, be, M, N, K, c_in=cin, accumulate=True)
    assert np.isnan(want[11]).all() and np.isnan(want[12]).all()
    assert_matmul_close(got, want, mag)


def test_accumulate_zero_does_not_read_c():
    rng = np.random.default_rng(5)
    M, N, K = 40, 36, 256
    a = spread_rows(rng, M, K)
    bc, bsc = O.quantize(spread_rows(rng, N, K), O.E2M1)
    got = fused(a, O.E4M3, bc, bsc, O.E2M1, N, c_in=np.full((M, N), np.nan, np.float32))
    qc, qs = O.quantize(a, O.E4M3)
    want, mag = O.block_matmul(qc, qs, O.E4M3, bc, bsc, O.E2M1, M, N, K)
    assert_matmul_close(got, want, mag)


def test_b_blocked_along_axis0():
    # B given as [K, N] blocked along axis 0 (the B^T storage)
    rng = np.random.default_rng(8)
    M, N, K = 96, 200, 512
    a = spread_rows(rng, M, K)
    b = spread_rows(rng, K, N)
    bt0 = B.quantize(dev(b), O.E2M1, axis=0)
    got = host(B.block_matmul_quantize_a(dev(a), O.E4M3, bt0))
    bc, bsc = O.quantize(np.ascontiguousarray(b.T), O.E2M1)
    qc, qs = O.quantize(a, O.E4M3)
    want, mag = O.block_matmul(qc, qs, O.E4M3, bc, bsc, O.E2M1, M, N, K)
    assert_matmul_close(got, want, mag)


def test_prefill_workload_equals_quantize_then_matmul():
    """The 2048x8192 activations (E4M3) times the 28672x8192 MXFP4 weight:
    every output equal, bit for bit, to mx_quantize followed by
    mx_block_matmul (whose every output the prefill parity test checks
    against the oracle within T1)."""
    a, bt = W.prefill_linear_case()
    ad = dev(a)
    btt = B.quantize(dev(bt), O.E2M1)
    two = B.block_matmul(B.quantize(ad, O.E4M3), btt)
    one = B.block_matmul_quantize_a(ad, O.E4M3, btt)
    assert_bits_equal(host(one), host(two), "fused against two calls")
