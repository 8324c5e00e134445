"""GPU parity of mx_block_matmul against the oracle.

The bound is the stated tolerance T1, per output element: |gpu - oracle| <=
1e-5 * sum_k |a_k b_k| (+ |C_in| when accumulating), with identical NaN
positions and an exact zero where the bound is zero.

* E2M1 x E2M1, and the mixed pairs E4M3 x E2M1 / E2M1 x E4M3: every test,
  random codes included.  The mixed pairs reach the scaled MFMA as two
  operands split on the E4M3 exponent (see the kernel source), so every
  group of 8 products is summed exactly and only the fp32 accumulation
  rounds.
* E4M3 x E4M3: the 8192^3 MXFP8 workload (every output) and quantized
  Gaussian data without outliers at K >= 1024.  This pair runs on one
  scaled FP8 instruction, whose group truncation can exceed T1 on other
  inputs (outliers, small K, random codes); those inputs are measured in
  test_gpu_fp8_characterisation.py and are not parity.
"""
import numpy as np
import pytest
import torch

from bit_gemm_mx_amd import binding as B
from bit_gemm_mx_amd import workloads as W
from oracle import mx_oracle as O

from gpu_util import assert_bits_equal, assert_matmul_close, dev, gpu_matmul, host

pytestmark = pytest.mark.gpu

PAIRS = [(O.E2M1, O.E2M1), (O.E4M3, O.E4M3), (O.E4M3, O.E2M1), (O.E2M1, O.E4M3)]
EXACT_GROUP_PAIRS = [(O.E2M1, O.E2M1), (O.E4M3, O.E2M1), (O.E2M1, O.E4M3)]


def rand_operand(rng, rows, K, elem, lo=112, hi=142, nan_codes=False):
    if elem == O.E2M1:
        el = rng.integers(0, 16, (rows, K), dtype=np.uint8)
        codes = O.pack_nibbles(el)
    else:
        el = rng.integers(0, 256, (rows, K), dtype=np.uint8)
        if not nan_codes:
            el[(el & 0x7F) == 0x7F] = 0x38
        codes = el
    return codes, rng.integers(lo, hi, (rows, K // 32), dtype=np.uint8)


# Small and decode-like shapes (one to four 16-row tiles of A, K split over
# the waves of a workgroup in one or many load batches, K not a multiple of
# 128, several row panels), shapes the 256x256-tile kernel does not take
# (K not a multiple of 128), and shapes it does take with partial tiles in M
# and N.  Up to 32 rows with K a multiple of 128 run the LDS-staged decode
# kernel: one K step in all (a partial batch), ranges of 2 and 1 steps with
# idle waves (K = 1152), two row tiles, ragged N.
SHAPES = [(1, 1, 32), (3, 4, 96), (16, 16, 128), (17, 33, 160), (64, 48, 1024),
          (33, 100, 4128), (5, 70, 8192), (2, 17, 65536), (32, 50, 1152), (24, 16, 384),
          (20, 300, 4224), (12, 1000, 2048), (200, 70, 1056),
          (100, 70, 3968), (256, 256, 512), (300, 257, 2080), (257, 300, 1152),
          (130, 520, 640), (512, 256, 128),
          # the tiled kernel (M > 64, K a multiple of 512) with partial tiles in M and N
          (300, 257, 1024), (257, 520, 2048), (1000, 300, 512), (65, 1000, 1536),
          (777, 1111, 3072),
          # the tiled kernel with per-stage scales (K a multiple of 128 but not of 512)
          (300, 257, 640), (1000, 300, 384), (65, 700, 1408), (513, 257, 2944)]


def quantized_normal(rng, rows, K, elem, sigma=1.0, outliers=0.01, factor=30.0):
    x = W.normal_with_outliers(rng, (rows, K), sigma, outliers, factor)
    x *= np.exp2(rng.integers(-20, 20, (rows, 1))).astype(np.float32)   # spread the scales
    return O.quantize(x, elem)


@pytest.mark.parametrize("ae,be", EXACT_GROUP_PAIRS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_quantized_normal_inputs(ae, be, M, N, K):
    rng = np.random.default_rng(M * 1000 + N * 10 + K + ae * 3 + be)
    ac, asc = quantized_normal(rng, M, K, ae)
    bc, bsc = quantized_normal(rng, N, K, be)
    got = gpu_matmul(ac, asc, ae, bc, bsc, be, M, N, K)
    want, mag = O.block_matmul(ac, asc, ae, bc, bsc, be, M, N, K)
    assert_matmul_close(got, want, mag)


@pytest.mark.parametrize("M,N,K", [s for s in SHAPES if s[2] >= 1024])
def test_quantized_gaussian_fp8(M, N, K):
    """E4M3 x E4M3 on quantized N(0,1) data (no outliers, row scales spread)."""
    rng = np.random.default_rng(M * 1000 + N * 10 + K + 7)
    ac, asc = quantized_normal(rng, M, K, O.E4M3, outliers=0.0)
    bc, bsc = quantized_normal(rng, N, K, O.E4M3, outliers=0.0)
    got = gpu_matmul(ac, asc, O.E4M3, bc, bsc, O.E4M3, M, N, K)
    want, mag = O.block_matmul(ac, asc, O.E4M3, bc, bsc, O.E4M3, M, N, K)
    assert_matmul_close(got, want, mag)


@pytest.mark.parametrize("ae,be", EXACT_GROUP_PAIRS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_random_codes(ae, be, M, N, K):
    """Uniformly random codes (every E4M3 exponent in one group) and scales."""
    rng = np.random.default_rng(M * 1000 + N * 10 + K + ae * 3 + be)
    ac, asc = rand_operand(rng, M, K, ae)
    bc, bsc = rand_operand(rng, N, K, be)
    got = gpu_matmul(ac, asc, ae, bc, bsc, be, M, N, K)
    want, mag = O.block_matmul(ac, asc, ae, bc, bsc, be, M, N, K)
    assert_matmul_close(got, want, mag)


@pytest.mark.parametrize("ae,be", EXACT_GROUP_PAIRS)
@pytest.mark.parametrize("M,N,K", [(512, 512, 8192), (16, 512, 8192), (300, 257, 16384)])
def test_one_signed_operands(ae, be, M, N, K):
    """Positive codes in A and B^T: every product has the same sign, so no
    rounding of the float32 accumulation over K cancels another (K = 8192
    and 16384: 128 and 256 MFMA steps into one accumulator in the tiled
    kernel, 8 K ranges summed in LDS in the decode kernel).  Every output
    within the tolerance; the worst is printed (measured: tiled kernel up to
    0.4 of it at K = 8192 and 0.6 at K = 16384, decode kernel 0.05)."""
    rng = np.random.default_rng(M + N + K + 3 * ae + be)

    def positive(rows, elem):
        if elem == O.E2M1:
            codes = O.pack_nibbles(rng.integers(1, 8, (rows, K), dtype=np.uint8))
        else:
            codes = rng.integers(1, 0x7F, (rows, K), dtype=np.uint8)
        return codes, rng.integers(120, 135, (rows, K // 32), dtype=np.uint8)
    ac, asc = positive(M, ae)
    bc, bsc = positive(N, be)
    got = gpu_matmul(ac, asc, ae, bc, bsc, be, M, N, K)
    want, mag = O.block_matmul(ac, asc, ae, bc, bsc, be, M, N, K)
    worst = assert_matmul_close(got, want, mag)
    print(f"one-signed {ae}x{be} {M}x{N}x{K}: worst error {worst:.3g} of the tolerance")


@pytest.mark.parametrize("M", [140, 24])
@pytest.mark.parametrize("ae,be", PAIRS)
def test_accumulate(ae, be, M):
    rng = np.random.default_rng(77 + M)
    fp8 = ae == be == O.E4M3
    N, K = (72, 2048) if fp8 else (72, 384)
    ac, asc = quantized_normal(rng, M, K, ae, outliers=0.0 if fp8 else 0.01)
    bc, bsc = quantized_normal(rng, N, K, be, outliers=0.0 if fp8 else 0.01)
    cin = (rng.standard_normal((M, N)) * 1e7).astype(np.float32)
    got = gpu_matmul(ac, asc, ae, bc, bsc, be, M, N, K, c_in=cin, accumulate=True)
    want, mag = O.block_matmul(ac, asc, ae, bc, bsc, be, M, N, K, c_in=cin, accumulate=True)
    assert_matmul_close(got, want, mag)


def test_accumulate_zero_overwrites_without_reading():
    rng = np.random.default_rng(78)
    M, N, K = 20, 20, 64
    ac, asc = rand_operand(rng, M, K, O.E2M1)
    bc, bsc = rand_operand(rng, N, K, O.E2M1)
    cin = np.full((M, N), np.nan, np.float32)          # must not leak into C
    got = gpu_matmul(ac, asc, O.E2M1, bc, bsc, O.E2M1, M, N, K, c_in=cin, accumulate=False)
    want, mag = O.block_matmul(ac, asc, O.E2M1, bc, bsc, O.E2M1, M, N, K)
    assert_matmul_close(got, want, mag)


@pytest.mark.parametrize("M", [33, 30])
@pytest.mark.parametrize("ae,be", PAIRS)
def test_nan_scales_and_codes(ae, be, M):
    """0xFF scales and E4M3 NaN codes poison exactly the oracle's outputs.
    M = 30 runs the LDS-staged decode kernel, whose waves here stage a batch
    of K steps and multiply only the first: the unused steps staged for B^T
    row 29 hold row 30's NaN code, which must not reach column 29."""
    rng = np.random.default_rng(79)
    N, K = 35, 256
    fp8 = ae == be == O.E4M3
    if fp8:      # Gaussian data: the single-instruction pair's T1 regime
        ac, asc = quantized_normal(rng, M, K, ae, outliers=0.0)
        bc, bsc = quantized_normal(rng, N, K, be, outliers=0.0)
    else:
        ac, asc = rand_operand(rng, M, K, ae)
        bc, bsc = rand_operand(rng, N, K, be)
    asc[3, 2] = 0xFF
    bsc[17, 7] = 0xFF
    if ae == O.E4M3:
        ac[9, 100] = 0x7F
    if be == O.E4M3:
        bc[30, 5] = 0xFF
    got = gpu_matmul(ac, asc, ae, bc, bsc, be, M, N, K)
    want, mag = O.block_matmul(ac, asc, ae, bc, bsc, be, M, N, K)
    assert np.isnan(want).sum() > 0
    assert np.array_equal(np.isnan(got), np.isnan(want)), "NaN positions differ"
    if not fp8:
        assert_matmul_close(got, want, mag)


def test_zero_rows_give_exact_zero():
    rng = np.random.default_rng(80)
    M, N, K = 8, 16, 128
    ac, asc = rand_operand(rng, M, K, O.E4M3)
    ac[2] = 0
    bc, bsc = rand_operand(rng, N, K, O.E2M1)
    got = gpu_matmul(ac, asc, O.E4M3, bc, bsc, O.E2M1, M, N, K)
    assert np.all(got[2] == 0)


def test_quantized_float_inputs_end_to_end():
    # quantize on the GPU (bit-exact against the oracle), then multiply
    rng = np.random.default_rng(81)
    M, N, K = 96, 80, 1024
    a = rng.standard_normal((M, K)).astype(np.float32)
    bt = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    at = B.quantize(dev(a), O.E4M3)
    btt = B.quantize(dev(bt), O.E2M1)
    oac, oas = O.quantize(a, O.E4M3)
    obc, obs = O.quantize(bt, O.E2M1)
    assert_bits_equal(host(at.codes), oac, "A codes")
    assert_bits_equal(host(btt.codes), obc, "B codes")
    got = host(B.block_matmul(at, btt))
    want, mag = O.block_matmul(oac, oas, O.E4M3, obc, obs, O.E2M1, M, N, K)
    assert_matmul_close(got, want, mag)


@pytest.mark.parametrize("offset", [0, 4, 1])
def test_scale_array_alignment(offset):
    """Scale arrays at a 16-byte boundary (16-byte scale slices), 4 bytes
    past one (dword scales per stage) and 1 byte past one (the skinny
    kernel): all within the tolerance, K a multiple of 512."""
    rng = np.random.default_rng(90 + offset)
    M, N, K = 300, 257, 1024
    ac, asc = quantized_normal(rng, M, K, O.E2M1)
    bc, bsc = quantized_normal(rng, N, K, O.E2M1, sigma=0.02)

    def shifted(arr):
        buf = torch.zeros(arr.size + offset, dtype=torch.uint8, device="cuda")
        view = buf[offset:].view(arr.shape)
        view.copy_(torch.from_numpy(arr))
        assert view.data_ptr() % 16 == offset
        return view

    a = B.MXTensor(dev(ac), shifted(asc), M, K, O.E2M1)
    b = B.MXTensor(dev(bc), shifted(bsc), N, K, O.E2M1)
    got = host(B.block_matmul(a, b))
    want, mag = O.block_matmul(ac, asc, O.E2M1, bc, bsc, O.E2M1, M, N, K)
    assert_matmul_close(got, want, mag)


@pytest.mark.parametrize("K,ae,be,accumulate", [(512, O.E2M1, O.E2M1, False),
                                                (640, O.E4M3, O.E2M1, True),
                                                (2048, O.E4M3, O.E4M3, True),
                                                (1024, O.E2M1, O.E4M3, False)])
def test_tail_round_split(K, ae, be, accumulate):
    """M = 300, N = 33230: 2 x 130 = 260 tiles of 256 x 256 on 256 CUs leave
    a last round of 4 tiles, so the last 2 tile columns (N from 32768 on,
    ragged at 462) are computed by a second launch of 128 x 256 tiles (M
    ragged at 44 in the third).  Every format pair, both scale-staging modes,
    with and without accumulation, every output."""
    rng = np.random.default_rng(95 + K + ae + 3 * be)
    M, N = 300, 33230
    out = 0.0 if ae == be == O.E4M3 else 0.01
    ac, asc = quantized_normal(rng, M, K, ae, outliers=out)
    bc, bsc = quantized_normal(rng, N, K, be, sigma=0.02, outliers=out)
    cin = (rng.standard_normal((M, N)) * 10).astype(np.float32) if accumulate else None
    got = gpu_matmul(ac, asc, ae, bc, bsc, be, M, N, K, c_in=cin, accumulate=accumulate)
    want, mag = O.block_matmul(ac, asc, ae, bc, bsc, be, M, N, K, c_in=cin,
                               accumulate=accumulate)
    assert_matmul_close(got, want, mag)


def test_mlp_down_projection_k11008():
    """K = 11008 (a multiple of 128, not of 512: per-stage scales in the tiled
    kernel), E4M3 activations x E2M1 weights, every output."""
    rng = np.random.default_rng(82)
    M, N, K = 512, 1024, 11008
    ac, asc = quantized_normal(rng, M, K, O.E4M3)
    bc, bsc = quantized_normal(rng, N, K, O.E2M1, sigma=0.02)
    got = gpu_matmul(ac, asc, O.E4M3, bc, bsc, O.E2M1, M, N, K)
    want, mag = O.block_matmul(ac, asc, O.E4M3, bc, bsc, O.E2M1, M, N, K)
    assert_matmul_close(got, want, mag)


def test_decode_shaped_full():
    """16x4096 . 4096x4096 MXFP4 x MXFP4, every output element."""
    a, bt = W.decode_matmul_case()
    ac, asc = O.quantize(a, O.E2M1)
    bc, bsc = O.quantize(bt, O.E2M1)
    got = gpu_matmul(ac, asc, O.E2M1, bc, bsc, O.E2M1, 16, 4096, 4096)
    want, mag = O.block_matmul(ac, asc, O.E2M1, bc, bsc, O.E2M1, 16, 4096, 4096)
    assert_matmul_close(got, want, mag)


def _full_large(a, bt, ae, be, all_a_rows: bool):
    """Quantize both operands with mx_quantize, multiply with mx_block_matmul
    and check A's codes and scales (every row, or sampled rows) and every
    output element against the oracle (float64 BLAS for the product)."""
    M, K = a.shape
    N = bt.shape[0]
    at = B.quantize(dev(a), ae)
    btt = B.quantize(dev(bt), be)
    c = host(B.block_matmul(at, btt))
    ac, asc = host(at.codes), host(at.scales)
    bc, bsc = host(btt.codes), host(btt.scales)
    del at, btt
    torch.cuda.empty_cache()
    # A's codes and scales bit-exact with the oracle's quantize
    r = (np.arange(M) if all_a_rows else
         np.unique(np.concatenate([[0, M - 1], np.random.default_rng(0).integers(0, M, 30)])))
    oac, oas = O.quantize(a[r], ae)
    assert_bits_equal(asc[r], oas, "A scales")
    assert_bits_equal(ac[r], oac, "A codes")
    del oac, oas
    want, mag = O.block_matmul(ac, asc, ae, bc, bsc, be, M, N, K)
    ratio = np.abs(c.astype(np.float64) - want) / (1e-5 * mag)
    print(f"T1 err/bound over {M * N} outputs: worst {ratio.max():.3g}, "
          f"{int((ratio > 1).sum())} above 1, 99.99th pct {np.percentile(ratio, 99.99):.3g}")
    assert_matmul_close(c, want, mag)


def test_square_fp8_full():
    a, bt = W.square_fp8_case()
    _full_large(a, bt, O.E4M3, O.E4M3, all_a_rows=False)   # 67M E4M3 codes: sampled rows


def test_prefill_linear_full():
    a, bt = W.prefill_linear_case()
    _full_large(a, bt, O.E4M3, O.E2M1, all_a_rows=True)
