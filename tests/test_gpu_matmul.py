"""GPU parity of mx_block_matmul against the oracle.

Two bounds, per output element (both also require identical NaN positions):

* T1, the stated tolerance: |gpu - oracle| <= 1e-5 * sum_k |a_k b_k|
  (+ |C_in| when accumulating).  Held by every E2M1 x E2M1 test and by the
  three matmul workloads in full: the decode-shaped 16x4096x4096 product, the
  8192^3 MXFP8 product and the 2048x28672x8192 prefill product, every output
  element, in the launch configuration the benchmark times.
* T2, the bound implied by the arithmetic of CDNA4's scaled MFMA, for every
  other input with E4M3 operands: T1 + sum over aligned groups g of 8
  consecutive K of 2^(E_g - 10), E_g = floor(log2 max_{k in g} |a_k b_k|).
  One-hot probes on gfx950 show that the instruction sums each such group in
  fixed point aligned to its largest product and truncates below about
  2^(E_g - 14); products themselves are exact and the groups are added in fp32.
  Data whose groups span more than ~2^13 (random E4M3 codes, heavy outliers at
  small K) can exceed T1 but never T2.
"""
import numpy as np
import pytest
import torch

from bit_gemm_mx_amd import binding as B
from bit_gemm_mx_amd import workloads as W
from oracle import mx_oracle as O

from gpu_util import (assert_bits_equal, assert_matmul_close, dev, gpu_matmul, host,
                      mfma_group_bound)

pytestmark = pytest.mark.gpu

PAIRS = [(O.E2M1, O.E2M1), (O.E4M3, O.E4M3), (O.E4M3, O.E2M1), (O.E2M1, O.E4M3)]


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
# and N.
SHAPES = [(1, 1, 32), (3, 4, 96), (16, 16, 128), (17, 33, 160), (64, 48, 1024),
          (33, 100, 4128), (5, 70, 8192), (2, 17, 65536), (200, 70, 1056),
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


def assert_t2(got, want, mag, ac, asc, ae, bc, bsc, be, K):
    """T1 everywhere except where the MFMA's group truncation may add error;
    there, T1 + sum_g 2^(E_g - 10)."""
    assert np.array_equal(np.isnan(got), np.isnan(want)), "NaN positions differ"
    err = np.abs(got.astype(np.float64) - want)
    over = np.argwhere(~np.isnan(want) & (err > 1e-5 * mag))
    if len(over) == 0:
        return
    rows, cols = over[:, 0], over[:, 1]
    extra = mfma_group_bound(O.dequantize_f64(ac, asc, ae, K), O.dequantize_f64(bc, bsc, be, K),
                             rows, cols)
    bound = 1e-5 * mag[rows, cols] + extra
    e = err[rows, cols]
    assert np.all(e <= bound), f"T2 exceeded: worst {np.max(e / bound):.3g}"


@pytest.mark.parametrize("ae,be", PAIRS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_quantized_normal_inputs(ae, be, M, N, K):
    rng = np.random.default_rng(M * 1000 + N * 10 + K + ae * 3 + be)
    ac, asc = quantized_normal(rng, M, K, ae)
    bc, bsc = quantized_normal(rng, N, K, be)
    got = gpu_matmul(ac, asc, ae, bc, bsc, be, M, N, K)
    want, mag = O.block_matmul(ac, asc, ae, bc, bsc, be, M, N, K)
    if ae == be == O.E2M1:
        assert_matmul_close(got, want, mag)
    else:
        assert_t2(got, want, mag, ac, asc, ae, bc, bsc, be, K)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_random_codes_e2m1(M, N, K):
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    ac, asc = rand_operand(rng, M, K, O.E2M1)
    bc, bsc = rand_operand(rng, N, K, O.E2M1)
    got = gpu_matmul(ac, asc, O.E2M1, bc, bsc, O.E2M1, M, N, K)
    want, mag = O.block_matmul(ac, asc, O.E2M1, bc, bsc, O.E2M1, M, N, K)
    assert_matmul_close(got, want, mag)


@pytest.mark.parametrize("ae,be", PAIRS[1:])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_random_codes_mfma_bound(ae, be, M, N, K):
    rng = np.random.default_rng(M * 1000 + N * 10 + K + ae * 3 + be)
    ac, asc = rand_operand(rng, M, K, ae)
    bc, bsc = rand_operand(rng, N, K, be)
    got = gpu_matmul(ac, asc, ae, bc, bsc, be, M, N, K)
    want, mag = O.block_matmul(ac, asc, ae, bc, bsc, be, M, N, K)
    assert_t2(got, want, mag, ac, asc, ae, bc, bsc, be, K)


@pytest.mark.parametrize("ae,be", PAIRS)
def test_accumulate(ae, be):
    rng = np.random.default_rng(77)
    M, N, K = 140, 72, 384
    ac, asc = quantized_normal(rng, M, K, ae)
    bc, bsc = quantized_normal(rng, N, K, be)
    cin = (rng.standard_normal((M, N)) * 1e7).astype(np.float32)
    got = gpu_matmul(ac, asc, ae, bc, bsc, be, M, N, K, c_in=cin, accumulate=True)
    want, mag = O.block_matmul(ac, asc, ae, bc, bsc, be, M, N, K, c_in=cin, accumulate=True)
    if ae == be == O.E2M1:
        assert_matmul_close(got, want, mag)
    else:
        assert_t2(got, want, mag, ac, asc, ae, bc, bsc, be, K)


def test_accumulate_zero_overwrites_without_reading():
    rng = np.random.default_rng(78)
    M, N, K = 20, 20, 64
    ac, asc = rand_operand(rng, M, K, O.E2M1)
    bc, bsc = rand_operand(rng, N, K, O.E2M1)
    cin = np.full((M, N), np.nan, np.float32)          # must not leak into C
    got = gpu_matmul(ac, asc, O.E2M1, bc, bsc, O.E2M1, M, N, K, c_in=cin, accumulate=False)
    want, mag = O.block_matmul(ac, asc, O.E2M1, bc, bsc, O.E2M1, M, N, K)
    assert_matmul_close(got, want, mag)


@pytest.mark.parametrize("ae,be", PAIRS)
def test_nan_scales_and_codes(ae, be):
    rng = np.random.default_rng(79)
    M, N, K = 33, 35, 256
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
    assert_t2(got, want, mag, ac, asc, ae, bc, bsc, be, K)


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
                                                (512, O.E4M3, O.E4M3, True),
                                                (1024, O.E2M1, O.E4M3, False)])
def test_tail_round_split(K, ae, be, accumulate):
    """M = 300, N = 33230: 2 x 130 = 260 tiles of 256 x 256 on 256 CUs leave
    a last round of 4 tiles, so the last 2 tile columns (N from 32768 on,
    ragged at 462) are computed by a second launch of 128 x 256 tiles (M
    ragged at 44 in the third).  Every format pair, both scale-staging modes,
    with and without accumulation, every output."""
    rng = np.random.default_rng(95 + K + ae + 3 * be)
    M, N = 300, 33230
    ac, asc = quantized_normal(rng, M, K, ae)
    bc, bsc = quantized_normal(rng, N, K, be, sigma=0.02)
    cin = (rng.standard_normal((M, N)) * 10).astype(np.float32) if accumulate else None
    got = gpu_matmul(ac, asc, ae, bc, bsc, be, M, N, K, c_in=cin, accumulate=accumulate)
    want, mag = O.block_matmul(ac, asc, ae, bc, bsc, be, M, N, K, c_in=cin,
                               accumulate=accumulate)
    if ae == be == O.E2M1:
        assert_matmul_close(got, want, mag)
    else:
        assert_t2(got, want, mag, ac, asc, ae, bc, bsc, be, K)


def test_mlp_down_projection_k11008():
    """K = 11008 (a multiple of 128, not of 512: per-stage scales in the tiled
    kernel), E4M3 activations x E2M1 weights, every output."""
    rng = np.random.default_rng(82)
    M, N, K = 512, 1024, 11008
    ac, asc = quantized_normal(rng, M, K, O.E4M3)
    bc, bsc = quantized_normal(rng, N, K, O.E2M1, sigma=0.02)
    got = gpu_matmul(ac, asc, O.E4M3, bc, bsc, O.E2M1, M, N, K)
    want, mag = O.block_matmul(ac, asc, O.E4M3, bc, bsc, O.E2M1, M, N, K)
    assert_t2(got, want, mag, ac, asc, O.E4M3, bc, bsc, O.E2M1, K)


def test_decode_shaped_full():
    """16x4096 . 4096x4096 MXFP4 x MXFP4, every output element."""
    a, bt = W.decode_matmul_case()
    ac, asc = O.quantize(a, O.E2M1)
    bc, bsc = O.quantize(bt, O.E2M1)
    got = gpu_matmul(ac, asc, O.E2M1, bc, bsc, O.E2M1, 16, 4096, 4096)
    want, mag = O.block_matmul(ac, asc, O.E2M1, bc, bsc, O.E2M1, 16, 4096, 4096)
    assert_matmul_close(got, want, mag)


def _full_large(a, bt, ae, be, t1: bool):
    """Quantize both operands with mx_quantize, multiply with mx_block_matmul
    and check every output element against the oracle (float64 BLAS)."""
    M, K = a.shape
    N = bt.shape[0]
    at = B.quantize(dev(a), ae)
    btt = B.quantize(dev(bt), be)
    c = host(B.block_matmul(at, btt))
    ac, asc = host(at.codes), host(at.scales)
    bc, bsc = host(btt.codes), host(btt.scales)
    del at, btt
    torch.cuda.empty_cache()
    # codes of sampled rows are bit-exact with the oracle's quantize
    r = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(0).integers(0, M, 6)]))
    oac, oas = O.quantize(a[r], ae)
    assert_bits_equal(ac[r], oac, "A codes")
    assert_bits_equal(asc[r], oas, "A scales")
    want, mag = O.block_matmul(ac, asc, ae, bc, bsc, be, M, N, K)
    ratio = np.abs(c.astype(np.float64) - want) / (1e-5 * mag)
    print(f"T1 err/bound over {M * N} outputs: worst {ratio.max():.3g}, "
          f"{int((ratio > 1).sum())} above 1, 99.99th pct {np.percentile(ratio, 99.99):.3g}")
    if t1:
        assert_matmul_close(c, want, mag)
    else:
        assert_t2(c, want, mag, ac, asc, ae, bc, bsc, be, K)


def test_square_fp8_full():
    a, bt = W.square_fp8_case()
    _full_large(a, bt, O.E4M3, O.E4M3, t1=True)


def test_prefill_linear_full():
    # Outlier-holding K-groups of the E4M3 activations exceed the MFMA's
    # alignment window: T2 holds for every element, T1 for all but a few.
    a, bt = W.prefill_linear_case()
    _full_large(a, bt, O.E4M3, O.E2M1, t1=False)
