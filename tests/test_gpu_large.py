"""GPU parity at sizes past 2^31 elements (64-bit indexing in every kernel).

Inputs are generated on the GPU with a seeded torch generator (2^31 floats
would take minutes through NumPy); only sampled rows, columns or outputs are
copied back and checked against the oracle: codes and scales bit-exact, the
matmul within the stated tolerance.
"""
import numpy as np
import pytest
import torch

from bit_gemm_mx_amd import binding as B
from oracle import mx_oracle as O

from gpu_util import assert_bits_equal

pytestmark = pytest.mark.gpu


def sample(n, k, seed):
    idx = np.random.default_rng(seed).choice(n, size=k, replace=False)
    return np.unique(np.concatenate([[0, n - 1], idx]))


def randn(rows, cols, seed, sigma=1.0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    x = torch.randn(rows, cols, device="cuda", generator=g)
    return x.mul_(sigma)


def test_codec_past_2g_elements():
    rows, cols = 65601, 32768                      # 2,149,613,568 elements
    x = randn(rows, cols, 11, 0.02)
    x[::4099, ::7] *= 1e3                          # outliers across the whole tensor
    q = B.quantize(x, B.MX_E2M1)
    y = B.dequantize(q)
    torch.cuda.synchronize()
    r = sample(rows, 8, 1)
    xr = x[torch.from_numpy(r).cuda()].cpu().numpy()
    codes = q.codes[torch.from_numpy(r).cuda()].cpu().numpy()
    scales = q.scales[torch.from_numpy(r).cuda()].cpu().numpy()
    oc, os_ = O.quantize(xr, O.E2M1)
    assert_bits_equal(scales, os_, "scales")
    assert_bits_equal(codes, oc, "codes")
    assert_bits_equal(y[torch.from_numpy(r).cuda()].cpu().numpy(),
                      O.dequantize(codes, scales, O.E2M1, cols), "dequantized")


def test_axis0_codec_past_2g_elements():
    rows, cols = 65536, 32801                      # blocks along axis 0; 2,149,646,336 elements
    x = randn(rows, cols, 12, 0.02)
    q = B.quantize(x, B.MX_E4M3, axis=0)
    y = B.dequantize(q)
    torch.cuda.synchronize()
    c = sample(cols, 8, 2)
    ct = torch.from_numpy(c).cuda()
    xt = x[:, ct].t().contiguous().cpu().numpy()    # the sampled columns as rows
    oc, os_ = O.quantize(xt, O.E4M3)
    codes = q.codes[ct].cpu().numpy()               # block-major: one row per column
    scales = q.scales[ct].cpu().numpy()
    assert_bits_equal(scales, os_, "scales")
    assert_bits_equal(codes, oc, "codes")
    assert_bits_equal(y[:, ct].t().contiguous().cpu().numpy(),
                      O.dequantize(codes, scales, O.E4M3, rows), "dequantized")


def test_matmul_output_past_2g_elements():
    M, N, K = 65836, 32845, 512                    # C: 2,162,383,420 elements (tiled kernel)
    a = B.quantize(randn(M, K, 13), B.MX_E4M3)
    bt = B.quantize(randn(N, K, 14, 0.02), B.MX_E2M1)
    c = B.block_matmul(a, bt)
    torch.cuda.synchronize()
    r, s = sample(M, 6, 3), sample(N, 6, 4)
    rt, st = torch.from_numpy(r).cuda(), torch.from_numpy(s).cuda()
    ac, asc = a.codes[rt].cpu().numpy(), a.scales[rt].cpu().numpy()
    bc, bsc = bt.codes[st].cpu().numpy(), bt.scales[st].cpu().numpy()
    got = c[rt][:, st].cpu().numpy()
    want, mag = O.block_matmul(ac, asc, O.E4M3, bc, bsc, O.E2M1, len(r), len(s), K)
    assert np.all(np.abs(got.astype(np.float64) - want) <= 1e-5 * mag)
    assert not np.isnan(got).any() and not np.isnan(want).any()


def test_skinny_matmul_operand_past_2g_bytes():
    M, N, K = 16, 4194319, 512                     # B^T codes: 2,147,491,328 bytes (E4M3)
    a = B.quantize(randn(M, K, 15), B.MX_E2M1)
    bt = B.quantize(randn(N, K, 16, 0.02), B.MX_E4M3)
    c = B.block_matmul(a, bt)
    torch.cuda.synchronize()
    s = sample(N, 10, 5)
    st = torch.from_numpy(s).cuda()
    ac, asc = a.codes.cpu().numpy(), a.scales.cpu().numpy()
    bc, bsc = bt.codes[st].cpu().numpy(), bt.scales[st].cpu().numpy()
    got = c[:, st].cpu().numpy()
    want, mag = O.block_matmul(ac, asc, O.E2M1, bc, bsc, O.E4M3, M, len(s), K)
    assert np.all(np.abs(got.astype(np.float64) - want) <= 1e-5 * mag)
    assert not np.isnan(got).any()


def test_f32b_matmul_output_past_2g_elements():
    M, N, K = 65552, 32800, 64                     # C: 2,150,105,600 elements (64x64 tiles)
    a = B.quantize(randn(M, K, 17, 0.02), B.MX_E2M1)
    b = randn(K, N, 18)
    c = B.block_matmul_f32b(a, b)
    torch.cuda.synchronize()
    r, s = sample(M, 6, 6), sample(N, 6, 7)
    rt, st = torch.from_numpy(r).cuda(), torch.from_numpy(s).cuda()
    ac, asc = a.codes[rt].cpu().numpy(), a.scales[rt].cpu().numpy()
    bs = b[:, st].cpu().numpy()
    got = c[rt][:, st].cpu().numpy()
    want, mag = O.block_matmul_f32b(ac, asc, O.E2M1, bs, len(r), len(s), K)
    assert np.all(np.abs(got.astype(np.float64) - want) <= 1e-5 * mag)
