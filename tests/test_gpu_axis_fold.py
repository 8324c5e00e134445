"""GPU parity of mx_quantize_axis / mx_dequantize_axis (blocks along axis 0)
and mx_fold_scale against the oracle: bit-exact.

Inputs: seeded normal data with outliers and spread block scales, the
hand-worked blocks placed as columns, every (code, scale byte) pair through
the axis-0 decode, ragged column counts and partial runs of block-rows, an
unaligned scale array (byte path), guard bytes around the outputs, and the
full 8192x8192 weight workload blocked along axis 0.  fold_scale: every byte
value with shifts across and beyond the E8M0 range, unaligned starts and
ragged lengths, guard bytes around the range.
"""
import ctypes

import numpy as np
import pytest
import torch

from bit_gemm_mx_amd import binding as B
from bit_gemm_mx_amd import workloads as W
from oracle import mx_oracle as O

from gpu_util import assert_bits_equal, dev, host

pytestmark = pytest.mark.gpu

ELEMS = [O.E2M1, O.E4M3]


def spread_normal(rng, rows, cols):
    x = W.normal_with_outliers(rng, (rows, cols), 1.0, 0.01, 50.0)
    x *= np.exp2(rng.integers(-30, 30, (1, cols))).astype(np.float32)
    return x


def gpu_quantize_axis0(x, elem):
    t = B.quantize(dev(x), elem, axis=0)
    return host(t.codes), host(t.scales)


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("rows,cols", [(32, 1), (32, 64), (64, 100), (96, 130), (256, 64),
                                        (288, 200), (512, 96), (1024, 33), (2048, 130)])
def test_quantize_axis0_bit_exact(elem, rows, cols):
    rng = np.random.default_rng(rows * 7 + cols + elem)
    x = spread_normal(rng, rows, cols)
    x[:32, 0] = 0.0                                    # an all-zero block
    gc, gs = gpu_quantize_axis0(x, elem)
    oc, os_ = O.quantize_axis0(x, elem)
    assert_bits_equal(gs, os_, "scales")
    assert_bits_equal(gc, oc, "codes")


@pytest.mark.parametrize("elem", ELEMS)
def test_quantize_axis0_special_values(elem):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((128, 70)).astype(np.float32)
    # ties of both grids, saturation, signed zeros, subnormal amax, NaN/Inf blocks
    x[:11, 3] = [6.0, 0.75, -0.75, 1.75, 3.5, 5.0, 7.0, -0.1, -0.0, 0.25, 0.2]
    x[32:36, 3] = [1.0, 0.001, 0.296875 / 256, 0.265625 / 256]
    x[64:96, 5] = -0.0
    x[96:128, 6] = 2.0 ** -140
    x[70, 9] = np.nan
    x[100, 10] = -np.inf
    x[7, 11] = np.finfo(np.float32).max
    gc, gs = gpu_quantize_axis0(x, elem)
    oc, os_ = O.quantize_axis0(x, elem)
    assert_bits_equal(gs, os_, "scales")
    assert_bits_equal(gc, oc, "codes")


@pytest.mark.parametrize("elem", ELEMS)
def test_quantize_axis0_matches_last_axis_of_transpose(elem):
    # same storage as mx_quantize of the transposed matrix (the B^T layout)
    rng = np.random.default_rng(6)
    x = spread_normal(rng, 256, 192)
    a = B.quantize(dev(x), elem, axis=0)
    b = B.quantize(dev(np.ascontiguousarray(x.T)), elem)
    assert_bits_equal(host(a.codes), host(b.codes), "codes")
    assert_bits_equal(host(a.scales), host(b.scales), "scales")


@pytest.mark.parametrize("elem", ELEMS)
def test_dequantize_axis0_every_code_and_byte(elem):
    n_codes = 16 if elem == O.E2M1 else 256
    bytes_ = np.array([0, 1, 2, 100, 126, 127, 128, 200, 253, 254, 255], np.uint8)
    rows = 32 * len(bytes_)
    cols = n_codes
    # column c holds code c in every element; block-row i uses scale byte bytes_[i]
    el = np.repeat(np.arange(n_codes, dtype=np.uint8)[:, None], rows, axis=1)   # [cols, rows]
    codes = O.pack_nibbles(el) if elem == O.E2M1 else el
    scales = np.repeat(bytes_[None, :], cols, axis=0)
    t = B.MXTensor(dev(codes), dev(scales), rows, cols, elem, axis=0)
    got = host(B.dequantize(t))
    want = O.dequantize_axis0(codes, scales, elem, rows)
    assert_bits_equal(got, want, "dequantize axis 0")


@pytest.mark.parametrize("elem", ELEMS)
def test_dequantize_axis0_tile_path(elem):
    """Shapes the workgroup-tiled decode takes (columns a multiple of 256,
    rows of 128): every code in every column and block-row position, scale
    bytes across the E8M0 range (0, subnormal results, 254, the 0xFF NaN
    byte), a scale array 4 bytes off a 16-byte boundary, and guard floats
    around the output."""
    n_codes = 16 if elem == O.E2M1 else 256
    bytes_ = np.array([0, 1, 2, 100, 126, 127, 128, 200, 252, 253, 254, 255], np.uint8)
    rows, cols = 32 * len(bytes_), 512
    c_idx = np.arange(cols)[:, None]
    r_idx = np.arange(rows)[None, :]
    el = ((c_idx + 7 * r_idx) % n_codes).astype(np.uint8)                      # [cols, rows]
    codes = O.pack_nibbles(el) if elem == O.E2M1 else el
    scales = bytes_[(np.arange(len(bytes_))[None, :] + np.arange(cols)[:, None]) % len(bytes_)]
    want = O.dequantize_axis0(codes, scales, elem, rows)
    cd = dev(np.ascontiguousarray(codes))
    sbuf = torch.full((scales.size + 8,), 0x33, dtype=torch.uint8, device="cuda")
    sbuf[4:4 + scales.size] = dev(scales.reshape(-1))
    ybuf = torch.full((rows * cols + 32,), -7.0, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    B.mx_dequantize_axis(cd.data_ptr(), sbuf.data_ptr() + 4, ybuf.data_ptr() + 64, rows, cols, 0,
                         elem, 32, stream)
    yb = host(ybuf)
    assert (yb[:16] == -7.0).all() and (yb[16 + rows * cols:] == -7.0).all()
    assert_bits_equal(yb[16:16 + rows * cols].reshape(rows, cols), want, "dequantize axis 0 tile")


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("rows,cols", [(32, 3), (96, 65), (256, 128), (800, 40)])
def test_dequantize_axis0_random(elem, rows, cols):
    rng = np.random.default_rng(rows + cols * 3 + elem)
    x = spread_normal(rng, rows, cols)
    oc, os_ = O.quantize_axis0(x, elem)
    os_ = os_.copy()
    os_[0, 0] = 0xFF
    t = B.MXTensor(dev(oc), dev(os_), rows, cols, elem, axis=0)
    got = host(B.dequantize(t))
    assert_bits_equal(got, O.dequantize_axis0(oc, os_, elem, rows), "dequantize axis 0")


@pytest.mark.parametrize("elem", ELEMS)
def test_axis0_unaligned_scales_and_guards(elem):
    # scale array starting one byte past an 8-byte boundary takes the byte path;
    # guard bytes around codes and scales must stay untouched
    rng = np.random.default_rng(9)
    rows, cols = 512, 70
    x = spread_normal(rng, rows, cols)
    oc, os_ = O.quantize_axis0(x, elem)
    cbuf = torch.full((oc.size + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((os_.size + 33,), 0x5A, dtype=torch.uint8, device="cuda")
    xd = dev(x)
    cptr = cbuf.data_ptr() + 16
    sptr = sbuf.data_ptr() + 1
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    B.mx_quantize_axis(xd.data_ptr(), cptr, sptr, rows, cols, 0, elem, 32, stream)
    cb, sb = host(cbuf), host(sbuf)
    assert_bits_equal(cb[16:16 + oc.size].reshape(oc.shape), oc, "codes")
    assert_bits_equal(sb[1:1 + os_.size].reshape(os_.shape), os_, "scales")
    assert (cb[:16] == 0xA5).all() and (cb[16 + oc.size:] == 0xA5).all()
    assert sb[0] == 0x5A and (sb[1 + os_.size:] == 0x5A).all()
    ybuf = torch.full((rows * cols + 8,), -7.0, dtype=torch.float32, device="cuda")
    B.mx_dequantize_axis(cptr, sptr, ybuf.data_ptr() + 16, rows, cols, 0, elem, 32, stream)
    yb = host(ybuf)
    assert_bits_equal(yb[4:4 + rows * cols].reshape(rows, cols),
                      O.dequantize_axis0(oc, os_, elem, rows), "dequantize")
    assert (yb[:4] == -7.0).all() and (yb[4 + rows * cols:] == -7.0).all()


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("rows,cols", [(1024, 70), (3072, 129)])
def test_axis0_staged_stores_and_guards(elem, rows, cols):
    # rows a multiple of 1024 with 16-byte aligned scales: the workgroup-staged
    # store path, ragged last strip; guard bytes around codes and scales
    rng = np.random.default_rng(rows + cols + elem)
    x = spread_normal(rng, rows, cols)
    oc, os_ = O.quantize_axis0(x, elem)
    cbuf = torch.full((oc.size + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((os_.size + 64,), 0x5A, dtype=torch.uint8, device="cuda")
    xd = dev(x)
    cptr, sptr = cbuf.data_ptr() + 16, sbuf.data_ptr() + 16
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    B.mx_quantize_axis(xd.data_ptr(), cptr, sptr, rows, cols, 0, elem, 32, stream)
    cb, sb = host(cbuf), host(sbuf)
    assert_bits_equal(cb[16:16 + oc.size].reshape(oc.shape), oc, "codes")
    assert_bits_equal(sb[16:16 + os_.size].reshape(os_.shape), os_, "scales")
    assert (cb[:16] == 0xA5).all() and (cb[16 + oc.size:] == 0xA5).all()
    assert (sb[:16] == 0x5A).all() and (sb[16 + os_.size:] == 0x5A).all()


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("rows,cols", [(1024, 68), (2048, 260), (1024, 512), (3072, 1028)])
def test_axis0_staged_column_counts_and_special_values(elem, rows, cols):
    # the workgroup-staged store path at column counts that end inside a
    # 64-column strip (68, 260, 1028) or on one (512), with special values in
    # the first and the last block-rows, and guard bytes around the outputs
    rng = np.random.default_rng(rows + 3 * cols + elem)
    x = spread_normal(rng, rows, cols)
    x[:6, 1] = [6.0, 0.75, -0.75, 1.75, 3.5, -0.0]     # grid ties of E2M1
    x[32:64, 2] = -0.0
    x[64, 3] = np.nan
    x[rows - 32, cols - 1] = np.inf
    x[rows - 31:, cols - 2] = 2.0 ** -140              # f32 subnormal block maximum
    oc, os_ = O.quantize_axis0(x, elem)
    cbuf = torch.full((oc.size + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((os_.size + 64,), 0x5A, dtype=torch.uint8, device="cuda")
    xd = dev(x)
    cptr, sptr = cbuf.data_ptr() + 16, sbuf.data_ptr() + 16
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    B.mx_quantize_axis(xd.data_ptr(), cptr, sptr, rows, cols, 0, elem, 32, stream)
    cb, sb = host(cbuf), host(sbuf)
    assert_bits_equal(cb[16:16 + oc.size].reshape(oc.shape), oc, "codes")
    assert_bits_equal(sb[16:16 + os_.size].reshape(os_.shape), os_, "scales")
    assert (cb[:16] == 0xA5).all() and (cb[16 + oc.size:] == 0xA5).all()
    assert (sb[:16] == 0x5A).all() and (sb[16 + os_.size:] == 0x5A).all()


def test_axis0_weight_workload_full():
    """The 8192x8192 MXFP4 weight workload blocked along axis 0: every code,
    scale and dequantized element."""
    x = W.weight_codec_case()
    t = B.quantize(dev(x), O.E2M1, axis=0)
    gc, gs = host(t.codes), host(t.scales)
    y = host(B.dequantize(t))
    del t
    torch.cuda.empty_cache()
    oc, os_ = O.quantize_axis0(x, O.E2M1)
    assert_bits_equal(gs, os_, "scales")
    assert_bits_equal(gc, oc, "codes")
    assert_bits_equal(y, O.dequantize_axis0(oc, os_, O.E2M1, 8192), "dequantize")


@pytest.mark.parametrize("ae,be", [(O.E2M1, O.E2M1), (O.E4M3, O.E2M1)])
def test_block_matmul_takes_b_blocked_along_axis0(ae, be):
    rng = np.random.default_rng(10)
    M, N, K = 70, 300, 1024
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)      # B [K, N]
    at = B.quantize(dev(a), ae)
    bq = B.quantize(dev(b), be, axis=0)
    got = host(B.block_matmul(at, bq))
    ac, asc = O.quantize(a, ae)
    bc, bsc = O.quantize_axis0(b, be)
    want, mag = O.block_matmul(ac, asc, ae, bc, bsc, be, M, N, K)
    err = np.abs(got.astype(np.float64) - want)
    assert np.all(err <= 1e-5 * mag)


# ------------------------------------------------------------------ fold_scale
@pytest.mark.parametrize("j", [-300, -255, -128, -5, 0, 1, 7, 127, 254, 300])
def test_fold_scale_every_byte(j):
    s = np.tile(np.arange(256, dtype=np.uint8), 37)               # 9472 bytes
    t = dev(s)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    B.mx_fold_scale(t.data_ptr(), s.size, j, stream)
    assert_bits_equal(host(t), O.fold_scale(s, j), f"fold j={j}")


@pytest.mark.parametrize("offset,n", [(0, 1), (1, 15), (3, 16), (15, 17), (7, 1000003), (0, 4096)])
def test_fold_scale_unaligned_and_ragged(offset, n):
    rng = np.random.default_rng(offset * 31 + n)
    s = rng.integers(0, 256, n, dtype=np.uint8)
    buf = torch.full((n + offset + 32,), 0xC3, dtype=torch.uint8, device="cuda")
    buf[offset:offset + n] = dev(s)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    B.mx_fold_scale(buf.data_ptr() + offset, n, -9, stream)
    h = host(buf)
    assert_bits_equal(h[offset:offset + n], O.fold_scale(s, -9), "fold")
    assert (h[:offset] == 0xC3).all() and (h[offset + n:] == 0xC3).all()


def test_fold_scale_then_matmul():
    # folding 2^j into A's scales scales C by 2^j exactly (dialect page, fold_scale)
    rng = np.random.default_rng(11)
    M, N, K = 64, 96, 512
    at = B.quantize(dev(rng.standard_normal((M, K)).astype(np.float32)), O.E4M3)
    bt = B.quantize(dev(rng.standard_normal((N, K)).astype(np.float32)), O.E2M1)
    c0 = host(B.block_matmul(at, bt))
    B.fold_scale(at, 5)
    c1 = host(B.block_matmul(at, bt))
    assert_bits_equal(c1, (c0.astype(np.float64) * 32.0).astype(np.float32), "C * 2^5")
