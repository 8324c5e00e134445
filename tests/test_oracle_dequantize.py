"""Pins of the oracle's dequantize step: exhaustive decode against closed forms.

E2M1 expectations come from the value formula of "Bit Layout", "The E2M1
element"; E4M3 expectations from PyTorch's float8_e4m3fn decoder; the scale
from "The E8M0 shared scale" (2^(byte-127), 0xFF is NaN for the whole block),
evaluated with Python's ``math.ldexp`` and rounded to float32 by ``struct``.
"""
import math
import struct

import numpy as np
import torch

from oracle import mx_oracle as O
from bit_gemm_mx_amd import workloads as W

NAN = 0x7FC00000


def f32_bits(v: float) -> int:
    try:
        return struct.unpack("<I", struct.pack("<f", v))[0]
    except OverflowError:
        return 0x7F800000 if v > 0 else 0xFF800000


def e2m1_value(code: int) -> float:
    s, e, m = code >> 3, (code >> 1) & 3, code & 1
    mag = 2.0 ** (e - 1) * (1 + m / 2) if e else m / 2
    return -mag if s else mag


def test_exhaustive_e2m1_decode_bits():
    codes = np.arange(16, dtype=np.uint8)
    # rows = scale bytes, each row one block of 32 elements: codes 0..15 twice
    rows = 256
    elems = np.tile(np.concatenate([codes, codes]), (rows, 1))
    packed = O.pack_nibbles(elems)
    scales = np.arange(256, dtype=np.uint8).reshape(rows, 1)
    y = O.dequantize(packed, scales, O.E2M1, 32).view(np.uint32)
    for b in range(256):
        for i in range(32):
            c = int(elems[b, i])
            if b == 255:
                exp = NAN
            else:
                exp = f32_bits(math.ldexp(e2m1_value(c), b - 127))
            assert int(y[b, i]) == exp, (b, c, hex(int(y[b, i])), hex(exp))


def test_exhaustive_e4m3_decode_bits():
    dec = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    codes = np.arange(256, dtype=np.uint8).reshape(8, 32)
    for b in range(256):
        scales = np.full((8, 1), b, dtype=np.uint8)
        y = O.dequantize(codes, scales, O.E4M3, 32).view(np.uint32).reshape(-1)
        for c in range(256):
            v = dec[c]
            if b == 255 or math.isnan(v):
                exp = NAN
            else:
                exp = f32_bits(math.ldexp(float(v), b - 127))
            assert int(y[c]) == exp, (b, c)


def test_nan_scale_poisons_exactly_its_block():
    case = W.roundtrip_case()
    codes, scales = O.quantize(case.x, O.E2M1)
    sc = scales.copy().reshape(-1)
    sc[case.ff_blocks] = 0xFF
    y = O.dequantize(codes, sc.reshape(scales.shape), O.E2M1, case.x.shape[1])
    isnan = np.isnan(y)
    assert isnan.sum() == 64
    blocks_nan = isnan.reshape(-1, 32).all(axis=1)
    assert np.array_equal(np.flatnonzero(blocks_nan), case.ff_blocks)
    assert np.all(y.view(np.uint32)[isnan] == NAN)


def test_roundtrip_case_properties():
    case = W.roundtrip_case()
    codes, scales = O.quantize(case.x, O.E2M1)
    assert codes.shape == (256, 512) and scales.shape == (256, 32)
    # the four zero rows: 128 blocks of byte 127 and zero codes
    assert np.all(scales[case.zero_rows] == 127)
    assert not codes[case.zero_rows].any()
    y = O.dequantize(codes, scales, O.E2M1, 1024)
    assert np.all(y[case.zero_rows] == 0)


def test_dequantize_is_exact_power_of_two_scaling():
    # Dequantized values are grid value x 2^(byte-127) with no rounding: the
    # float32 result divided by the scale is exactly on the grid.
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((16, 128)) * 1e-3).astype(np.float32)
    for elem, grid in ((O.E2M1, O.e2m1_magnitudes()), (O.E4M3, O.e4m3_magnitudes())):
        c, s = O.quantize(x, elem)
        y = O.dequantize(c, s, elem, 128).astype(np.float64)
        t = np.abs(y) / np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=1)
        assert np.all(np.isin(t, grid))
