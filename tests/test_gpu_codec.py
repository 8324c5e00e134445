"""GPU parity of mx_quantize / mx_dequantize against the oracle: bit-exact.

Inputs are the seeded workloads (round trip 256x1024, weight codec 8192x8192,
prefill activations 2048x8192 to E4M3), special values, exhaustive decode of
every (code, scale byte) pair, sweeps of float32 values around every rounding
midpoint, and ragged tails with guard bytes around the outputs.
"""
import numpy as np
import pytest
import torch

from bit_gemm_mx_amd import binding as B
from bit_gemm_mx_amd import workloads as W
from oracle import mx_oracle as O

from closed_forms import e4m3_codes_at_unit_scale
from gpu_util import assert_bits_equal, dev, gpu_dequantize, gpu_quantize, host

pytestmark = pytest.mark.gpu

ELEMS = [O.E2M1, O.E4M3]


def check_quantize(x, elem, what=""):
    gc, gs = gpu_quantize(x, elem)
    oc, os_ = O.quantize(x, elem)
    assert_bits_equal(gs, os_, f"scales {what}")
    assert_bits_equal(gc, oc, f"codes {what}")
    return gc, gs


def test_roundtrip_workload_bit_exact():
    case = W.roundtrip_case()
    codes, scales = check_quantize(case.x, O.E2M1, "round trip")
    sc = scales.copy().reshape(-1)
    sc[case.ff_blocks] = 0xFF
    sc = sc.reshape(scales.shape)
    y = gpu_dequantize(codes, sc, O.E2M1, 1024)
    want = O.dequantize(codes, sc, O.E2M1, 1024)
    assert_bits_equal(y, want, "dequantize round trip")
    assert np.isnan(y).sum() == 64


@pytest.mark.parametrize("elem", ELEMS)
def test_special_values(elem):
    f = np.float32
    rows = []
    def blk(*vals):
        r = np.zeros(32, np.float32)
        r[:len(vals)] = vals
        rows.append(r)
    blk(6.0, 0.75, -0.75, 1.75, 3.5, 5.0, 7.0, -0.1, -0.0, 0.25, 0.2)
    blk(1.0, 0.001, 0.296875 / 256, 0.265625 / 256)
    blk(1.9375, -1.9375, 1.0)
    blk(np.frombuffer(np.uint32(0x40FFFFFF).tobytes(), np.float32)[0])
    blk(2.0 ** -126)
    blk(-0.0, 0.0, -0.0)
    blk(np.finfo(np.float32).max, -np.finfo(np.float32).max, 1.0)
    blk(np.nan, 1.0)
    blk(np.inf, -1.0)
    blk(-np.inf, 3.0)
    blk(f(1e-45), f(-1e-45), f(3e-45))                         # subnormal amax
    sub = np.frombuffer(np.arange(1, 33, dtype=np.uint32) * np.uint32(0x3FFFF), np.float32)
    rows.append(sub.astype(np.float32).copy())                 # all-subnormal block
    rows.append(-sub.astype(np.float32))
    blk(2.0 ** -125, 2.0 ** -127, -(2.0 ** -130))              # around the lower clip
    blk(*(np.arange(32, dtype=np.float32) - 16) * f(0.37))
    x = np.stack(rows)
    codes, scales = check_quantize(x, elem, "special")
    y = gpu_dequantize(codes, scales, elem, 32)
    assert_bits_equal(y, O.dequantize(codes, scales, elem, 32), "dequantize special")
    # The same blocks inside a tensor of whole wave iterations (2560 blocks,
    # a multiple of 32), where the quantize stages codes and scale bytes
    # through LDS: placed at iteration boundaries among Gaussian blocks.
    rng = np.random.default_rng(elem)
    big = (rng.standard_normal((2560, 32)) * np.exp2(rng.integers(-30, 30, (2560, 1)))).astype(np.float32)
    at = [0, 1, 7, 8, 31, 32, 33, 255, 256, 511, 1000, 1023, 1024, 2000, 2047, 2558, 2559][:len(rows)]
    big[at] = x[:len(at)]
    check_quantize(big.reshape(64, 40 * 32), elem, "special, staged stores")


def _sweep_values(lo_bits, hi_bits, stride, grid):
    v = np.arange(lo_bits, hi_bits, stride, dtype=np.uint32).view(np.float32)
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)
    near = [mids.view(np.uint32).astype(np.int64) + d for d in range(-8, 9)]
    near = np.concatenate(near).astype(np.uint32).view(np.float32)
    vals = np.concatenate([v, near, grid.astype(np.float32)])
    sign = np.where(np.arange(vals.size) % 2 == 1, -1.0, 1.0).astype(np.float32)
    return vals * sign


@pytest.mark.parametrize("elem", ELEMS)
def test_value_sweep_with_anchor(elem):
    # Element 0 of every block is an anchor forcing e = 0 (floor(log2 anchor) = emax),
    # so elements 1..31 run through a sweep of y values directly.
    if elem == O.E2M1:
        vals = _sweep_values(0x3E000000, 0x41000000, 7, O.e2m1_magnitudes())   # [2^-3, 8)
        anchor = 7.0
    else:
        vals = _sweep_values(0x3A800000, 0x44000000, 211, O.e4m3_magnitudes())  # [2^-10, 512)
        anchor = 511.0
    nb = -(-vals.size // 31)
    flat = np.zeros(nb * 31, np.float32)
    flat[:vals.size] = vals
    x = np.empty((nb, 32), np.float32)
    x[:, 0] = anchor
    x[:, 1:] = flat.reshape(nb, 31)
    codes, scales = check_quantize(x, elem, "sweep")
    assert np.all(scales == 127)


def _bits(v):
    return np.asarray(v, np.float32).view(np.uint32).astype(np.int64)


def _f32(bits):
    return np.asarray(bits, np.int64).astype(np.uint32).view(np.float32)


def _blocks_of(anchor_bits, vals, shifts):
    """Blocks [anchor, 31 values] for every power-of-two shift 2^j of the
    whole block, padded (by repeating blocks) to a multiple of 32 blocks:
    the kernel quantizes 32 blocks per wave and zero-fills a partial set,
    and a zero element would send the wave down its exact path."""
    nb = -(-vals.size // 31)
    flat = np.resize(vals, nb * 31).astype(np.float32)
    base = np.empty((nb, 32), np.float32)
    base[:, 0] = _f32(anchor_bits)
    base[:, 1:] = flat.reshape(nb, 31)
    x = np.concatenate([base * np.float32(2.0 ** j) for j in shifts])
    pad = (-x.shape[0]) % 32
    return np.concatenate([x, x[:pad]]) if pad else x


@pytest.mark.parametrize("elem", ELEMS)
def test_hardware_convert_near_every_midpoint(elem):
    """Values within 1..8 ulp of every rounding midpoint and grid value, both
    signs, never exactly on one, with an anchor whose low mantissa bits are
    not zero: every wave of this input rounds with gfx950's scaled convert
    (the exact fallback only runs for waves holding a value whose low
    mantissa bits are all zero, such as a midpoint, a grid value or 0).
    The whole block is also shifted by 2^j over a wide range, which moves
    the scale the convert applies while y stays the same."""
    if elem == O.E2M1:
        grid, anchor, low_bits = O.e2m1_magnitudes(), 0x40FFFFFF, 21    # 7.9999995, e = 0
    else:
        grid, anchor, low_bits = O.e4m3_magnitudes(), 0x43FFFFFF, 19    # 511.99997, e = 0
    mids = (grid[:-1] + grid[1:]) / 2
    pts = _bits(np.concatenate([mids, grid[1:], [448.0 + 16.0]] if elem == O.E4M3
                               else [mids, grid[1:]]))
    near = np.concatenate([pts + d for d in range(-8, 9) if d != 0])
    vals = _f32(near)
    vals = vals[(vals < _f32(anchor)) & (vals > 0)]
    assert np.all((_bits(vals) & ((1 << low_bits) - 1)) != 0)
    vals = np.concatenate([vals, -vals])
    shifts = range(-100, 121 if elem == O.E2M1 else 118)   # the anchor stays finite
    x = _blocks_of(anchor, vals, shifts)
    assert np.all(np.isfinite(x)) and np.all((_bits(x) & ((1 << low_bits) - 1)) != 0)
    codes, scales = check_quantize(x, elem, "near midpoints")
    assert set(np.unique(scales).tolist()) == {127 + j for j in shifts}


@pytest.mark.parametrize("elem", ELEMS)
def test_subnormal_elements_in_a_normal_block(elem):
    """f32 subnormals of both signs next to a normal block maximum: they all
    round to zero magnitude, the negative ones keep their sign bit (code 0x8
    or 0x80), on the hardware-convert path (no element has its low mantissa
    bits all zero)."""
    anchor = 0x40FFFFFF if elem == O.E2M1 else 0x43FFFFFF
    sub = np.arange(1, 0x800000, 4099, dtype=np.int64)
    sub = sub[(sub & 0x1FFFFF) != 0]
    vals = np.concatenate([_f32(sub), -_f32(sub)])
    x = _blocks_of(anchor, vals, [0])
    codes, _ = check_quantize(x, elem, "subnormal elements")
    el = O.unpack_nibbles(codes) if elem == O.E2M1 else codes
    assert np.all((el[:, 1:] & (0x7 if elem == O.E2M1 else 0x7F)) == 0)


def test_e2m1_exhaustive_sweep():
    """Every float32 in [2^-3, 8), both signs (100,663,296 values), 31 per
    block after an anchor forcing e = 0, against the oracle."""
    lo, hi = 0x3E000000, 0x41000000
    allv = np.arange(lo, hi, dtype=np.uint32).view(np.float32)
    vals = np.concatenate([allv, -allv])
    del allv
    nb = -(-vals.size // 31)
    flat = np.zeros(nb * 31, np.float32)
    flat[:vals.size] = vals
    del vals
    x = np.empty((nb, 32), np.float32)
    x[:, 0] = 7.0
    x[:, 1:] = flat.reshape(nb, 31)
    del flat
    gc, gs = gpu_quantize(x, O.E2M1)
    assert np.all(gs == 127)
    step = 1 << 20
    for r0 in range(0, nb, step):
        oc, os_ = O.quantize(x[r0:r0 + step], O.E2M1)
        assert_bits_equal(gs[r0:r0 + step], os_, f"scales, blocks {r0}..")
        assert_bits_equal(gc[r0:r0 + step], oc, f"codes, blocks {r0}..")
        print(f"exhaustive E2M1 sweep: blocks {r0}..{min(nb, r0 + step)} of {nb} match", flush=True)


def test_e4m3_exhaustive_sweep():
    """Every float32 in [2^-10, 512), both signs (318,767,104 values), 31 per
    block after an anchor (511) forcing e = 0, so each code must be the
    nearest E4M3 grid magnitude of |x| itself ("Bit Layout", "Reference
    encode and decode": nearest grid entry, the smaller on a tie, saturating
    at the top).  Checked against that rule in closed form
    (closed_forms.e4m3_codes_at_unit_scale, itself checked against the oracle
    in test_oracle_quantize.py)."""
    lo, hi = 0x3A800000, 0x44000000
    allv = np.arange(lo, hi, dtype=np.uint32).view(np.float32)
    vals = np.concatenate([allv, -allv])
    del allv
    n_vals = vals.size
    nb = -(-n_vals // 31)
    flat = np.zeros(nb * 31, np.float32)                # zero pads after the last value
    flat[:n_vals] = vals
    del vals
    x = np.empty((nb, 32), np.float32)
    x[:, 0] = 511.0
    x[:, 1:] = flat.reshape(nb, 31)
    del flat
    gc, gs = gpu_quantize(x, O.E4M3)
    assert np.all(gs == 127)
    assert np.all(gc[:, 0] == 0x7E)                     # 511 saturates to 448
    step = 1 << 20
    for r0 in range(0, nb, step):
        xs = x[r0:r0 + step, 1:]
        want = e4m3_codes_at_unit_scale(xs)
        got = gc[r0:r0 + step, 1:]
        bad = np.argwhere(got != want)
        assert bad.size == 0, (f"blocks {r0}..: {len(bad)} codes differ, first x="
                               f"{xs[tuple(bad[0])]!r} code {got[tuple(bad[0])]:#x} want "
                               f"{want[tuple(bad[0])]:#x}")
    print(f"exhaustive E4M3 sweep: {n_vals} values in {nb} blocks match the rounding rule", flush=True)


@pytest.mark.parametrize("elem", ELEMS)
def test_exhaustive_decode(elem):
    if elem == O.E2M1:
        el = np.tile(np.concatenate([np.arange(16), np.arange(16)]).astype(np.uint8), (256, 1))
        codes = O.pack_nibbles(el)
        scales = np.arange(256, dtype=np.uint8).reshape(256, 1)
        cols = 32
    else:
        codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
        scales = np.repeat(np.arange(256, dtype=np.uint8).reshape(256, 1), 8, axis=1)
        cols = 256
    y = gpu_dequantize(codes, scales, elem, cols)
    assert_bits_equal(y, O.dequantize(codes, scales, elem, cols), "exhaustive decode")


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("rows,cols", [(1, 32), (3, 96), (5, 1056), (7, 4128), (33, 2080), (1, 65536)])
def test_ragged_sizes_and_guard_bytes(elem, rows, cols):
    rng = np.random.default_rng(rows * 7919 + cols)
    x = (rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-8, 8, (rows, 1)))).astype(np.float32)
    oc, os_ = O.quantize(x, elem)
    guard = 4096
    nbytes = B.mx_codes_bytes(rows, cols, elem)
    nsc = B.mx_num_scale_blocks(rows, cols)
    cbuf = torch.full((nbytes + guard,), 0xAB, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((nsc + guard,), 0xCD, dtype=torch.uint8, device="cuda")
    xd = dev(x)
    B.mx_quantize(xd.data_ptr(), cbuf.data_ptr(), sbuf.data_ptr(), rows, cols, elem)
    c, s = host(cbuf), host(sbuf)
    assert np.all(c[nbytes:] == 0xAB) and np.all(s[nsc:] == 0xCD)
    assert_bits_equal(c[:nbytes], oc.reshape(-1), "codes")
    assert_bits_equal(s[:nsc], os_.reshape(-1), "scales")
    ybuf = torch.full((rows * cols + guard,), 7.0, dtype=torch.float32, device="cuda")
    B.mx_dequantize(cbuf.data_ptr(), sbuf.data_ptr(), ybuf.data_ptr(), rows, cols, elem)
    y = host(ybuf)
    assert np.all(y[rows * cols:] == 7.0)
    assert_bits_equal(y[:rows * cols], O.dequantize(oc, os_, elem, cols).reshape(-1), "dequant")


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("offset", [1, 3, 8])
def test_unaligned_scales_and_guard_bytes(elem, offset):
    """Scale array starting 1, 3 or 8 bytes past a 16-byte boundary: the
    quantize stores scale bytes one by one (no 16-byte pieces); the bytes
    around the array stay untouched."""
    rows, cols = 37, 4160  # 4810 blocks: whole wave iterations and a ragged tail
    rng = np.random.default_rng(offset * 31 + elem)
    x = (rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-6, 6, (rows, 1)))).astype(np.float32)
    oc, os_ = O.quantize(x, elem)
    nbytes = B.mx_codes_bytes(rows, cols, elem)
    nsc = B.mx_num_scale_blocks(rows, cols)
    guard = 4096
    cbuf = torch.full((nbytes + guard,), 0xAB, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((guard + nsc + guard,), 0xCD, dtype=torch.uint8, device="cuda")
    B.mx_quantize(dev(x).data_ptr(), cbuf.data_ptr(), sbuf.data_ptr() + guard + offset, rows, cols,
                  elem)
    c, s = host(cbuf), host(sbuf)
    assert np.all(c[nbytes:] == 0xAB)
    assert np.all(s[:guard + offset] == 0xCD) and np.all(s[guard + offset + nsc:] == 0xCD)
    assert_bits_equal(c[:nbytes], oc.reshape(-1), "codes")
    assert_bits_equal(s[guard + offset:guard + offset + nsc], os_.reshape(-1), "scales")
    y = torch.empty(rows * cols, dtype=torch.float32, device="cuda")
    B.mx_dequantize(cbuf.data_ptr(), sbuf.data_ptr() + guard + offset, y.data_ptr(), rows, cols,
                    elem)
    assert_bits_equal(host(y), O.dequantize(oc, os_, elem, cols).reshape(-1), "dequant")


def test_weight_codec_full_size():
    """8192x8192 N(0, 0.02) with 0.1% outliers x50, quantized in one launch as
    the benchmark does: every code and scale, and every dequantized value,
    bit-exact."""
    x = W.weight_codec_case()
    xd = dev(x)
    t = B.quantize(xd, O.E2M1)
    gc, gs = host(t.codes), host(t.scales)
    step = 1024
    for r0 in range(0, 8192, step):
        oc, os_ = O.quantize(x[r0:r0 + step], O.E2M1)
        assert_bits_equal(gs[r0:r0 + step], os_, f"scales, rows {r0}..")
        assert_bits_equal(gc[r0:r0 + step], oc, f"codes, rows {r0}..")
    y = host(B.dequantize(t))
    assert_bits_equal(y, O.dequantize(gc, gs, O.E2M1, 8192), "dequantize full")


def test_prefill_activation_quantize_full_size():
    """2048x8192 activations (0.5% outliers x20) to E4M3: every code and scale."""
    a, _ = W.prefill_linear_case(N=32)
    t = B.quantize(dev(a), O.E4M3)
    gc, gs = host(t.codes), host(t.scales)
    step = 256
    for r0 in range(0, 2048, step):
        oc, os_ = O.quantize(a[r0:r0 + step], O.E4M3)
        assert_bits_equal(gs[r0:r0 + step], os_, f"scales, rows {r0}..")
        assert_bits_equal(gc[r0:r0 + step], oc, f"codes, rows {r0}..")


@pytest.mark.parametrize("elem", ELEMS)
def test_repeatable(elem):
    x = W.weight_codec_case(512, 4096, seed=3)
    a = gpu_quantize(x, elem)
    b = gpu_quantize(x, elem)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
