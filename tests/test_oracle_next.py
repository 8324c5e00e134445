"""Pins of the oracle's fold_scale, axis-0 codec and f32-B block_matmul.

* fold_scale: the E8M0 value set ("Bit Layout", "The E8M0 shared scale":
  byte s stands for 2^(s-127), 0xFF is NaN) searched by brute force, exact
  value scaling of dequantized blocks, and the matmul scale linearity the
  dialect page's "The four ops" relies on for fold_scale.
* axis-0 codec: the hand-worked blocks of tests/golden/worked_examples.json
  placed as columns, block independence, shape checks.
* f32-B block_matmul (the dialect page's "The four ops": block-scaled A,
  ordinary f32 B, C += A.B): exact-rational brute force, identity B, and
  agreement with the quantized-B product when B holds dequantized values.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import mx_oracle as O

from exact_rational import round_f32, value_exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_operand(rng, rows, K, elem, byte_lo=118, byte_hi=136):
    if elem == O.E2M1:
        el = rng.integers(0, 16, (rows, K), dtype=np.uint8)
        codes = O.pack_nibbles(el)
    else:
        el = rng.integers(0, 256, (rows, K), dtype=np.uint8)
        el[(el & 0x7F) == 0x7F] = 0x3C
        codes = el
    scales = rng.integers(byte_lo, byte_hi, (rows, K // 32), dtype=np.uint8)
    return el, codes, scales


# ------------------------------------------------------------------ fold_scale
def _e8m0_value(byte):
    return None if byte == 0xFF else Fraction(2) ** (int(byte) - 127)


def test_fold_scale_brute_force_over_every_byte():
    """For every byte s and shift j: the folded byte's value is 2^j times s's
    value when some finite E8M0 byte has that value, and 0xFF otherwise."""
    values = {b: _e8m0_value(b) for b in range(255)}
    by_value = {v: b for b, v in values.items()}
    all_bytes = np.arange(256, dtype=np.uint8)
    for j in list(range(-300, 301, 7)) + [-255, -254, -128, -1, 0, 1, 127, 254, 255]:
        out = O.fold_scale(all_bytes, j)
        for s in range(256):
            if s == 0xFF:
                assert out[s] == 0xFF
                continue
            want = by_value.get(values[s] * Fraction(2) ** j)
            assert out[s] == (0xFF if want is None else want), (s, j)


@pytest.mark.parametrize("elem", [O.E2M1, O.E4M3])
def test_fold_scale_multiplies_dequantized_values(elem):
    rng = np.random.default_rng(11)
    rows, cols = 6, 128
    _, codes, scales = _rand_operand(rng, rows, cols, elem, 0, 255)
    base = O.dequantize_f64(codes, scales, elem, cols)
    for j in (-40, -3, 0, 5, 90):
        folded = O.fold_scale(scales, j)
        got = O.dequantize_f64(codes, folded, elem, cols)
        ok = np.repeat((scales.astype(int) + j >= 0) & (scales.astype(int) + j <= 254), 32, axis=1)
        assert np.array_equal(got[ok], base[ok] * 2.0 ** j)
        assert np.isnan(got[~ok]).all()


def test_fold_scale_composes_and_keeps_nan():
    s = np.array([3, 100, 127, 200, 251, 255], np.uint8)
    assert np.array_equal(O.fold_scale(O.fold_scale(s, 3), -3), s)
    assert np.array_equal(O.fold_scale(O.fold_scale(s, -3), 3), s)
    assert np.array_equal(O.fold_scale(s, 0), s)
    # a block pushed out of range does not come back
    edge = np.array([0, 254], np.uint8)
    assert np.array_equal(O.fold_scale(edge, -1), [0xFF, 253])
    assert np.array_equal(O.fold_scale(O.fold_scale(edge, 1), -1), [0, 0xFF])


def test_fold_scale_is_matmul_scale_linearity():
    rng = np.random.default_rng(12)
    M, N, K = 4, 5, 96
    _, ac, asc = _rand_operand(rng, M, K, O.E4M3)
    _, bc, bsc = _rand_operand(rng, N, K, O.E2M1)
    c0, _ = O.block_matmul(ac, asc, O.E4M3, bc, bsc, O.E2M1, M, N, K)
    for j in (-6, 4):
        c1, _ = O.block_matmul(ac, O.fold_scale(asc, j), O.E4M3, bc, bsc, O.E2M1, M, N, K)
        assert np.array_equal(c1, (c0.astype(np.float64) * 2.0 ** j).astype(np.float32))


def test_fold_scale_golden_ones_times_halves():
    # The matmul worked example: adding 3 to A's scale byte multiplies C = 32 by 8.
    g = json.load(open(os.path.join(GOLDEN, "worked_examples.json")))["matmul_ones_halves"]
    K = g["K"]
    ac = O.pack_nibbles(np.full((1, K), g["a_code"], np.uint8))
    bc = O.pack_nibbles(np.full((1, K), g["b_code"], np.uint8))
    asc = np.full((1, K // 32), g["a_byte"], np.uint8)
    bsc = np.full((1, K // 32), g["b_byte"], np.uint8)
    shift = g["a_byte_shifted"] - g["a_byte"]
    c, _ = O.block_matmul(ac, O.fold_scale(asc, shift), O.E2M1, bc, bsc, O.E2M1, 1, 1, K)
    assert c[0, 0] == g["c_shifted"]


# ------------------------------------------------------------- axis-0 codec
def _golden_blocks():
    g = json.load(open(os.path.join(GOLDEN, "worked_examples.json")))
    out = []
    for name, e in g.items():
        if not isinstance(e, dict) or "x_head" not in e or "codes_head" not in e:
            continue
        x = np.zeros(e.get("pad_zeros_to", 32), np.float32)
        x[:len(e["x_head"])] = np.array(e["x_head"], np.float32)
        out.append((name, e, x))
    return out


@pytest.mark.parametrize("elem_name", ["E2M1", "E4M3"])
def test_axis0_golden_blocks_as_columns(elem_name):
    elem = O.E2M1 if elem_name == "E2M1" else O.E4M3
    blocks = [(n, e, x) for n, e, x in _golden_blocks() if e["elem"] == elem_name]
    assert blocks
    # column c of a [64, C] matrix: the golden block in rows 0..31, zeros below
    mat = np.zeros((64, len(blocks)), np.float32)
    for c, (_, _, x) in enumerate(blocks):
        mat[:32, c] = x
    codes, scales = O.quantize_axis0(mat, elem)
    assert scales.shape == (len(blocks), 2)
    el = O.unpack_nibbles(codes) if elem == O.E2M1 else codes
    for c, (name, e, _) in enumerate(blocks):
        assert scales[c, 0] == e["scale_byte"], name
        assert scales[c, 1] == 127, name                  # the all-zero block below
        head = e["codes_head"]
        assert list(el[c, :len(head)]) == head, name
        assert not el[c, 32:].any()
    y = O.dequantize_axis0(codes, scales, elem, 64)
    assert y.shape == mat.shape
    for c, (name, e, _) in enumerate(blocks):
        if "decoded_head" in e:
            head = np.array(e["decoded_head"], np.float32)
            assert np.array_equal(y[:len(head), c].view(np.uint32), head.view(np.uint32)), name


def test_axis0_blocks_are_independent():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((96, 40)).astype(np.float32)
    c0, s0 = O.quantize_axis0(x, O.E4M3)
    x2 = x.copy()
    x2[40, 7] = 1000.0                                   # block (1, 7): rows 32..63 of column 7
    c1, s1 = O.quantize_axis0(x2, O.E4M3)
    diff_s = np.argwhere(s0 != s1)
    assert diff_s.tolist() == [[7, 1]]
    diff_c = np.argwhere(c0 != c1)
    assert set(diff_c[:, 0]) == {7} and diff_c[:, 1].min() >= 32 and diff_c[:, 1].max() < 64


def test_axis0_rejects_ragged_rows():
    with pytest.raises(ValueError):
        O.quantize_axis0(np.zeros((48, 8), np.float32), O.E2M1)


# ----------------------------------------------------------- f32-B matmul
def _exact_value(code, byte, elem):
    return value_exact(code, byte, elem == O.E2M1)


@pytest.mark.parametrize("elem", [O.E2M1, O.E4M3])
@pytest.mark.parametrize("K", [32, 64])
def test_f32b_brute_force_exact_rationals(elem, K):
    rng = np.random.default_rng(K + elem)
    M, N = 3, 4
    el, ac, asc = _rand_operand(rng, M, K, elem)
    b = (rng.standard_normal((K, N)) * np.exp2(rng.integers(-30, 30, (K, N)))).astype(np.float32)
    c, mag = O.block_matmul_f32b(ac, asc, elem, b, M, N, K)
    for m in range(M):
        for n in range(N):
            terms = [_exact_value(int(el[m, k]), asc[m, k // 32], elem) * Fraction(float(b[k, n]))
                     for k in range(K)]
            assert c[m, n] == round_f32(sum(terms))
            absum = float(sum(abs(t) for t in terms))
            assert abs(mag[m, n] - absum) <= 1e-12 * absum


def test_f32b_identity_returns_dequantized_a():
    rng = np.random.default_rng(21)
    M, K = 5, 64
    _, ac, asc = _rand_operand(rng, M, K, O.E4M3)
    c, _ = O.block_matmul_f32b(ac, asc, O.E4M3, np.eye(K, dtype=np.float32), M, K, K)
    assert np.array_equal(c, O.dequantize(ac, asc, O.E4M3, K))


def test_f32b_agrees_with_quantized_b_product():
    rng = np.random.default_rng(22)
    M, N, K = 6, 7, 128
    _, ac, asc = _rand_operand(rng, M, K, O.E2M1)
    _, bc, bsc = _rand_operand(rng, N, K, O.E4M3)
    b = np.ascontiguousarray(O.dequantize(bc, bsc, O.E4M3, K).T)   # exact float32 [K, N]
    c1, m1 = O.block_matmul_f32b(ac, asc, O.E2M1, b, M, N, K)
    c2, m2 = O.block_matmul(ac, asc, O.E2M1, bc, bsc, O.E4M3, M, N, K)
    assert np.array_equal(c1, c2)
    assert np.allclose(m1, m2, rtol=1e-15, atol=0)


def test_f32b_accumulate_brute_force_exact_rationals():
    # "The accumulator operand" with the page's f32 B: C_in + A.B formed
    # exactly and rounded to float32 once.
    rng = np.random.default_rng(23)
    M, N, K = 4, 3, 64
    el, ac, asc = _rand_operand(rng, M, K, O.E2M1)
    b = (rng.standard_normal((K, N)) * np.exp2(rng.integers(-6, 6, (K, N)))).astype(np.float32)
    cin = rng.standard_normal((M, N)).astype(np.float32)
    c, mag = O.block_matmul_f32b(ac, asc, O.E2M1, b, M, N, K, c_in=cin, accumulate=True)
    for m in range(M):
        for n in range(N):
            terms = [_exact_value(int(el[m, k]), asc[m, k // 32], O.E2M1) * Fraction(float(b[k, n]))
                     for k in range(K)]
            exact = Fraction(float(cin[m, n])) + sum(terms)
            assert c[m, n] == round_f32(exact)
            absum = float(abs(Fraction(float(cin[m, n]))) + sum(abs(t) for t in terms))
            assert abs(mag[m, n] - absum) <= 1e-12 * absum


def test_f32b_accumulate_rounds_once():
    # A row: 1.0 and 0.5 under scale byte 103 (2^-24 and 2^-25); B column:
    # 1.0 and 2^-25.  A.B = 2^-24 + 2^-50, C_in = 1: one rounding gives
    # 1 + 2^-23, rounding A.B to float32 first gives 1.0.
    el = np.zeros((1, 32), np.uint8)
    el[0, 0], el[0, 1] = 0x2, 0x1
    ac, asc = O.pack_nibbles(el), np.array([[103]], np.uint8)
    b = np.zeros((32, 1), np.float32)
    b[0, 0], b[1, 0] = 1.0, 2.0 ** -25
    c, _ = O.block_matmul_f32b(ac, asc, O.E2M1, b, 1, 1, 32, c_in=np.ones((1, 1), np.float32),
                               accumulate=True)
    want = round_f32(1 + Fraction(1, 2 ** 24) + Fraction(1, 2 ** 50))
    assert want == np.float32(1 + 2.0 ** -23) and c[0, 0] == want
    assert np.float32(1.0) + np.float32(2.0 ** -24 + 2.0 ** -50) != want


def test_f32b_nan_scale_poisons_its_row():
    rng = np.random.default_rng(24)
    M, N, K = 4, 3, 64
    _, ac, asc = _rand_operand(rng, M, K, O.E2M1)
    b = rng.standard_normal((K, N)).astype(np.float32)
    asc = asc.copy()
    asc[2, 1] = 0xFF
    c2, _ = O.block_matmul_f32b(ac, asc, O.E2M1, b, M, N, K)
    assert np.isnan(c2[2]).all() and not np.isnan(np.delete(c2, 2, axis=0)).any()
