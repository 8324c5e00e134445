"""Pins of the oracle's block_matmul: exact rational brute force and
algebraic properties fixed by the dialect page ("The four ops", "The block
axis") and the E8M0 scale definition ("Bit Layout", "The E8M0 shared scale").
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
        el[(el & 0x7F) == 0x7F] = 0x3C            # keep the E4M3 NaN codes out
        codes = el
    scales = rng.integers(byte_lo, byte_hi, (rows, K // 32), dtype=np.uint8)
    return el, codes, scales


def _value_exact(code, byte, elem):
    return value_exact(code, byte, elem == O.E2M1)


@pytest.mark.parametrize("a_elem,b_elem", [(O.E2M1, O.E2M1), (O.E4M3, O.E4M3), (O.E4M3, O.E2M1)])
@pytest.mark.parametrize("K", [32, 64, 96])
def test_brute_force_exact_rationals(a_elem, b_elem, K):
    rng = np.random.default_rng(K * 10 + a_elem * 3 + b_elem)
    M, N = 3, 4
    ae, ac, asc = _rand_operand(rng, M, K, a_elem)
    be, bc, bsc = _rand_operand(rng, N, K, b_elem)
    c, mag = O.block_matmul(ac, asc, a_elem, bc, bsc, b_elem, M, N, K)
    for m in range(M):
        for n in range(N):
            exact = sum(_value_exact(int(ae[m, k]), asc[m, k // 32], a_elem) *
                        _value_exact(int(be[n, k]), bsc[n, k // 32], b_elem) for k in range(K))
            # the exact sum rounded once to float32
            assert c[m, n] == round_f32(exact)
            absum = sum(abs(_value_exact(int(ae[m, k]), asc[m, k // 32], a_elem) *
                            _value_exact(int(be[n, k]), bsc[n, k // 32], b_elem)) for k in range(K))
            # the tolerance scale only needs to be accurate, not exact
            assert abs(mag[m, n] - float(absum)) <= 1e-12 * float(absum)


def test_golden_ones_times_halves():
    g = json.load(open(os.path.join(GOLDEN, "worked_examples.json")))["matmul_ones_halves"]
    K = g["K"]
    ac = O.pack_nibbles(np.full((1, K), g["a_code"], np.uint8))
    bc = O.pack_nibbles(np.full((1, K), g["b_code"], np.uint8))
    asc = np.full((1, K // 32), g["a_byte"], np.uint8)
    bsc = np.full((1, K // 32), g["b_byte"], np.uint8)
    c, _ = O.block_matmul(ac, asc, O.E2M1, bc, bsc, O.E2M1, 1, 1, K)
    assert c[0, 0] == g["c"]
    asc2 = np.full((1, K // 32), g["a_byte_shifted"], np.uint8)
    c2, _ = O.block_matmul(ac, asc2, O.E2M1, bc, bsc, O.E2M1, 1, 1, K)
    assert c2[0, 0] == g["c_shifted"]


def test_one_hot_b_selects_a_column():
    rng = np.random.default_rng(1)
    M, K = 5, 96
    _, ac, asc = _rand_operand(rng, M, K, O.E4M3)
    adq = O.dequantize(ac, asc, O.E4M3, K)
    for k in (0, 31, 32, 95):
        el = np.zeros((1, K), np.uint8)
        el[0, k] = 0x2                             # E2M1 code of 1.0
        bsc = np.full((1, K // 32), 127, np.uint8)
        c, _ = O.block_matmul(ac, asc, O.E4M3, O.pack_nibbles(el), bsc, O.E2M1, M, 1, K)
        assert np.array_equal(c[:, 0], adq[:, k])


def test_scale_linearity():
    # Adding j to every A scale byte multiplies C by exactly 2^j (no over/underflow).
    rng = np.random.default_rng(2)
    M, N, K = 4, 6, 128
    _, ac, asc = _rand_operand(rng, M, K, O.E2M1)
    _, bc, bsc = _rand_operand(rng, N, K, O.E4M3)
    c0, _ = O.block_matmul(ac, asc, O.E2M1, bc, bsc, O.E4M3, M, N, K)
    for j in (-5, 3, 7):
        c1, _ = O.block_matmul(ac, (asc.astype(int) + j).astype(np.uint8), O.E2M1,
                               bc, bsc, O.E4M3, M, N, K)
        assert np.array_equal(c1, (c0.astype(np.float64) * 2.0 ** j).astype(np.float32))


@pytest.mark.parametrize("a_elem,b_elem", [(O.E2M1, O.E2M1), (O.E4M3, O.E2M1), (O.E4M3, O.E4M3)])
def test_accumulate_brute_force_exact_rationals(a_elem, b_elem):
    # "The accumulator operand": C = C_in + A.B.  The oracle forms C_in + A.B
    # exactly (every partial sum fits float64 at these sizes and scales) and
    # rounds it to float32 once.
    rng = np.random.default_rng(40 + a_elem * 3 + b_elem)
    M, N, K = 3, 4, 64
    ae, ac, asc = _rand_operand(rng, M, K, a_elem, 124, 131)
    be, bc, bsc = _rand_operand(rng, N, K, b_elem, 124, 131)
    cin = (rng.standard_normal((M, N)) * 2.0 ** rng.integers(-3, 4, (M, N))).astype(np.float32)
    c, mag = O.block_matmul(ac, asc, a_elem, bc, bsc, b_elem, M, N, K, c_in=cin, accumulate=True)
    for m in range(M):
        for n in range(N):
            terms = [_value_exact(int(ae[m, k]), asc[m, k // 32], a_elem) *
                     _value_exact(int(be[n, k]), bsc[n, k // 32], b_elem) for k in range(K)]
            exact = Fraction(float(cin[m, n])) + sum(terms)
            assert c[m, n] == round_f32(exact)
            absum = abs(Fraction(float(cin[m, n]))) + sum(abs(t) for t in terms)
            assert abs(mag[m, n] - float(absum)) <= 1e-12 * float(absum)


def _two_block_row(codes01, bytes01):
    """One E2M1 row of K = 64: element 0 of block j has code codes01[j], the
    rest are zero; block j has scale byte bytes01[j]."""
    el = np.zeros((1, 64), np.uint8)
    el[0, 0], el[0, 32] = codes01
    return O.pack_nibbles(el), np.array([bytes01], np.uint8)


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_accumulate_rounds_once(sign):
    # A.B = 2^-24 + 2^-50 (two blocks, 1.0 x 1.0 under scale bytes 115 and
    # 102 on both sides) and C_in = 1: the exact sum 1 + 2^-24 + 2^-50 lies
    # above the midpoint between 1 and 1 + 2^-23, so it rounds to 1 + 2^-23.
    # Rounding A.B to float32 first (to 2^-24) and then adding C_in lands on
    # the midpoint and rounds to even, 1.0: a double rounding fails here.
    s = 0x8 if sign < 0 else 0x0
    ac, asc = _two_block_row((0x2 | s, 0x2 | s), (115, 102))
    bc, bsc = _two_block_row((0x2, 0x2), (115, 102))
    cin = np.array([[sign]], np.float32)
    c, _ = O.block_matmul(ac, asc, O.E2M1, bc, bsc, O.E2M1, 1, 1, 64, c_in=cin, accumulate=True)
    exact = Fraction(int(sign)) * (1 + Fraction(1, 2 ** 24) + Fraction(1, 2 ** 50))
    want = round_f32(exact)
    assert want == np.float32(sign * (1 + 2.0 ** -23))
    assert c[0, 0] == want
    ab_first = np.float32(sign * (2.0 ** -24 + 2.0 ** -50))           # A.B rounded on its own
    assert np.float32(np.float32(sign) + ab_first) != want          # the slip this pin catches


def test_nan_scale_propagates_to_row_and_column():
    rng = np.random.default_rng(6)
    M, N, K = 4, 5, 64
    _, ac, asc = _rand_operand(rng, M, K, O.E2M1)
    _, bc, bsc = _rand_operand(rng, N, K, O.E2M1)
    asc = asc.copy(); bsc = bsc.copy()
    asc[1, 1] = 0xFF
    bsc[3, 0] = 0xFF
    c, _ = O.block_matmul(ac, asc, O.E2M1, bc, bsc, O.E2M1, M, N, K)
    nan = np.isnan(c)
    assert nan[1, :].all() and nan[:, 3].all()
    assert nan.sum() == N + M - 1


def test_entries_match_full_product():
    rng = np.random.default_rng(8)
    M, N, K = 7, 9, 160
    _, ac, asc = _rand_operand(rng, M, K, O.E4M3)
    _, bc, bsc = _rand_operand(rng, N, K, O.E2M1)
    c, mag = O.block_matmul(ac, asc, O.E4M3, bc, bsc, O.E2M1, M, N, K)
    rows = np.array([0, 6, 3, 3])
    cols = np.array([8, 0, 4, 5])
    ce, me = O.block_matmul_entries(ac, asc, O.E4M3, bc, bsc, O.E2M1, K, rows, cols)
    assert np.array_equal(ce, c[rows, cols])
    assert np.allclose(me, mag[rows, cols], rtol=1e-15)
