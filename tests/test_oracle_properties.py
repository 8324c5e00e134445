"""Property pins of the oracle's quantize / dequantize on generated blocks.

Each property follows from the definitions on the "Bit Layout" page
("Reference encode and decode": amax, exponent, nearest grid index, sign from
x < 0; "The E8M0 shared scale": value 2^(byte-127)) and would fail for a
plausible slip in the oracle (a wrong sign rule, an off-by-one exponent, a
mixed-up element or block index):

* sign symmetry: negating a block flips exactly the sign bits of its
  non-zero-magnitude elements and the x < 0 rule for zero magnitudes;
* power-of-two equivariance: scaling a block by 2^k keeps every code and adds
  k to the scale byte while the exponent stays inside [-127, 127];
* permutation: permuting the elements of a block permutes its codes the same
  way and keeps the scale;
* block independence: changing one block changes no other block's codes or
  scale;
* round trip: dequantize(quantize(x)) is within half a grid step (times the
  block scale) of x for every element not above the grid's top.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import mx_oracle as O

ELEMS = [O.E2M1, O.E4M3]
SIGN = {O.E2M1: 0x8, O.E4M3: 0x80}


def elements(codes, elem):
    return O.unpack_nibbles(codes) if elem == O.E2M1 else codes


finite32 = st.floats(min_value=-2.0 ** 124, max_value=2.0 ** 124, allow_nan=False,
                     allow_infinity=False, width=32)


@st.composite
def blocks(draw, n_blocks=2):
    vals = draw(st.lists(finite32, min_size=32 * n_blocks, max_size=32 * n_blocks))
    x = np.array(vals, dtype=np.float32).reshape(1, 32 * n_blocks)
    shift = draw(st.integers(-40, 40))
    with np.errstate(over="ignore"):
        y = x * np.float32(2.0 ** shift)
    return y if np.all(np.isfinite(y)) else x


@pytest.mark.parametrize("elem", ELEMS)
@settings(max_examples=150, deadline=None)
@given(x=blocks())
def test_sign_symmetry(elem, x):
    c, s = O.quantize(x, elem)
    cn, sn = O.quantize(-x, elem)
    assert np.array_equal(s, sn)
    e, en = elements(c, elem), elements(cn, elem)
    mag_mask = SIGN[elem] - 1
    assert np.array_equal(e & mag_mask, en & mag_mask)
    all_zero = np.repeat(~np.abs(x).reshape(-1, 32).any(axis=1), 32)   # all-zero blocks: codes 0
    for i, v in enumerate(x.reshape(-1)):
        if all_zero[i]:
            continue
        assert bool(e.reshape(-1)[i] & SIGN[elem]) == bool(v < 0)
        assert bool(en.reshape(-1)[i] & SIGN[elem]) == bool(-v < 0)


@pytest.mark.parametrize("elem", ELEMS)
@settings(max_examples=150, deadline=None)
@given(x=blocks(), k=st.integers(-20, 20))
def test_power_of_two_equivariance(elem, x, k):
    c, s = O.quantize(x, elem)
    y = x.astype(np.float64) * 2.0 ** k
    with np.errstate(over="ignore"):
        finite = np.all(np.isfinite(y.astype(np.float32)))
    if not finite or np.any(
            (y != 0) & (np.abs(y) < 2.0 ** -100)):
        return                                   # scaling left float32's normal range
    y = y.astype(np.float32)
    if not np.array_equal(y.astype(np.float64), x.astype(np.float64) * 2.0 ** k):
        return                                   # scaling was not exact in float32
    cy, sy = O.quantize(y, elem)
    s_i, sy_i = s.astype(int), sy.astype(int)
    inside = (s_i + k >= 1) & (s_i + k <= 253) & (s_i != 127)   # unclipped, non-zero blocks
    for b in np.flatnonzero(inside.reshape(-1)):
        assert sy_i.reshape(-1)[b] == s_i.reshape(-1)[b] + k
        eb = elements(c, elem).reshape(-1, 32)[b]
        ey = elements(cy, elem).reshape(-1, 32)[b]
        assert np.array_equal(eb, ey)


@pytest.mark.parametrize("elem", ELEMS)
@settings(max_examples=100, deadline=None)
@given(x=blocks(1), perm=st.permutations(list(range(32))))
def test_permutation_within_block(elem, x, perm):
    c, s = O.quantize(x, elem)
    xp = x[:, perm]
    cp, sp = O.quantize(xp, elem)
    assert np.array_equal(s, sp)
    assert np.array_equal(elements(cp, elem)[0], elements(c, elem)[0][perm])


@pytest.mark.parametrize("elem", ELEMS)
@settings(max_examples=100, deadline=None)
@given(x=blocks(3), j=st.integers(0, 31), v=finite32)
def test_block_independence(elem, x, j, v):
    c, s = O.quantize(x, elem)
    x2 = x.copy()
    x2[0, 32 + j] = v                            # change one element of the middle block
    c2, s2 = O.quantize(x2, elem)
    e, e2 = elements(c, elem)[0], elements(c2, elem)[0]
    assert s[0, 0] == s2[0, 0] and s[0, 2] == s2[0, 2]
    assert np.array_equal(e[:32], e2[:32]) and np.array_equal(e[64:], e2[64:])


@pytest.mark.parametrize("elem", ELEMS)
@settings(max_examples=150, deadline=None)
@given(x=blocks())
def test_round_trip_error_bound(elem, x):
    c, s = O.quantize(x, elem)
    y = O.dequantize_f64(c, s, elem, x.shape[1]).reshape(-1, 32)
    xb = x.astype(np.float64).reshape(-1, 32)
    grid = O.e2m1_magnitudes() if elem == O.E2M1 else O.e4m3_magnitudes()
    gaps = np.diff(grid)
    for b in range(xb.shape[0]):
        byte = int(s.reshape(-1)[b])
        scale = 2.0 ** (byte - 127)
        for t in range(32):
            mag = abs(xb[b, t]) / scale
            if mag > grid[-1]:
                assert abs(y[b, t]) == grid[-1] * scale          # saturated
                continue
            i = min(np.searchsorted(grid, mag), len(grid) - 1)
            half = gaps[max(i - 1, 0)] / 2
            assert abs(abs(y[b, t]) - abs(xb[b, t])) <= half * scale * (1 + 1e-12)
