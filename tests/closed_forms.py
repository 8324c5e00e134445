"""Closed forms of the rounding rule, independent of the oracle and of the
GPU path, for checks too large for the oracle's argmin.

"Bit Layout", "Reference encode and decode": an element's code is the index
of the grid magnitude nearest to |x| / 2^e, the smaller index on a tie,
saturating at the top of the grid, with the sign bit set for negative x.
"""
import numpy as np


def e4m3_magnitudes() -> np.ndarray:
    """The 127 finite f8E4M3FN magnitudes from their bit formula: code c =
    (e << 3) | m gives (1 + m/8) 2^(e-7) for e >= 1 and m 2^-9 for e = 0."""
    c = np.arange(127)
    e, m = c >> 3, (c & 7).astype(np.float64)
    return np.where(e == 0, m * 2.0 ** -9, (1 + m / 8) * np.exp2(e.astype(np.float64) - 7))


def e4m3_codes_at_unit_scale(y: np.ndarray) -> np.ndarray:
    """E4M3 codes of values y already divided by their block scale: the
    magnitude index is the number of grid midpoints strictly below |y|
    (np.searchsorted, side "left", so a value on a midpoint takes the smaller
    index; values above the last midpoint take the top, 448), and 0x80 marks
    y < 0.  Midpoints of float64 grid values are exact in float64."""
    grid = e4m3_magnitudes()
    mids = (grid[:-1] + grid[1:]) / 2
    mag = np.searchsorted(mids, np.abs(np.asarray(y, np.float64)), side="left")
    return (mag | np.where(np.asarray(y) < 0, 0x80, 0)).astype(np.uint8)
