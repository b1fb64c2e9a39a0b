"""The fact the device-resident step schedule rests on, checked with the
oracle's own scalars and no library code.

The schedule stores the bias corrections f32(1 - b^t) only up to the first
t at which b^t < 2^-26, and uses the last entry for every later t. That is
exact only if, from that t on, f32(1 - b^t) is exactly 1 for both betas.
In real arithmetic: b^t < 2^-26 < 2^-25 puts 1 - b^t above the midpoint
1 - 2^-25 between the binary32 neighbours 1 - 2^-24 and 1, so it rounds
to 1, and b^t only shrinks as t grows. The test checks this for the
oracle's binary64 power at the boundary, densely after it, and at powers
of two up to 2^62; it also checks that the entry just before the boundary
can still differ from 1 (the table is not longer than it needs to be by
more than that one step)."""
import math

import numpy as np
import pytest

import oracle

BETAS = [0.5, 0.8, 0.9, 0.95, 0.98, 0.99, 0.995, 0.999, 0.9995, 0.9999]


def _table_end(b1, b2):
    """First t with both b1^t and b2^t below 2^-26 (the schedule's rule)."""
    tiny = 2.0 ** -26
    t = 1
    while b1 ** t >= tiny or b2 ** t >= tiny:
        t += 1
    return t


def _bc(b1, b2, t):
    sc = oracle.step_scalars(1e-3, b1, b2, 1e-8, t, 1)
    return float(sc[6]), float(sc[7])


@pytest.mark.parametrize("b2", BETAS)
def test_bias_corrections_are_one_past_the_table(b2):
    b1 = 0.9
    end = _table_end(b1, b2)
    # analytic length: ceil(26 ln 2 / -ln b) for the slower beta
    want = max(math.ceil(26 * math.log(2) / -math.log(b)) for b in (b1, b2))
    assert abs(end - want) <= 1
    for t in list(range(end, end + 2000)) + [end * k for k in (2, 3, 10, 100)] + \
            [2 ** k for k in range(int(math.log2(end)) + 1, 63)]:
        assert _bc(b1, b2, t) == (1.0, 1.0), (b2, t)
    # the table is tight: some t shortly before its end still differs from 1
    lo = max(1, end - 2 * int(math.log(2) / -math.log(max(b1, b2))) - 2)
    assert any(_bc(b1, b2, t) != (1.0, 1.0) for t in range(lo, end))


def test_table_lengths_of_common_betas():
    """Table sizes the library allocates (two floats per step)."""
    assert _table_end(0.9, 0.999) == 18_013
    assert _table_end(0.9, 0.9999) == 180_210
    assert _table_end(0.9, 0.95) == 352
    # 0.99999999 needs ~1.8e9 steps: over the library's 2^22 limit
    assert 26 * math.log(2) / -math.log(0.99999999) > 2 ** 22
    assert np.float32(1 - 0.999 ** 18_013) == np.float32(1.0)
