"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)


def test_oracle_full_size_sampled_rows_match_packed_reader(orc):
    """At the lm_head shape, the logical and packed readers of the oracle agree
    on sampled rows (both are oracle code; this checks the packed-index rules at
    a real size, where an off-by-one in tile arithmetic would show)."""
    import numpy as np
    import synthetic
    n, k, g = 152064, 3584, 128
    q, s, x = synthetic.logical(3, n, k, g)
    pw, ps = orc.pack(q, s, g)
    rows = np.array([0, 1, 2, 3, 4, 77777, n - 5, n - 1], np.int64)
    y1, a1 = orc.gemv(q, s, x, g, rows=rows)
    y2, a2 = orc.gemv_packed(pw, ps, x, n, k, g, rows=rows)
    assert np.array_equal(y1, y2) and np.array_equal(a1, a2)
