"""Pins for the oracle's fixed-depth control reads (uniform depth; whole
4-bit channels by |q_c|): hand-worked cases, and the properties that fix each
allocation uniquely, checked on random queries at every budget."""

import numpy as np
import pytest

import oracle as O

U, T = O.CONTROL_UNIFORM, O.CONTROL_TOP_CHANNELS


def test_hand_worked():
    # |q| = (.1, .5, .3, .5): order c1, c3 (tie -> lower index), c2, c0
    q = np.array([0.1, -0.5, 0.3, 0.5], np.float32)
    assert O.control_allocation(q, 6, T).tolist() == [0, 4, 0, 2]
    assert O.control_allocation(q, 6, U).tolist() == [1, 2, 1, 2]
    assert O.control_allocation(q, 0, T).tolist() == [0, 0, 0, 0]
    assert O.control_allocation(q, 16, T).tolist() == [4, 4, 4, 4]
    assert O.control_allocation(q, 16, U).tolist() == [4, 4, 4, 4]
    assert O.control_allocation(q, 3, U).tolist() == [0, 1, 1, 1]
    # zero query: the order is the channel index
    z = np.zeros(4, np.float32)
    assert O.control_allocation(z, 5, T).tolist() == [4, 1, 0, 0]
    assert O.control_allocation(z, 5, U).tolist() == [2, 1, 1, 1]


def test_widths_of_the_pages_configurations():
    q = np.random.default_rng(3).standard_normal(128).astype(np.float32)
    top = O.control_allocation(q, 136, T)
    assert (top == 4).sum() == 34 and top.sum() == 136
    uni = O.control_allocation(q, 136, U)
    assert (uni == 2).sum() == 8 and (uni == 1).sum() == 120
    top68 = O.control_allocation(q, 68, T)
    assert (top68 == 4).sum() == 17 and top68.sum() == 68


def _check_properties(q, B, mode, b):
    """Sum, range, and monotonicity in (|q_c| desc, c asc); TOP has at most
    one partial channel and UNIFORM spreads by at most one plane.  Together
    these admit exactly one allocation."""
    d = len(q)
    a = np.abs(q.astype(np.float32))
    assert b.sum() == B and b.min() >= 0 and b.max() <= 4
    for x in range(d):
        for y in range(d):
            before = a[x] > a[y] or (a[x] == a[y] and x < y)
            if before:
                assert b[x] >= b[y], (x, y)
    if mode == T:
        assert ((b > 0) & (b < 4)).sum() <= 1
    else:
        assert b.max() - b.min() <= 1


@pytest.mark.parametrize("mode", [U, T])
def test_properties_every_budget(mode):
    rng = np.random.default_rng(11 + mode)
    for trial in range(6):
        d = int(rng.integers(1, 10))
        q = rng.standard_normal(d).astype(np.float32)
        if trial % 3 == 0:
            q[: d // 2] = q[d - d // 2:][: d // 2]      # duplicated magnitudes
        for B in range(0, 4 * d + 1):
            _check_properties(q, B, mode, O.control_allocation(q, B, mode).astype(np.int64))


def test_rejects_bad_input():
    q = np.ones(4, np.float32)
    with pytest.raises(ValueError):
        O.control_allocation(q, 17, T)
    with pytest.raises(ValueError):
        O.control_allocation(q, 4, 7)
