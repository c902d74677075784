"""Pins for the oracle's per-query allocation (reverse water-filling under a
total budget): hand-worked ladders, brute-force optimality on tiny d,
exchange optimality on d = 128, budget conservation and metamorphic
properties."""

import itertools

import numpy as np
import pytest

import oracle as O


def test_hand_worked_ladder(golden):
    g = golden["allocation_ladder"]
    q = np.array(g["q"], np.float32)
    var = np.array(g["var"], np.float32)
    for B, expect in g["by_budget"].items():
        assert O.allocate(q, var, int(B)).tolist() == expect, B


def test_hand_worked_two_channels(golden):
    g = golden["two_channels"]
    q = np.array(g["q"], np.float32)
    var = np.array(g["var"]["value"], np.float32)
    for key, expect in g["alloc"].items():
        if key == "why":
            continue
        assert O.allocate(q, var, int(key[1:])).tolist() == expect


def _brute_min(w, B):
    d = len(w)
    best = None
    for b in itertools.product(range(5), repeat=d):
        if sum(b) != B:
            continue
        D = O.distortion(w, b)
        best = D if best is None else min(best, D)
    return best


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_optimal(seed):
    """On d <= 5 the allocation reaches the minimum of sum w 4^-b over every
    allocation with sum b = B (checked for every B)."""
    rng = np.random.default_rng(seed)
    d = 3 + seed % 3
    q = rng.standard_normal(d).astype(np.float32)
    var = rng.lognormal(0, 1, d).astype(np.float32)
    if seed % 2:                              # forced ties: duplicated channel
        q[1], var[1] = q[0], var[0]
    w = O.importance(q, var)
    for B in range(4 * d + 1):
        b = O.allocate(q, var, B)
        assert int(b.sum()) == B
        assert np.isclose(O.distortion(w, b), _brute_min(w, B), rtol=1e-12, atol=0)


@pytest.mark.parametrize("seed", range(4))
def test_exchange_optimal_full_width(seed):
    """d = 128: no single-plane exchange lowers the distortion.  The value of
    the last plane taken in any channel is >= the value of the next plane
    of any channel that could still take one."""
    rng = np.random.default_rng(100 + seed)
    q = rng.standard_normal(128).astype(np.float32)
    var = rng.lognormal(0, 1, 128).astype(np.float32)
    w = O.importance(q, var).astype(np.float64)
    for B in (1, 37, 68, 92, 136, 300, 511):
        b = O.allocate(q, var, B).astype(np.int64)
        assert b.sum() == B and b.min() >= 0 and b.max() <= 4
        last = np.where(b > 0, w * 4.0 ** -(b - 1).clip(0), np.inf)
        nxt = np.where(b < 4, w * 4.0 ** -b, -np.inf)
        assert last.min() >= nxt.max()


def test_budget_extremes():
    rng = np.random.default_rng(9)
    q = rng.standard_normal(128).astype(np.float32)
    var = rng.lognormal(0, 1, 128).astype(np.float32)
    assert np.all(O.allocate(q, var, 0) == 0)
    assert np.all(O.allocate(q, var, 512) == 4)
    with pytest.raises(ValueError):
        O.allocate(q, var, 513)
    with pytest.raises(ValueError):
        O.allocate(q, var, -1)


def test_metamorphic():
    rng = np.random.default_rng(21)
    q = rng.standard_normal(128).astype(np.float32)
    var = rng.lognormal(0, 1, 128).astype(np.float32)
    prev = O.allocate(q, var, 0)
    for B in range(1, 513):                    # monotone in B, one plane at a time
        cur = O.allocate(q, var, B)
        assert np.all(cur >= prev) and int((cur - prev).sum()) == 1
        prev = cur
    for m in (-3, 1, 4):                       # q -> 2^m q leaves b unchanged
        q2 = (q * np.float32(2.0 ** m)).astype(np.float32)
        for B in (17, 92, 200):
            assert np.array_equal(O.allocate(q2, var, B), O.allocate(q, var, B))
    perm = rng.permutation(128)                # permuting channels permutes b (no ties)
    for B in (17, 92, 200):
        assert np.array_equal(O.allocate(q[perm], var[perm], B), O.allocate(q, var, B)[perm])


def test_zero_importance_channels_tie_to_low_index():
    q = np.zeros(128, np.float32)
    var = np.ones(128, np.float32)
    b = O.allocate(q, var, 10)
    # all w = 0: every candidate of plane 0 ties (K = 0), lower channels first
    assert b[:10].tolist() == [1] * 10 and b[10:].sum() == 0


def test_continuous_water_level_bracket():
    """The integer allocation sits within one plane of the continuous reverse
    water-filling solution b* = clip(log4(w / theta), 0, 4) at the water level
    theta set by the last plane taken."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal(128).astype(np.float32)
    var = rng.lognormal(0, 1, 128).astype(np.float32)
    w = O.importance(q, var).astype(np.float64)
    for B in (68, 92, 136):
        b = O.allocate(q, var, B)
        taken_vals = [w[c] * 4.0 ** -j for c in range(128) for j in range(int(b[c]))]
        theta = min(taken_vals)
        bstar = np.clip(np.log(w / theta) / np.log(4.0), 0, 4)
        assert np.all(np.abs(b - bstar) <= 1 + 1e-9)


def test_signed_zero_variance_is_zero():
    """-0 and +0 are the same variance: the allocation cannot depend on the
    sign of a zero (a bit-pattern ordering without the +0 normalisation would
    rank -0 channels below every other candidate)."""
    rng = np.random.default_rng(12)
    q = rng.standard_normal(128).astype(np.float32)
    var = rng.lognormal(0, 1, 128).astype(np.float32)
    var[::5] = 0.0
    neg = var.copy()
    neg[::10] = -0.0            # half of the zero channels carry the sign
    assert np.signbit(neg[0]) and not np.signbit(neg[5])
    for B in (0, 1, 100, 300, 400, 450, 511, 512):
        assert np.array_equal(O.allocate(q, neg, B), O.allocate(q, var, B)), B


@pytest.mark.parametrize("bad", [-1.0, np.nan, np.inf])
def test_variance_must_be_finite_and_non_negative(bad):
    var = np.ones(128, np.float32)
    var[7] = bad
    with pytest.raises(AssertionError):
        O.allocate(np.ones(128, np.float32), var, 92)
