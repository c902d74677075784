"""CPU model of the allocation kernel's two-stage water-level search.

The kernel finds the B-th largest candidate key (channel top key minus
j 2^24, j = 0..3, as unsigned offsets u) without sorting the 512 candidates:
a search on the top byte T of u, then the (m + 1)-th smallest low 24 bits f
over the channels whose count still changes inside [T 2^24, (T + 1) 2^24).
This model restates those two stages in numpy and checks them against a full
sort of the candidates, which is the definition, on random weights with
zeros, ties and every budget range; it also checks that the selected rank,
taken from the nearer end, never exceeds 64 (the kernel's selection limit).
"""

import numpy as np

S24 = 1 << 24


def _by_sort(u, B):
    cand = np.concatenate([u - j * S24 for j in range(4)])
    return int(np.sort(cand)[::-1][B - 1])


def _two_stage(u, B):
    U, f = u >> 24, u & (S24 - 1)

    def count_at(T):   # candidates >= T 2^24
        return int(np.clip(U - T + 1, 0, 4).sum())

    lo, hi = 0, 256    # count_at(0) = 512 >= B > count_at(256) = 0
    while hi - lo > 1:
        step = max(1, (hi - lo) // 4)
        t1 = min(lo + step, hi - 1)
        t2 = min(t1 + step, hi - 1)
        t3 = min(t2 + step, hi - 1)
        if count_at(t3) >= B:
            lo = t3
        elif count_at(t2) >= B:
            lo, hi = t2, t3
        elif count_at(t1) >= B:
            lo, hi = t1, t2
        else:
            hi = t1
    a = U - lo + 1
    in_play = (a >= 1) & (a <= 4)
    m = count_at(lo) - B
    s = int(in_play.sum())
    assert 0 <= m < s
    rank = min(m + 1, s - m)
    assert rank <= 64
    return lo * S24 + int(np.sort(f[in_play])[m])


def test_two_stage_search_equals_sorted_candidates():
    rng = np.random.default_rng(7)
    for trial in range(3000):
        scale = rng.choice([1e-6, 1e-2, 1.0, 1e3])
        w = (rng.standard_normal(128) ** 2 * rng.lognormal(0, rng.choice([0.1, 1, 3]), 128) * scale)
        w = w.astype(np.float32)
        if trial % 7 == 0:
            w[rng.integers(0, 128, 20)] = 0.0
        if trial % 11 == 0:
            w[:] = w[0]
        u = w.view(np.int32).astype(np.int64) + 3 * S24
        B = int(rng.integers(1, 512))
        assert _two_stage(u, B) == _by_sort(u, B), (trial, B)
