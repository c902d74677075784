"""Pins for decode-time appends to a packed head: a hand-worked code, the
clamp for keys outside the packed range, and the identity with packing the
whole sequence under the first part's quantizer (written through the
independent quantize + pack_planes route)."""

import numpy as np

import oracle as O


def test_hand_worked_codes():
    lo = np.array([0.0, -1.0], np.float32)
    step = np.array([0.25, 0.0], np.float32)        # r = 4; a constant channel
    keys = np.array([[1.3, 5.0], [-1.0, -1.0], [100.0, 2.0], [3.99, 0.0]], np.float32)
    codes = O.append_codes(keys, lo, step)
    # 1.3 * 4 = 5.2 -> 5; below lo -> 0; above the range -> 15; 3.99 * 4 = 15.96 -> 15
    assert codes[:, 0].tolist() == [5, 0, 15, 15]
    assert codes[:, 1].tolist() == [0, 0, 0, 0]   # inv = 0 on a constant channel


def test_append_equals_packing_under_the_same_quantizer():
    rng = np.random.default_rng(4)
    n0, m, d = 100, 45, 8
    keys = rng.standard_normal((n0 + m, d)).astype(np.float32)
    lo, hi = O.key_range(keys[:n0])
    step, inv = O.quant_scale(lo, hi)
    keys[n0:] = np.clip(keys[n0:], lo, hi)           # inside the packed range
    ldw = O.plane_ldw(n0 + m)
    planes = O.pack_planes(O.quantize(keys[:n0], lo, inv), ldw)
    grown = O.append_planes(planes, n0, O.append_codes(keys[n0:], lo, step))
    whole = O.pack_planes(O.quantize(keys, lo, inv), ldw)
    assert np.array_equal(grown, whole)


def test_append_replaces_stale_bits_and_keeps_others():
    rng = np.random.default_rng(5)
    d, ldw = 4, 4
    planes = rng.integers(0, 2 ** 32, (d, 4, ldw), dtype=np.uint64).astype(np.uint32)
    codes = rng.integers(0, 16, (3, d)).astype(np.uint8)
    out = O.append_planes(planes, 30, codes)            # keys 30, 31, 32: crosses a word
    bits_before = O.unpack_plane_bits(planes, 128)
    bits_after = O.unpack_plane_bits(out, 128)
    changed = np.any(bits_before != bits_after, axis=(0, 1))
    assert not changed[:30].any() and not changed[33:].any()
    for t in range(3):
        for j in range(4):
            assert bits_after[:, j, 30 + t].tolist() == [(int(c) >> (3 - j)) & 1 for c in codes[t]]
