"""Pins for the oracle's quantizer, bit planes and channel variance.

Each test checks the oracle against something other than itself: hand-worked
values, an independently written t-bit quantizer, a textbook variance routine
or an exact round trip.
"""

import numpy as np
import pytest

import oracle as O
from sparse_kv_cache_amd import synth


def test_plane_ldw():
    assert O.plane_ldw(1) == 4
    assert O.plane_ldw(32 * 4) == 4
    assert O.plane_ldw(32 * 4 + 1) == 8
    assert O.plane_ldw(4096) == 128
    assert O.plane_ldw(131072) == 4096
    assert O.plane_ldw(1 << 20) == 32768


def test_hand_worked_one_channel(golden):
    g = golden["one_channel"]
    keys = np.array(g["keys"], np.float32)[:, None]
    planes, lo, step, var, codes = O.pack_head(keys)
    assert lo[0] == g["lo"] and step[0] == g["step"]
    assert codes[:, 0].tolist() == g["codes"]
    assert planes[0, :, 0].tolist() == g["plane_words"]["word0"]
    assert np.all(planes[0, :, 1:] == 0)
    assert var[0] == np.float32(g["var"]["value"])


def test_hand_worked_two_channels(golden):
    g = golden["two_channels"]
    keys = np.array(g["keys"], np.float32)
    planes, lo, step, var, codes = O.pack_head(keys)
    assert lo.tolist() == g["lo"] and step.tolist() == g["step"]
    assert codes.tolist() == g["codes"]
    assert var.tolist() == g["var"]["value"]


def _tbit_quantizer(keys, lo, hi, t):
    """Independent t-bit floor quantizer on [lo, hi] with 2^t bins, written
    directly (not by truncating 4-bit codes)."""
    r = (hi - lo).astype(np.float32)
    inv_t = np.zeros_like(r)
    pos = r > 0
    inv_t[pos] = np.float32(2 ** t) / r[pos]
    u = ((keys - lo[None, :]).astype(np.float32) * inv_t[None, :]).astype(np.float32)
    return np.minimum(np.floor(u), 2 ** t - 1).astype(np.int64)


@pytest.mark.parametrize("seed", [0, 1, 7])
def test_prefix_is_tbit_quantizer(seed):
    """A t-plane prefix read from the packed planes equals the channel's t-bit
    quantizer, for t = 0..4 (the property the pages rest on)."""
    keys = synth.forced_tie_keys(seed, 3000, 128)
    n = keys.shape[0]
    planes, lo, step, var, codes = O.pack_head(keys)
    lo_, hi_ = O.key_range(keys)
    bits = O.unpack_plane_bits(planes, n).astype(np.int64)     # [d, 4, n]
    for t in range(5):
        prefix = np.zeros((keys.shape[1], n), np.int64)
        for j in range(t):
            prefix = (prefix << 1) | bits[:, j, :]
        direct = _tbit_quantizer(keys, lo_, hi_, t).T
        assert np.array_equal(prefix, direct), f"t={t}"


def test_planes_round_trip_and_padding():
    rng = np.random.default_rng(3)
    n = 1000          # ragged: not a multiple of 32
    keys = rng.standard_normal((n, 128), dtype=np.float32)
    planes, lo, step, var, codes = O.pack_head(keys)
    assert planes.shape == (128, 4, O.plane_ldw(n))
    bits = O.unpack_plane_bits(planes, O.plane_ldw(n) * 32).astype(np.int64)
    rebuilt = bits[:, 0] * 8 + bits[:, 1] * 4 + bits[:, 2] * 2 + bits[:, 3]
    assert np.array_equal(rebuilt[:, :n].T, codes.astype(np.int64))
    assert np.all(bits[:, :, n:] == 0)


def test_code_range_and_extremes():
    keys = synth.forced_tie_keys(5, 2048, 128)
    _, lo, step, var, codes = O.pack_head(keys)
    assert codes.min() >= 0 and codes.max() <= 15
    # every non-constant channel uses both end bins (its min and max keys)
    nonconst = step > 0
    assert np.all(codes.min(axis=0)[nonconst] == 0)
    assert np.all(codes.max(axis=0)[nonconst] == 15)
    # the constant channel quantizes to 0 with zero step and variance
    assert step[0] == 0 and var[0] == 0 and np.all(codes[:, 0] == 0)


@pytest.mark.parametrize("seed", [0, 2])
def test_variance_against_numpy_var(seed):
    """The exact-integer-moment variance agrees with numpy's float64 variance
    of the dequantized reconstructions to fp32 rounding."""
    keys = synth.forced_tie_keys(seed, 5000, 128)
    _, lo, step, var, codes = O.pack_head(keys)
    recon = lo.astype(np.float64)[None, :] + (codes.astype(np.float64) + 0.5) * step.astype(np.float64)[None, :]
    ref = np.var(recon, axis=0)
    assert np.allclose(var.astype(np.float64), ref, rtol=2e-7, atol=1e-30)


def test_quant_scale_is_correctly_rounded():
    rng = np.random.default_rng(11)
    lo = rng.standard_normal(1000).astype(np.float32)
    hi = (lo + rng.random(1000).astype(np.float32) * 10).astype(np.float32)
    step, inv = O.quant_scale(lo, hi)
    r = (hi - lo).astype(np.float32)
    # 16 / r correctly rounded: |inv - 16/r| <= half an ulp of inv
    exact = 16.0 / r.astype(np.float64)
    ulp = np.spacing(inv.astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(inv.astype(np.float64) - exact) <= 0.5 * ulp)
    assert np.array_equal(step, (r / np.float32(16)).astype(np.float32))
