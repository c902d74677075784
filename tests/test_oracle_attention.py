"""Pins for the oracle's attention over selected rows: closed forms (equal
keys give the plain mean of the values; one dominant key gives its value;
two keys by hand), the dense/sparse identity on the full index set,
invariance to the order of the index set and to a common shift of the
scores, and the error measure."""

import numpy as np
import pytest

import oracle as O


def test_equal_keys_give_the_mean_value():
    rng = np.random.default_rng(1)
    K = np.tile(rng.standard_normal((1, 8)), (5, 1))
    V = rng.standard_normal((5, 8))
    q = rng.standard_normal(8).astype(np.float32)
    assert np.allclose(O.attention(K, V, q, 0.3), V.mean(axis=0), rtol=0, atol=1e-14)


def test_dominant_key_gives_its_value():
    d = 6
    K = np.zeros((4, d))
    K[2, 0] = 1000.0
    V = np.arange(24, dtype=np.float64).reshape(4, d)
    q = np.zeros(d, np.float32)
    q[0] = 1.0
    assert np.allclose(O.attention(K, V, q, 1.0), V[2], rtol=0, atol=1e-12)


def test_two_keys_by_hand():
    # scores 0 and ln 3 after scaling: weights 1/4 and 3/4
    K = np.array([[0.0, 0.0], [np.log(3.0) / 0.5, 0.0]])
    V = np.array([[4.0, 0.0], [0.0, 8.0]])
    q = np.array([1.0, 0.0], np.float32)
    assert np.allclose(O.attention(K, V, q, 0.5), [1.0, 6.0], rtol=0, atol=1e-12)


def test_full_index_set_is_dense_and_order_free():
    rng = np.random.default_rng(2)
    n, d = 300, 16
    K = rng.standard_normal((n, d)).astype(np.float32)
    V = rng.standard_normal((n, d)).astype(np.float32)
    q = rng.standard_normal(d).astype(np.float32)
    dense = O.attention(K, V, q, d ** -0.5)
    perm = rng.permutation(n)
    assert np.allclose(O.sparse_attention(K, V, q, perm, d ** -0.5), dense, rtol=1e-12, atol=1e-12)
    sub = perm[:40]
    a = O.sparse_attention(K, V, q, sub, d ** -0.5)
    b = O.sparse_attention(K, V, q, sub[::-1], d ** -0.5)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)
    assert O.attention_error(dense, dense) == 0.0
    assert O.attention_error(a, dense) > 0.0


def test_shift_invariance_of_scores():
    # adding the same vector to every key along q's direction shifts all
    # scores equally, which the softmax ignores
    rng = np.random.default_rng(3)
    K = rng.standard_normal((20, 4))
    V = rng.standard_normal((20, 4))
    q = np.array([1.0, 0.0, 0.0, 0.0], np.float32)
    shifted = K + np.array([5.0, 0.0, 0.0, 0.0])
    assert np.allclose(O.attention(K, V, q, 0.7), O.attention(shifted, V, q, 0.7), rtol=1e-12, atol=1e-12)


def test_empty_rows_rejected():
    with pytest.raises(ValueError):
        O.attention(np.zeros((0, 4)), np.zeros((0, 4)), np.zeros(4, np.float32), 1.0)
