"""Pins of the oracle's Hadamard matrix against definitions other than its own
construction (Walsh functions, integer orthogonality, the butterfly transform)."""
import numpy as np
import pytest

import oracle


def _popcount(v):
    return bin(v).count("1")


def test_sylvester_entries_are_walsh_functions():
    # S[i][j] = (-1)^popcount(i & j), a definition independent of the doubling
    S = oracle.sylvester(128)
    ref = np.array([[(-1) ** _popcount(i & j) for j in range(128)] for i in range(128)])
    assert np.array_equal(S, ref)


def test_sylvester_is_orthogonal_in_integers():
    S = oracle.sylvester(128)
    assert np.array_equal(S @ S.T, 128 * np.eye(128, dtype=np.int64))


def test_small_orders_by_hand():
    assert oracle.sylvester(2).tolist() == [[1, 1], [1, -1]]
    assert oracle.sylvester(4).tolist() == [[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]]


def test_normalised_matrix_is_a_symmetric_involution():
    H = oracle.hadamard(128)
    assert np.array_equal(H, H.T)
    assert np.max(np.abs(H @ H - np.eye(128))) < 1e-15
    assert np.allclose(np.abs(H), 1 / np.sqrt(128), rtol=0, atol=1e-17)


def _butterfly(v):
    v = np.array(v, dtype=np.float64)
    h = 1
    while h < len(v):
        for i in range(0, len(v), 2 * h):
            for j in range(i, i + h):
                a, b = v[j], v[j + h]
                v[j], v[j + h] = a + b, a - b
        h *= 2
    return v


def test_butterfly_transform_equals_matrix():
    S = oracle.sylvester(128)
    for k in (0, 1, 5, 64, 127):
        e = np.zeros(128)
        e[k] = 1
        assert np.array_equal(_butterfly(e), S[:, k])
    x = np.random.default_rng(0).standard_normal(128)
    assert np.allclose(_butterfly(x) / np.sqrt(128), oracle.hadamard(128) @ x, rtol=0, atol=1e-13)


def test_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        oracle.sylvester(96)
