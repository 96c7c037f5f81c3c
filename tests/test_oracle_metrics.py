"""Pins for the overlap / Jaccard metrics and the greedy layer selection.

Pinned to: set identities (J(A,A) = O(A,A) = 1, disjoint -> 0, J = O/(2-O)
for equal sizes), hand-counted examples, the pages' greedy toy example
("FFSFS") and the pages' forward-count sum K(N-1) - K(K-1)/2.
"""
import json
import os

import numpy as np
import pytest

import oracle


def test_overlap_jaccard_identities():
    rng = np.random.default_rng(0)
    for _ in range(50):
        k = int(rng.integers(1, 20))
        a = rng.choice(100, k, replace=False).astype(np.int32)
        b = rng.choice(100, k, replace=False).astype(np.int32)
        assert oracle.overlap(a, a) == 1.0 and oracle.jaccard(a, a) == 1.0
        o, j = oracle.overlap(a, b), oracle.jaccard(a, b)
        assert abs(j - o / (2 - o)) < 1e-12
        assert oracle.overlap(a, a[::-1]) == 1.0
    a = np.array([0, 1, 2, 3], np.int32)
    assert oracle.overlap(a, a + 10) == 0.0 and oracle.jaccard(a, a + 10) == 0.0


def test_overlap_hand_examples():
    a = np.array([1, 2, 3, 4], np.int32)
    b = np.array([3, 4, 5, 6], np.int32)
    assert oracle.overlap(a, b) == 0.5
    assert oracle.jaccard(a, b) == pytest.approx(2 / 6)
    # -1 padding is not a member
    a = np.array([7, 3, -1, -1], np.int32)
    b = np.array([3, 9, -1, -1], np.int32)
    assert oracle.overlap(a, b) == 0.5
    assert oracle.jaccard(a, b) == pytest.approx(1 / 3)
    m, mn = oracle.mean_overlap(np.stack([a, a]), np.stack([a, b]))
    assert m == 0.75 and mn == 0.5


def test_greedy_toy_example(golden_dir):
    with open(os.path.join(golden_dir, "greedy_toy.json")) as f:
        g = json.load(f)
    imp = g["importance"]

    def loss(p):
        return sum(v for r, v in zip(p, imp) if r == "S")

    pat, evals = oracle.greedy_pattern(g["n_layers"], g["removals"], loss)
    assert pat == g["expected_pattern"]
    assert pat[0] == "F" and pat.count("F") == g["expected_f_count"]
    N, K = g["n_layers"], g["removals"]
    assert evals == K * (N - 1) - K * (K - 1) // 2


def test_greedy_forward_count_formula(golden_dir):
    with open(os.path.join(golden_dir, "greedy_toy.json")) as f:
        g = json.load(f)
    for N, K, want in g["forward_count_cases"]:
        if N <= 12:
            _, evals = oracle.greedy_pattern(N, K, lambda p: p.count("S") * 0.0)
            assert evals == want
        assert K * (N - 1) - K * (K - 1) // 2 == want


def test_overlap_matrix_hand_example():
    # three layers, two rows each; counted by hand
    l0 = np.array([[1, 2, 3, 4], [5, 6, -1, -1]], np.int32)
    l1 = np.array([[3, 4, 5, 6], [5, 7, -1, -1]], np.int32)
    l2 = np.array([[9, 8, 7, 6], [-1, -1, -1, -1]], np.int32)
    m = oracle.overlap_matrix(np.stack([l0, l1, l2]))
    want = np.array([
        [1.0, (2 / 4 + 1 / 2) / 2, (0 / 4 + 0 / 2) / 2],
        [(2 / 4 + 1 / 2) / 2, 1.0, (1 / 4 + 0 / 2) / 2],
        [(0 / 4 + 0.0) / 2, (1 / 4 + 0.0) / 2, 1.0],  # empty A, non-empty B -> 0
    ])
    assert np.allclose(m, want, atol=0, rtol=0)


def test_overlap_matrix_identities():
    rng = np.random.default_rng(1)
    sel = np.stack([np.stack([rng.choice(200, 8, replace=False) for _ in range(5)])] * 3)
    assert np.array_equal(oracle.overlap_matrix(sel), np.ones((3, 3)))
    disjoint = np.stack([np.arange(8, dtype=np.int32).reshape(1, 8) + 8 * i for i in range(4)])
    assert np.array_equal(oracle.overlap_matrix(disjoint), np.eye(4))


def test_overlap_proxy_loss_hand_examples():
    m = np.eye(4)
    m[2, 1], m[2, 0], m[1, 0], m[3, 0] = 0.75, 0.5, 0.25, 0.125
    assert oracle.overlap_proxy_loss("FFFF", m) == 0.0
    assert oracle.overlap_proxy_loss("FFSF", m) == (1 - 0.75) / 4
    assert oracle.overlap_proxy_loss("FSSS", m) == ((1 - 0.25) + (1 - 0.5) + (1 - 0.125)) / 4
    with pytest.raises(ValueError):
        oracle.overlap_proxy_loss("SFFF", m)
