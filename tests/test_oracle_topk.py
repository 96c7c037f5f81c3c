"""Pins for the oracle's per-query top-k.

Pinned to: brute-force enumeration of subsets on tiny rows (the unique subset
whose every member beats every non-member), library sort on distinct scores,
all-equal rows (the first positions), signed zero handling and causality.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle


def _canon(v):
    v = np.array(v, dtype=np.float32, copy=True)
    v[v == 0] = 0.0
    return v


def brute_force_topk_set(row, n_cand, k):
    vals = _canon(row[:n_cand])

    def beats(a, b):
        return vals[a] > vals[b] or (vals[a] == vals[b] and a < b)

    m = min(k, n_cand)
    found = []
    for sub in itertools.combinations(range(n_cand), m):
        inside = set(sub)
        if all(beats(a, b) for a in inside for b in range(n_cand) if b not in inside):
            found.append(inside)
    assert len(found) == 1
    return found[0]


def test_topk_brute_force_tiny_rows():
    rng = np.random.default_rng(11)
    for trial in range(60):
        n = int(rng.integers(1, 9))
        row = rng.integers(-2, 3, n).astype(np.float32)  # heavy ties
        if trial % 3 == 0:
            row = np.where(row == 0, -0.0, row).astype(np.float32)
        for k in range(1, 10):
            for n_cand in range(1, n + 1):
                got = oracle.topk_row(row, n_cand, k)
                m = min(k, n_cand)
                assert (got[m:] == -1).all()
                assert set(got[:m].tolist()) == brute_force_topk_set(row, n_cand, k)
                # sorted under the total order
                v = _canon(row)
                for a, b in zip(got[: m - 1], got[1:m]):
                    assert v[a] > v[b] or (v[a] == v[b] and a < b)


def test_topk_distinct_matches_library_sort():
    g = torch.Generator().manual_seed(5)
    x = torch.randn(64, 300, generator=g)
    for k in (1, 7, 64, 299, 300):
        ref = torch.topk(x, k, dim=-1, sorted=True).indices.numpy()
        got = np.stack([oracle.topk_row(r, 300, k) for r in x.numpy()])
        assert np.array_equal(got, ref)


def test_all_equal_rows_pick_first_positions():
    L, k = 20, 7
    for w_sign in (1.0, -1.0):
        scores = np.full((1, L, L), 0.0, np.float32) * w_sign
        idx = oracle.topk(scores, k, 0)
        for t in range(L):
            m = min(k, t + 1)
            assert idx[0, t, :m].tolist() == list(range(m))
            assert (idx[0, t, m:] == -1).all()


def test_signed_zero_counts_as_zero():
    row = np.array([-0.0, 0.0, -0.0, 0.0], np.float32)
    assert oracle.topk_row(row, 4, 3).tolist() == [0, 1, 2]
    row = np.array([0.0, -0.0, 1.0, -1.0], np.float32)
    assert oracle.topk_row(row, 4, 4).tolist() == [2, 0, 1, 3]


def test_topk_reads_only_causal_prefix():
    rng = np.random.default_rng(2)
    s = rng.standard_normal((2, 6, 10)).astype(np.float32)
    a = oracle.topk(s, 4, q_pos0=3)
    s2 = s.copy()
    for i in range(6):
        s2[:, i, 3 + i + 1:] = 1e30  # anything beyond t must be ignored
    b = oracle.topk(s2, 4, q_pos0=3)
    assert np.array_equal(a, b)
    assert (a >= -1).all()
    for i in range(6):
        assert (a[:, i] <= 3 + i).all()


def test_short_rows_return_all_positions():
    rng = np.random.default_rng(4)
    s = rng.standard_normal((1, 5, 5)).astype(np.float32)
    idx = oracle.topk(s, 16, 0)
    for t in range(5):
        assert sorted(idx[0, t, : t + 1].tolist()) == list(range(t + 1))
        assert (idx[0, t, t + 1:] == -1).all()


def test_position_order_keeps_the_set_and_sorts_positions():
    ix = np.array([[5, 2, 9, -1], [3, -1, -1, -1], [7, 0, 1, 4]])
    want = np.array([[2, 5, 9, -1], [3, -1, -1, -1], [0, 1, 4, 7]])
    assert np.array_equal(oracle.position_order(ix), want)
    rng = np.random.default_rng(3)
    sc = rng.standard_normal((1, 40, 40))
    top = oracle.topk(sc, 8, 0)
    po = oracle.position_order(top)
    for a, b in zip(top[0], po[0]):
        v = b[b >= 0]
        assert set(a[a >= 0]) == set(v) and np.all(np.diff(v) > 0)
        assert np.all(b[len(v):] == -1)


def test_ragged_positions_equal_per_sequence_runs():
    # a decode batch of sequences with their own lengths, keys padded to the
    # longest: each row equals the uniform path run on its own sequence alone
    rng = np.random.default_rng(5)
    lens = [5, 9, 12, 1]
    B, Lk, H_I, d_I, k = len(lens), max(lens), 3, 4, 6
    q = rng.integers(-4, 5, size=(B, 1, H_I, d_I)).astype(np.float64)
    kk = rng.integers(-4, 5, size=(B, Lk, d_I)).astype(np.float64)
    w = rng.choice([0.25, 0.5, 1.0], size=(B, 1, H_I))
    q_pos = np.array([[n - 1] for n in lens])
    sc = oracle.indexer_scores(q, kk, w, 0, q_pos=q_pos)
    got = oracle.topk(sc, k, 0, q_pos=q_pos)
    for b, n in enumerate(lens):
        one = oracle.indexer_scores(q[b:b + 1], kk[b:b + 1, :n], w[b:b + 1], n - 1)
        assert np.array_equal(sc[b, 0, :n], one[0, 0])
        assert np.all(np.isneginf(sc[b, 0, n:]))
        assert np.array_equal(got[b], oracle.topk(one, k, n - 1)[0])
    # per-row positions q_pos0 + i reproduce the uniform chunk
    q2 = rng.integers(-4, 5, size=(1, 4, H_I, d_I)).astype(np.float64)
    w2 = rng.choice([0.25, 0.5, 1.0], size=(1, 4, H_I))
    kk2 = kk[2:3]
    uni = oracle.indexer_scores(q2, kk2, w2, 7)
    rag = oracle.indexer_scores(q2, kk2, w2, 0, q_pos=np.arange(7, 11).reshape(1, 4))
    assert np.array_equal(uni, rag)
    # a negative position selects nothing; one past the keys reads as the last key
    neg = oracle.topk(oracle.indexer_scores(q2, kk2, w2, 0, q_pos=np.full((1, 4), -1)), k, 0,
                      q_pos=np.full((1, 4), -1))
    assert np.all(neg == oracle.PAD)
    far = oracle.indexer_scores(q2, kk2, w2, 0, q_pos=np.full((1, 4), 10 ** 6))
    last = oracle.indexer_scores(q2, kk2, w2, 0, q_pos=np.full((1, 4), Lk - 1))
    assert np.array_equal(far, last)
