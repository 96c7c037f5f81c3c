"""Pins for the oracle's lightning-indexer scores.

Pinned to: the one-head/unit-weight special case (a textbook causally masked
GEMM followed by ReLU), the closed form ReLU(x) + ReLU(-x) = |x|, linearity
and antisymmetry in the head weights, the sign placement of ReLU under
negative weights, one-hot queries (exact key entries), causality, chunked ==
unchunked rows, batch independence and integer exactness.
"""
import numpy as np
import pytest
import torch

import idxc_inputs
import oracle


def _rand_int(rng, shape, lo=-4, hi=4):
    return rng.integers(lo, hi + 1, shape).astype(np.float64)


def test_single_head_unit_weight_is_masked_relu_gemm():
    rng = np.random.default_rng(0)
    B, L, d = 2, 33, 8
    q = rng.standard_normal((B, L, 1, d))
    k = rng.standard_normal((B, L, d))
    w = np.ones((B, L, 1))
    got = oracle.indexer_scores(q, k, w, 0)
    qt = torch.from_numpy(q[:, :, 0, :])
    kt = torch.from_numpy(k)
    full = torch.relu(qt @ kt.transpose(1, 2))               # [B, L, L]
    mask = torch.tril(torch.ones(L, L, dtype=torch.bool))
    ref = torch.where(mask, full, torch.tensor(-float("inf"), dtype=torch.float64))
    ref = ref.to(torch.float32).numpy()
    assert np.array_equal(got, ref)


def test_relu_pair_gives_abs():
    rng = np.random.default_rng(1)
    B, L, d = 1, 17, 6
    q0 = _rand_int(rng, (B, L, 1, d))
    q = np.concatenate([q0, -q0], axis=2)
    k = _rand_int(rng, (B, L, d))
    for a in (1.0, 0.5, -0.25):
        w = np.full((B, L, 2), a)
        got = oracle.indexer_scores(q, k, w, 0)
        dots = np.einsum("bid,bsd->bis", q0[:, :, 0, :], k)
        for t in range(L):
            assert np.array_equal(got[0, t, : t + 1],
                                  (a * np.abs(dots[0, t, : t + 1])).astype(np.float32))


def test_linear_and_antisymmetric_in_weights():
    rng = np.random.default_rng(2)
    B, L, H, d = 1, 20, 3, 5
    q = _rand_int(rng, (B, L, H, d))
    k = _rand_int(rng, (B, L, d))
    w1 = rng.choice([0.25, 0.5, 1.0, -0.5], (B, L, H))
    w2 = rng.choice([0.25, 0.5, 1.0, -1.0], (B, L, H))
    s1 = oracle.indexer_scores(q, k, w1, 0)
    s2 = oracle.indexer_scores(q, k, w2, 0)
    s12 = oracle.indexer_scores(q, k, w1 + w2, 0)
    tri = np.tril(np.ones((L, L), bool))[None]
    assert np.array_equal((s1 + s2)[tri], s12[tri])
    sneg = oracle.indexer_scores(q, k, -w1, 0)
    assert np.array_equal(sneg[tri], -s1[tri])


def test_negative_weight_keeps_relu_inside():
    # w = -1, one head: score = -max(0, x) <= 0 (not max(0, -x) >= 0)
    rng = np.random.default_rng(3)
    q = _rand_int(rng, (1, 9, 1, 4))
    k = _rand_int(rng, (1, 9, 4))
    s = oracle.indexer_scores(q, k, -np.ones((1, 9, 1)), 0)
    dots = np.einsum("bid,bsd->bis", q[:, :, 0, :], k)
    for t in range(9):
        assert np.array_equal(s[0, t, : t + 1],
                              (-np.maximum(dots[0, t, : t + 1], 0)).astype(np.float32) + 0.0)
        assert (s[0, t, : t + 1] <= 0).all()
        row = s[0, t, : t + 1]
        assert not np.signbit(row[row == 0]).any()  # -0.0 is reported as +0.0


def test_one_hot_query_reads_exact_key_entry():
    rng = np.random.default_rng(4)
    L, d = 11, 7
    k = rng.standard_normal((1, L, d))
    for j in range(d):
        q = np.zeros((1, L, 1, d))
        q[..., j] = 1.0
        s = oracle.indexer_scores(q, k, np.full((1, L, 1), 0.5), 0)
        for t in range(L):
            assert np.array_equal(s[0, t, : t + 1],
                                  (0.5 * np.maximum(k[0, : t + 1, j], 0)).astype(np.float32))


def test_causal_mask_and_future_keys_ignored():
    rng = np.random.default_rng(5)
    B, L, H, d = 1, 15, 2, 4
    q = rng.standard_normal((B, L, H, d))
    k = rng.standard_normal((B, L, d))
    w = rng.standard_normal((B, L, H))
    s = oracle.indexer_scores(q, k, w, 0)
    assert np.isneginf(s[0][~np.tril(np.ones((L, L), bool))]).all()
    assert np.isfinite(s[0][np.tril(np.ones((L, L), bool))]).all()
    t = 6
    k2 = k.copy()
    k2[:, t + 1:] = 123.0
    s2 = oracle.indexer_scores(q, k2, w, 0)
    assert np.array_equal(s[0, t], s2[0, t])


def test_chunked_rows_equal_unchunked():
    rng = np.random.default_rng(6)
    B, L, H, d = 2, 24, 3, 4
    q = rng.standard_normal((B, L, H, d))
    k = rng.standard_normal((B, L, d))
    w = rng.standard_normal((B, L, H))
    full = oracle.indexer_scores(q, k, w, 0)
    for p0, n in ((0, 8), (8, 8), (16, 8), (23, 1)):
        part = oracle.indexer_scores(q[:, p0:p0 + n], k[:, : p0 + n], w[:, p0:p0 + n], p0)
        assert np.array_equal(part, full[:, p0:p0 + n, : p0 + n])
    # decode row (one query at the last position) == last prefill row
    dec = oracle.indexer_scores(q[:, L - 1:], k, w[:, L - 1:], L - 1)
    assert np.array_equal(dec[:, 0], full[:, L - 1])


def test_batches_are_independent():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((2, 6, 2, 3))
    k = rng.standard_normal((2, 6, 3))
    w = rng.standard_normal((2, 6, 2))
    s = oracle.indexer_scores(q, k, w, 0)
    sw = oracle.indexer_scores(q[::-1], k[::-1], w[::-1], 0)
    assert np.array_equal(s[::-1], sw)


def test_integer_inputs_give_exact_quarter_multiples():
    q, k, w = idxc_inputs.indexer_inputs(1, 64, 64, 4, 32, kind="int", seed=0,
                                         w_kind="quarter")
    s = oracle.indexer_scores(idxc_inputs.to_f64(q), idxc_inputs.to_f64(k),
                              idxc_inputs.to_f64(w), 0)
    tri = np.tril(np.ones((64, 64), bool))
    v = s[0][tri].astype(np.float64)
    assert np.array_equal(v * 4, np.round(v * 4))
    assert np.abs(v).max() <= 4 * 16 * 32          # |w|<=1, |dot|<=16*32, 4 heads
    assert (v >= 0).all()                          # w > 0 and ReLU
    assert not np.signbit(s[0][tri]).any()         # no -0.0
