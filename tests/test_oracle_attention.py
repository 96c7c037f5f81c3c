"""Pins for the oracle's gathered sparse attention.

Pinned to: dense causal MQA when every earlier position is selected (torch's
scaled_dot_product_attention on CPU in fp64 with K/V repeated over heads), the
exact copy of one V row for one selected key, the two-key logistic closed form,
uniform weights for a zero query, permutation invariance and -1 padding.
"""
import numpy as np
import torch

import idxc_inputs
import oracle


def _inputs(B, L, H, D, seed):
    Q, K, V = idxc_inputs.attn_inputs(B, L, L, H, D, seed=seed)
    return idxc_inputs.to_f64(Q), idxc_inputs.to_f64(K), idxc_inputs.to_f64(V)


def test_all_positions_selected_is_dense_causal_mqa():
    B, L, H, D = 2, 40, 4, 16
    Q, K, V = _inputs(B, L, H, D, 0)
    k = 64  # >= L: every s <= t selected
    idx = np.full((B, L, k), -1, np.int32)
    for t in range(L):
        idx[:, t, : t + 1] = np.arange(t + 1)[::-1]  # any order
    got = oracle.sparse_attention(Q, K, V, idx, D ** -0.5)
    q = torch.from_numpy(Q).permute(0, 2, 1, 3)                      # [B,H,L,D]
    kk = torch.from_numpy(K)[:, None].expand(B, H, L, D)
    vv = torch.from_numpy(V)[:, None].expand(B, H, L, D)
    ref = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, is_causal=True,
                                                           scale=D ** -0.5)
    ref = ref.permute(0, 2, 1, 3).numpy()
    assert np.abs(got - ref).max() < 1e-6


def test_single_key_copies_v_row():
    B, L, H, D = 1, 30, 3, 8
    Q, K, V = _inputs(B, L, H, D, 1)
    rng = np.random.default_rng(0)
    idx = np.full((B, L, 4), -1, np.int32)
    for t in range(L):
        idx[0, t, 0] = rng.integers(0, t + 1)
    got = oracle.sparse_attention(Q, K, V, idx, D ** -0.5)
    for t in range(L):
        for h in range(H):
            assert np.array_equal(got[0, t, h], V[0, idx[0, t, 0]].astype(np.float32))


def test_two_keys_logistic_closed_form():
    B, L, H, D = 1, 12, 2, 8
    Q, K, V = _inputs(B, L, H, D, 2)
    idx = np.full((B, L, 2), -1, np.int32)
    idx[0, 1:, 0] = 0
    idx[0, 1:, 1] = 1
    idx[0, 0, 0] = 0
    sc = 0.3
    got = oracle.sparse_attention(Q, K, V, idx, sc)
    for t in range(1, L):
        for h in range(H):
            za = sc * Q[0, t, h] @ K[0, 0]
            zb = sc * Q[0, t, h] @ K[0, 1]
            pa = 1.0 / (1.0 + np.exp(zb - za))
            ref = pa * V[0, 0] + (1 - pa) * V[0, 1]
            assert np.abs(got[0, t, h] - ref).max() < 1e-6


def test_zero_query_gives_mean_of_selected_rows():
    B, L, H, D = 1, 20, 2, 8
    Q, K, V = _inputs(B, L, H, D, 3)
    Q[:] = 0.0
    idx = idxc_inputs.index_sets(B, L, 0, 6, seed=1).numpy()
    got = oracle.sparse_attention(Q, K, V, idx, D ** -0.5)
    for t in range(L):
        sel = idx[0, t][idx[0, t] >= 0]
        assert np.abs(got[0, t] - V[0, sel].mean(axis=0)).max() < 1e-6


def test_permutation_and_padding_invariance():
    B, L, H, D = 2, 25, 4, 16
    Q, K, V = _inputs(B, L, H, D, 4)
    idx = idxc_inputs.index_sets(B, L, 0, 8, seed=2).numpy()
    base = oracle.sparse_attention(Q, K, V, idx, D ** -0.5)
    rng = np.random.default_rng(1)
    perm = idx.copy()
    for b in range(B):
        for t in range(L):
            n = int((perm[b, t] >= 0).sum())
            perm[b, t, :n] = rng.permutation(perm[b, t, :n])
    assert np.abs(oracle.sparse_attention(Q, K, V, perm, D ** -0.5) - base).max() < 1e-6
    padded = np.concatenate([idx, np.full((B, L, 5), -1, np.int32)], axis=2)
    assert np.array_equal(oracle.sparse_attention(Q, K, V, padded, D ** -0.5), base)
