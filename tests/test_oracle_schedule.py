"""Pins for the oracle's pattern validation, nearest-F rule and index-cache loop.

Pinned to: the pages' FSSF, k=2 worked example (tests/golden), the f(l)
equation checked by brute force over every pattern up to 10 layers, the
indexer-call count and the error cases of the state machine.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_fssf_worked_example(golden_dir):
    g = _golden(golden_dir, "fssf_worked_example.json")
    # The page's example has one query row of 4 scores per layer, every
    # position a candidate: treat it as B=1, Lq=1, query position t=3.
    scores = [np.asarray(s, dtype=np.float32)[None] for s in g["layer_scores"]]
    sel, calls = oracle.schedule(scores, g["pattern"], g["k"], q_pos0=3)
    assert calls == g["expected_calls"]
    assert np.array_equal(sel[1], sel[0])
    assert np.array_equal(sel[2], sel[0])
    assert not np.array_equal(sel[3], sel[0])
    for l in range(4):
        assert sel[l][0].tolist() == g["expected_selected"][l]
    # layer 2's own top-2 differs from the reused one: reuse is observable
    own2 = oracle.topk(scores[2], g["k"], q_pos0=3)
    assert own2[0].tolist() == g["own_topk_layer2"]
    assert not np.array_equal(own2, sel[2])


@pytest.mark.parametrize("bad,n", [("SFSF", 4), ("FSS", 4), ("FSXF", 4), ("", 0),
                                   ("fssf", 4), ("F1SF", 4), ("FSSFS", 4)])
def test_pattern_errors(bad, n):
    with pytest.raises(ValueError):
        oracle.validate_pattern(bad, n)


def test_schedule_errors():
    sc = [np.zeros((1, 1, 4), np.float32)] * 3
    with pytest.raises(ValueError):
        oracle.schedule(sc, "SFF", 2, q_pos0=3)
    with pytest.raises(ValueError):
        oracle.schedule(sc, "FF", 2, q_pos0=3)
    with pytest.raises(ValueError):
        oracle.schedule(sc, "FQF", 2, q_pos0=3)


def _brute_source(pattern, l):
    """f(l) by scanning backwards from l (F layers map to themselves)."""
    j = l
    while pattern[j] != "F":
        j -= 1
    return j


def test_nearest_full_brute_force_all_patterns():
    rng = np.random.default_rng(7)
    for n in range(1, 11):
        for tail in itertools.product("FS", repeat=n - 1):
            pat = "F" + "".join(tail)
            src = oracle.nearest_full(pat)
            assert src == [_brute_source(pat, l) for l in range(n)]
            # f(l) < l for S layers and c_{f(l)} = F, nothing F in between
            for l, c in enumerate(pat):
                if c == "S":
                    assert src[l] < l and pat[src[l]] == "F"
                    assert all(pat[j] == "S" for j in range(src[l] + 1, l))
        # the cache loop: S layers carry the source layer's own top-k, calls = #F
        for tail in itertools.product("FS", repeat=n - 1):
            pat = "F" + "".join(tail)
            scores = [rng.standard_normal((1, 3, 6)).astype(np.float32)
                      for _ in range(n)]
            sel, calls = oracle.schedule(scores, pat, 2, q_pos0=3)
            assert calls == pat.count("F")
            for l in range(n):
                want = oracle.topk(scores[_brute_source(pat, l)], 2, q_pos0=3)
                assert np.array_equal(sel[l], want)


def test_layer_stack_calls_and_reuse():
    rng = np.random.default_rng(3)
    B, L, H_I, d_I, H, D, k = 1, 12, 2, 4, 2, 8, 3
    layers = []
    for _ in range(5):
        layers.append(dict(q_idx=rng.integers(-2, 3, (B, L, H_I, d_I)).astype(float),
                           k_idx=rng.integers(-2, 3, (B, L, d_I)).astype(float),
                           w=np.ones((B, L, H_I)),
                           q=rng.standard_normal((B, L, H, D)),
                           k=rng.standard_normal((B, L, D)),
                           v=rng.standard_normal((B, L, D))))
    res = oracle.layer_stack("FSFSS", layers, k, D ** -0.5, 0)
    assert res["calls"] == 2
    assert np.array_equal(res["indices"][1], res["indices"][0])
    assert np.array_equal(res["indices"][3], res["indices"][2])
    assert np.array_equal(res["indices"][4], res["indices"][2])
    own2 = oracle.topk(oracle.indexer_scores(layers[2]["q_idx"], layers[2]["k_idx"],
                                             layers[2]["w"], 0), k, 0)
    assert np.array_equal(res["indices"][2], own2)
    assert res["scores"][1] is None and res["scores"][2] is not None
