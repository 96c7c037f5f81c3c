"""GPU test of idxc_layer_stack_forward_noalloc (the stack entry point whose
scratch is the library's static per-GPU array instead of a caller workspace):
on successive calls with shrinking inputs, which reuse the one array, its
indices, outputs and indexer-call counts equal those of
idxc_layer_stack_forward with a caller workspace, and on the integer-input
tiny stack they equal the oracle's (indices bit-exact, attention within
2e-2)."""
import sys

import numpy as np
import pytest
import torch

import idxc_inputs as gen
import oracle
import dsa_lightning_indexer_score_amd as idxc

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _layers(cfg, device="cuda"):
    out = []
    for l in range(cfg.n_layers):
        L = {n: t.to(device) for n, t in gen.layer_inputs(cfg, l).items()}
        if cfg.pattern[l] == "S":  # never read on S layers
            L["q_idx"] = L["k_idx"] = L["w"] = None
        out.append(L)
    return out


def _both(cfg, layers):
    ref = idxc.idxc_layer_stack_forward(cfg.pattern, layers, cfg.k, cfg.scale,
                                        q_pos0=cfg.q_pos0, debug_indices=True)
    got = idxc.idxc_layer_stack_forward_noalloc(cfg.pattern, layers, cfg.k, cfg.scale,
                                                q_pos0=cfg.q_pos0, debug_indices=True)
    torch.cuda.synchronize()
    assert got["indexer_calls"] == ref["indexer_calls"] == cfg.pattern.count("F")
    assert torch.equal(got["debug_indices"], ref["debug_indices"])
    assert torch.equal(got["index_cache"], ref["index_cache"])
    for l in range(cfg.n_layers):
        assert torch.equal(got["out"][l], ref["out"][l]), "layer %d output differs" % l
    return got


def test_noalloc_matches_workspace_entry_point_on_successive_calls():
    assert torch.cuda.is_available()
    # 1: a decode batch (few rows, per-chunk top-k segments, split attention)
    dec = gen.StackConfig("noalloc-decode-B16-Lk40000", 4, "FSFS", 16, 1, 40000, 39999,
                          64, 128, 64, 128, 2048, "normal")
    _say("noalloc call 1: %s" % dec.name)
    _both(dec, _layers(dec))
    # 2: a smaller prefill (candidate lists, one pass per row)
    pre = gen.StackConfig("noalloc-prefill-L2000", 3, "FSF", 1, 2000, 2000, 0, 64, 128,
                          64, 128, 512, "normal")
    _say("noalloc call 2: %s" % pre.name)
    _both(pre, _layers(pre))
    # 3: the tiny integer stack, also against the oracle
    cfg = gen.C1
    _say("noalloc call 3: %s" % cfg.name)
    layers = _layers(cfg)
    got = _both(cfg, layers)
    host = [{n: gen.to_f64(t) for n, t in gen.layer_inputs(cfg, l).items()}
            for l in range(cfg.n_layers)]
    ref = oracle.layer_stack(cfg.pattern, host, cfg.k, cfg.scale, cfg.q_pos0)
    assert got["indexer_calls"] == ref["calls"] == 2
    dbg = got["debug_indices"].cpu().numpy()
    for l in range(cfg.n_layers):
        assert np.array_equal(dbg[l], oracle.position_order(ref["indices"][l])), l
        err = float(np.abs(got["out"][l].float().cpu().numpy() - ref["out"][l]).max())
        assert err <= 2e-2, (l, err)
    _say("noalloc: three successive calls equal the workspace entry point")
