"""Benchmark of the IndexCache hot path on one MI355X.

A step is one pass of the whole hot path over a 47-layer stack: on every F
layer the fused lightning indexer + top-k refreshes the index cache, on every
layer the gathered sparse attention reads it (one idxc_layer_stack_forward
call). The headline line is the 47-layer prefill at L = 32768 with the 12-F
pattern (F at layers 0, 4, ..., 44, i.e. 1/4 of the indexers kept); the same
stack with all 47 layers F, and the 47-layer decode step (64 sequences x 65536
cached tokens, one new query each) with both patterns, are reported next to
it. Inputs are seeded synthetic bf16 tensors resident in HBM before timing.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--skip-cpu]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill & decode tokens/s, 47-layer DSA stack, 1/4-F vs all-F; MFMA %"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
N_SETS = 7                  # distinct per-layer input sets, cycled over the 47 layers


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--only", default="", help="prefill-12f | prefill-allf | decode (profiling)")
    return ap.parse_args()


# --------------------------------------------------------------------------- #
# inputs
# --------------------------------------------------------------------------- #
def build_stack(cfg, n_sets, device="cuda"):
    """Per-layer dicts cycling over n_sets distinct seeded input sets (each set
    is far larger than the 256 MB last-level cache, so HBM traffic per layer is
    that of distinct layers)."""
    import torch
    import idxc_inputs as gen
    sets = []
    for s in range(n_sets):
        L = gen.layer_inputs(cfg, s, device=device)
        L["out"] = torch.empty_like(L["q"])
        sets.append(L)
    torch.cuda.synchronize()
    return [sets[l % n_sets] for l in range(cfg.n_layers)], sets


def time_steps(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def event_ms(fn, reps):
    """Average device time of fn() on torch's current stream (HIP events)."""
    import torch
    st = torch.cuda.current_stream()
    fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(st)
    for _ in range(reps):
        fn()
    b.record(st)
    b.synchronize()
    return a.elapsed_time(b) / reps


# --------------------------------------------------------------------------- #
# algorithmic work (per launch)
# --------------------------------------------------------------------------- #
def causal_pairs(q_pos0, Lq):
    # sum over t = q_pos0 .. q_pos0+Lq-1 of (t+1)
    return Lq * (2 * q_pos0 + Lq + 1) // 2


def selected_pairs(q_pos0, Lq, k):
    tot = 0
    for t in range(q_pos0, q_pos0 + Lq):
        tot += min(k, t + 1)
    return tot


def indexer_flops(cfg):
    return cfg.B * causal_pairs(cfg.q_pos0, cfg.Lq) * 2 * cfg.H_I * cfg.d_I


def indexer_bytes(cfg):
    rows = cfg.B * cfg.Lq
    return (rows * cfg.H_I * cfg.d_I * 2 + cfg.B * cfg.Lk * cfg.d_I * 2 + rows * cfg.H_I * 2
            + rows * cfg.k * 4)


def attn_bytes(cfg):
    rows = cfg.B * cfg.Lq
    sel = cfg.B * selected_pairs(cfg.q_pos0, cfg.Lq, cfg.k)
    return sel * 2 * cfg.D * 2 + rows * cfg.H * cfg.D * 2 * 2 + rows * cfg.k * 4


def attn_flops(cfg):
    return cfg.B * selected_pairs(cfg.q_pos0, cfg.Lq, cfg.k) * 4 * cfg.H * cfg.D


# --------------------------------------------------------------------------- #
# CPU oracle baseline on a bounded sample
# --------------------------------------------------------------------------- #
def cpu_baseline(cfg, n_rows=2048):
    """Time the oracle (as it stands) on n_rows query rows of one F layer and
    one S layer of the prefill stack, then compose the 47-layer stack time."""
    import numpy as np
    import torch
    import idxc_inputs as gen
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    L = gen.layer_inputs(cfg, 0, device="cpu")
    rows = np.unique(np.linspace(0, cfg.Lq - 1, n_rows).astype(int))
    k_idx = gen.to_f64(L["k_idx"])
    Kf, Vf = gen.to_f64(L["k"]), gen.to_f64(L["v"])
    t_f = t_s = 0.0
    for i in rows:
        q_idx = gen.to_f64(L["q_idx"][:, i:i + 1])
        w = gen.to_f64(L["w"][:, i:i + 1])
        Q = gen.to_f64(L["q"][:, i:i + 1])
        t0 = time.perf_counter()
        sc = oracle.indexer_scores(q_idx, k_idx, w, cfg.q_pos0 + int(i), cfg.Lk)
        idx = oracle.topk(sc, cfg.k, cfg.q_pos0 + int(i))
        t1 = time.perf_counter()
        oracle.sparse_attention(Q, Kf, Vf, idx, cfg.scale)
        t2 = time.perf_counter()
        t_f += t1 - t0
        t_s += t2 - t1
    # rows are spread uniformly over positions, so the mean per-row time times
    # Lq estimates one layer
    per_row_idx = t_f / len(rows)
    per_row_att = t_s / len(rows)
    nF = cfg.pattern.count("F")
    stack_s = cfg.B * cfg.Lq * (nF * per_row_idx + cfg.n_layers * per_row_att)
    return dict(value=cfg.B * cfg.Lq / stack_s, unit="tokens/s", cores=int(cores), kind="oracle",
                sample="%d query rows (evenly spaced over positions 0..%d) of one F layer "
                       "(indexer+top-k+attention) and attention of one S layer of %s; "
                       "per-row times composed to the 47-layer stack (%d F, %d layers); "
                       "measured %.1f s" % (len(rows), cfg.Lq - 1, cfg.name, nF, cfg.n_layers,
                                           t_f + t_s),
                composed_stack_seconds=stack_s)


# --------------------------------------------------------------------------- #
def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(decode shards by sequence and prefill by query rows with no collective "
              "inside a layer; see the design notes). Re-run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import idxc_inputs as gen
    import dsa_lightning_indexer_score_amd as idxc
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    log("library %s on %s" % (idxc.idxc_version(), torch.cuda.get_device_name(0)))

    res = {}
    extra = {}
    # ----------------------------------------------------------------- prefill
    cfg12, cfgF = gen.C3_12F, gen.C3_ALLF
    t0 = time.perf_counter()
    layers, sets = build_stack(cfg12, N_SETS)
    log("prefill inputs ready (%d sets, %.1f s)" % (N_SETS, time.perf_counter() - t0))
    ws = torch.empty(idxc.idxc_workspace_bytes(cfg12.B, cfg12.Lq, cfg12.Lk, cfg12.q_pos0,
                                               cfg12.H_I, cfg12.d_I, cfg12.k, cfg12.H, cfg12.D),
                     dtype=torch.uint8, device="cuda")
    cache = torch.empty((cfg12.B, cfg12.Lq, cfg12.k), dtype=torch.int32, device="cuda")
    call12 = idxc.StackCall(cfg12.pattern, layers, cfg12.k, cfg12.scale, cfg12.q_pos0,
                            index_cache=cache, workspace=ws)
    callF = idxc.StackCall(cfgF.pattern, layers, cfgF.k, cfgF.scale, cfgF.q_pos0,
                           index_cache=cache, workspace=ws)
    if args.only in ("", "prefill-12f"):
        s12 = time_steps(call12, args.steps, args.warmup)
        assert call12.calls.value == 12
        log("prefill 12-F: %.2f ms/step" % (s12 * 1e3))
        res["prefill_12F"] = s12
    if args.only in ("", "prefill-allf"):
        sF = time_steps(callF, args.steps, args.warmup)
        assert callF.calls.value == 47
        log("prefill all-F: %.2f ms/step" % (sF * 1e3))
        res["prefill_allF"] = sF
    # per-layer breakdown with HIP events on the launch stream
    L0 = sets[0]
    idx_ms = event_ms(lambda: idxc.idxc_indexer_topk(L0["q_idx"], L0["k_idx"], L0["w"], cfg12.k,
                                                     workspace=ws, out=cache), 3)
    att_ms = event_ms(lambda: idxc.idxc_sparse_attn(L0["q"], L0["k"], L0["v"], cache,
                                                    cfg12.scale, out=L0["out"]), 3)
    log("prefill per layer: indexer+top-k %.3f ms, attention %.3f ms" % (idx_ms, att_ms))
    del layers, sets, call12, callF, ws, cache, L0
    torch.cuda.empty_cache()

    # ------------------------------------------------------------------ decode
    dec = {}
    if not args.skip_decode and args.only in ("", "decode"):
        d12, dF = gen.C4_12F, gen.C4_ALLF
        t0 = time.perf_counter()
        dlayers, dsets = build_stack(d12, N_SETS)
        log("decode inputs ready (%.1f s)" % (time.perf_counter() - t0))
        dws = torch.empty(idxc.idxc_workspace_bytes(d12.B, d12.Lq, d12.Lk, d12.q_pos0, d12.H_I,
                                                    d12.d_I, d12.k, d12.H, d12.D),
                          dtype=torch.uint8, device="cuda")
        dcache = torch.empty((d12.B, d12.Lq, d12.k), dtype=torch.int32, device="cuda")
        dc12 = idxc.StackCall(d12.pattern, dlayers, d12.k, d12.scale, d12.q_pos0,
                              index_cache=dcache, workspace=dws)
        dcF = idxc.StackCall(dF.pattern, dlayers, dF.k, dF.scale, dF.q_pos0,
                             index_cache=dcache, workspace=dws)
        dec["decode_12F"] = time_steps(dc12, args.decode_steps, args.warmup)
        dec["decode_allF"] = time_steps(dcF, args.decode_steps, args.warmup)
        D0 = dsets[0]
        dec_idx_ms = event_ms(lambda: idxc.idxc_indexer_topk(
            D0["q_idx"], D0["k_idx"], D0["w"], d12.k, q_pos0=d12.q_pos0, workspace=dws,
            out=dcache), 10)
        dec_att_ms = event_ms(lambda: idxc.idxc_sparse_attn(D0["q"], D0["k"], D0["v"], dcache,
                                                            d12.scale, out=D0["out"]), 10)
        log("decode: 12-F %.3f ms/step, all-F %.3f ms/step; per layer indexer+top-k %.3f ms, "
            "attention %.3f ms" % (dec["decode_12F"] * 1e3, dec["decode_allF"] * 1e3,
                                   dec_idx_ms, dec_att_ms))
        extra["decode_per_layer_ms"] = {"indexer_topk": dec_idx_ms, "attention": dec_att_ms}
        extra["decode_indexer_hbm_gbs"] = indexer_bytes(d12) / (dec_idx_ms * 1e-3) / 1e9
        extra["decode_attention_gbs"] = attn_bytes(d12) / (dec_att_ms * 1e-3) / 1e9
        del dlayers, dsets, dc12, dcF, dws, dcache, D0
        torch.cuda.empty_cache()

    # ------------------------------------------------------------------ report
    cfg = cfg12
    s12 = res.get("prefill_12F")
    sF = res.get("prefill_allF")
    value = cfg.B * cfg.Lq / s12 if s12 else None
    idx_tflops = indexer_flops(cfg) / (idx_ms * 1e-3) / 1e12
    att_gbs = attn_bytes(cfg) / (att_ms * 1e-3) / 1e9
    nF = cfg.pattern.count("F")
    # dominant kernel of the headline workload by total time per step
    idx_total, att_total = nF * idx_ms, cfg.n_layers * att_ms
    roof_idx = {"kernel": "indexer_rows_kernel + topk_rows_kernel (fused indexer + top-k of one F "
                          "layer, idxc_indexer_topk)",
                "bound": "mfma", "achieved": idx_tflops, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": idx_tflops / PEAK_BF16_TFLOPS, "traffic": None,
                "algorithmic": "%.4g flop per launch = causal pairs %d x 2*H_I*d_I"
                               % (indexer_flops(cfg), causal_pairs(cfg.q_pos0, cfg.Lq)),
                "launch_ms": idx_ms}
    roof_att = {"kernel": "sparse_attn_kernel (one layer, idxc_sparse_attn)",
                "bound": "hbm", "achieved": att_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": att_gbs / PEAK_HBM_GBS, "traffic": None,
                "algorithmic": "%.4g B per launch = selected pairs x 2*D*2 (K+V rows) + Q + O "
                               "+ indices" % attn_bytes(cfg),
                "launch_ms": att_ms}
    dominant, other = (roof_idx, roof_att) if idx_total >= att_total else (roof_att, roof_idx)
    extra.update({
        "prefill_allF_tokens_per_s": cfg.B * cfg.Lq / sF if sF else None,
        "prefill_allF_ms_per_step": sF * 1e3 if sF else None,
        "prefill_speedup_12F_vs_allF": (sF / s12) if (sF and s12) else None,
        "prefill_per_layer_ms": {"indexer_topk": idx_ms, "attention": att_ms},
        "indexer_mfma_frac": idx_tflops / PEAK_BF16_TFLOPS,
        "other_roofline": other,
    })
    if dec:
        extra.update({
            "decode_12F_tokens_per_s": gen.C4_12F.B / dec["decode_12F"],
            "decode_allF_tokens_per_s": gen.C4_ALLF.B / dec["decode_allF"],
            "decode_speedup_12F_vs_allF": dec["decode_allF"] / dec["decode_12F"],
            "decode_12F_ms_per_step": dec["decode_12F"] * 1e3,
            "decode_allF_ms_per_step": dec["decode_allF"] * 1e3,
        })
    cpu = None
    if not args.skip_cpu:
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(cfg)
        log("cpu oracle: %.3g tokens/s on %d threads" % (cpu["value"], cpu["cores"]))
    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": s12 * 1e3 if s12 else None, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "layers": cfg.n_layers, "pattern": "12F (F at l%4==0)",
                   "B": cfg.B, "L": cfg.Lq, "H_I": cfg.H_I, "d_I": cfg.d_I, "k": cfg.k,
                   "H": cfg.H, "D": cfg.D, "input_sets": N_SETS},
        "roofline": dominant,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
