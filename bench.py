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
    ap.add_argument("--only", default="",
                    help="prefill-12f | prefill-allf | decode | sweep | pmc | dispatch | topk "
                         "(profiling)")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "CMD_F", "CMD_W"),
                    help="write profiles/hbm_traffic.md from the two counter passes (no GPU)")
    ap.add_argument("--dispatch-summary", nargs=2, metavar=("TRACE_CSV", "CMD"),
                    help="write profiles/dispatch_counts.md from a --only dispatch kernel trace")
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


_SLEEP_CYCLES_PER_MS = None


def gpu_head_start(ms):
    """Queue a spin kernel of about `ms` milliseconds (torch.cuda._sleep,
    calibrated once with HIP events) on the current stream."""
    global _SLEEP_CYCLES_PER_MS
    import torch
    if _SLEEP_CYCLES_PER_MS is None:
        cycles = 1 << 20
        torch.cuda._sleep(cycles)  # warm-up
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(cycles)
        b.record()
        b.synchronize()
        _SLEEP_CYCLES_PER_MS = cycles / max(a.elapsed_time(b), 1e-3)
    torch.cuda._sleep(int(min(ms, 2000.0) * _SLEEP_CYCLES_PER_MS))


def kernel_pass(cfg, layers, ws, cache, steps):
    """Run the stack layer by layer through the per-layer entry points (the
    same launches, in the same order, as one stack call) with HIP events on
    the launch stream around every F layer's indexer + top-k and every
    attention launch. Returns (mean ms of one indexer + top-k, mean ms of one
    attention launch, ms per step of the pass)."""
    import torch
    import dsa_lightning_indexer_score_amd as idxc
    st = torch.cuda.current_stream()

    def one_step(events):
        for l, L in enumerate(layers):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(st)
            if cfg.pattern[l] == "F":
                idxc.idxc_indexer_topk(L["q_idx"], L["k_idx"], L["w"], cfg.k, q_pos0=cfg.q_pos0,
                                       workspace=ws, out=cache, order="position")
            e[1].record(st)
            idxc.idxc_sparse_attn(L["q"], L["k"], L["v"], cache, cfg.scale, workspace=ws,
                                  out=L["out"])
            e[2].record(st)
            events.append((cfg.pattern[l] == "F", e))

    one_step([])
    # Keep the GPU busy while the host enqueues the timed steps: decode
    # launches are shorter than their host-side launch work, and events taken
    # while the GPU waits for the host would time the host.
    gpu_head_start(steps * 10.0 * len(layers) / 47.0)
    events = []
    for _ in range(steps):
        one_step(events)
    torch.cuda.synchronize()
    idx = [e[0].elapsed_time(e[1]) for f, e in events if f]
    att = [e[1].elapsed_time(e[2]) for f, e in events]
    total = events[0][1][0].elapsed_time(events[-1][1][2])
    return sum(idx) / len(idx), sum(att) / len(att), total / steps


def hbm_traffic(kernel):
    """Scaled HBM bytes per launch of `kernel` from the committed counter
    summary, or None when the kernel's sources changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    if not os.path.exists(path):
        return None
    rec = None
    for line in open(path):
        if line.startswith("traffic-json: "):
            rec = json.loads(line[len("traffic-json: "):]).get(kernel)
    if not rec:
        return None
    h = hashlib.sha256()
    for f in rec["sources"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest()[:16] != rec["sha"]:
        return None
    return rec["bytes"]


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
# long-context indexer + top-k (query chunks) and the standalone top-k
# --------------------------------------------------------------------------- #
def events_ms(fn, reps=1):
    """Mean device time of fn() over reps calls on torch's current stream (the
    stream the library launches on), after one untimed call, with the GPU
    kept busy while the host enqueues them."""
    import torch
    st = torch.cuda.current_stream()
    fn()
    gpu_head_start(1.0 * reps)  # the reps queue up behind it (short launches)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(st)
    for _ in range(reps):
        fn()
    b.record(st)
    b.synchronize()
    return a.elapsed_time(b) / reps


def long_context(L, chunk, H_I=64, d_I=128, k=2048, seed=0):
    """Fused indexer + top-k of one layer at L tokens, processed in query
    chunks of `chunk` rows against all preceding keys (chunk c: q_pos0 =
    c*chunk, keys [0, (c+1)*chunk)); scores never reach HBM."""
    import torch
    import idxc_inputs as gen
    import dsa_lightning_indexer_score_amd as idxc
    q, kk, w = gen.indexer_inputs(1, L, L, H_I, d_I, kind="normal", seed=seed, device="cuda")
    ws = torch.empty(idxc.idxc_workspace_bytes(1, chunk, L, L - chunk, H_I, d_I, k),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((1, chunk, k), dtype=torch.int32, device="cuda")
    n = L // chunk

    def one_pass():
        for c in range(n):
            idxc.idxc_indexer_topk(q[:, c * chunk:(c + 1) * chunk], kk[:, :(c + 1) * chunk],
                                   w[:, c * chunk:(c + 1) * chunk], k, q_pos0=c * chunk,
                                   workspace=ws, out=out)
    ms = events_ms(one_pass, 1)
    flops = causal_pairs(0, L) * 2 * H_I * d_I
    return {"L": L, "chunk": chunk, "chunks": n, "ms": ms, "tokens_per_s": L / (ms * 1e-3),
            "indexer_flops": flops, "TFLOPs": flops / (ms * 1e-3) / 1e12,
            "mfma_frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def decode_layer(lens, k=2048, H_I=64, d_I=128, H=64, D=128, seed=0, ragged=True):
    """One F decode layer (fused indexer + top-k, then sparse attention) for a
    batch of sequences with cache lengths `lens` (one new query each), keys
    padded to the longest. ragged=False times the same batch as a uniform one
    (every sequence at the longest length). Returns per-layer ms."""
    import torch
    import idxc_inputs as gen
    import dsa_lightning_indexer_score_amd as idxc
    B, Lk = len(lens), max(lens)
    q, kk, w = gen.indexer_inputs(B, 1, Lk, H_I, d_I, kind="normal", seed=seed,
                                  idx_std=d_I ** -0.5, device="cuda")
    Q, K, V = gen.attn_inputs(B, 1, Lk, H, D, seed=seed + 1, device="cuda")
    pos = torch.tensor([[n - 1] for n in lens], dtype=torch.int32, device="cuda")
    ws = torch.empty(idxc.idxc_workspace_bytes(B, 1, Lk, Lk - 1, H_I, d_I, k, H, D),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((B, 1, k), dtype=torch.int32, device="cuda")
    o = torch.empty_like(Q)
    scale = D ** -0.5

    def sel():
        if ragged:
            idxc.idxc_indexer_topk_ragged(q, kk, w, k, pos, workspace=ws, out=out,
                                          order="position")
        else:
            idxc.idxc_indexer_topk(q, kk, w, k, q_pos0=Lk - 1, workspace=ws, out=out,
                                   order="position")
    idx_ms = events_ms(sel, 10)
    att_ms = events_ms(lambda: idxc.idxc_sparse_attn(Q, K, V, out, scale, workspace=ws, out=o),
                       10)
    del q, kk, w, Q, K, V, ws
    torch.cuda.empty_cache()
    return idx_ms, att_ms


def context_sweep():
    """The pages' context grid (about 10K, 60K, 120K and 200K tokens): prefill
    indexer + top-k of one layer in query chunks, and one decode layer for 64
    sequences at that cache length, composed to the 47-layer 12-F decode step;
    then a ragged decode batch (64 lengths spread over 1K..196K) against the
    same batch padded to its longest sequence."""
    import torch
    out = {}
    for L, chunk in ((10240, 2048), (61440, 4096), (122880, 4096), (196608, 4096)):
        lc = long_context(L, chunk)
        torch.cuda.empty_cache()
        idx_ms, att_ms = decode_layer([L] * 64)
        step12 = 12 * idx_ms + 47 * att_ms
        out[str(L)] = {"prefill_indexer_topk_ms": lc["ms"],
                       "prefill_indexer_topk_tokens_per_s": lc["tokens_per_s"],
                       "prefill_indexer_TFLOPs": lc["TFLOPs"],
                       "decode_layer_indexer_topk_ms": idx_ms,
                       "decode_layer_attention_ms": att_ms,
                       "decode_12F_step_ms_composed": step12,
                       "decode_12F_tokens_per_s_composed": 64 / (step12 * 1e-3)}
        log("context %d: prefill indexer+top-k %.1f ms (%.0f TFLOP/s); decode layer %.3f + %.3f ms"
            % (L, lc["ms"], lc["TFLOPs"], idx_ms, att_ms))
    import random
    rnd = random.Random(0)
    lens = [int(1024 + (196608 - 1024) * i / 63) for i in range(64)]
    rnd.shuffle(lens)
    r_idx, r_att = decode_layer(lens, ragged=True)
    p_idx, p_att = decode_layer(lens, ragged=False)
    out["ragged_decode"] = {
        "lengths": "64 sequences, cache lengths evenly spread over 1024..196608 (mean %d)"
                   % (sum(lens) // len(lens)),
        "indexer_topk_ms": r_idx, "attention_ms": r_att,
        "padded_indexer_topk_ms": p_idx, "padded_attention_ms": p_att,
        "indexer_speedup_vs_padded": p_idx / r_idx}
    log("ragged decode: indexer+top-k %.3f ms vs %.3f ms padded to the longest"
        % (r_idx, p_idx))
    return out


def distill_rate(Lq=2048, Lk=32768, n_teachers=4, seed=0):
    """idxc_distill_loss on one query chunk (the last Lq rows of an Lk-token
    context) against n_teachers teachers (an F layer and the S layers it
    serves under the 12-F pattern); algorithmic bytes = per causal (row, key)
    pair one logit read, n_teachers teacher reads and one gradient write."""
    import torch
    import dsa_lightning_indexer_score_amd as idxc
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    q_pos0 = Lk - Lq
    logits = torch.randn((1, Lq, Lk), generator=g, device="cuda")
    teachers = torch.rand((n_teachers, 1, Lq, Lk), generator=g, device="cuda")
    teachers /= teachers.sum(-1, keepdim=True)  # synthetic distributions (full rows)
    loss = torch.empty((1, Lq), device="cuda")
    grad = torch.empty_like(logits)
    d = idxc.make_dims(1, Lq, Lk, q_pos0)
    lib = idxc._lib.load()
    import ctypes

    def call():
        idxc._lib.check(lib.idxc_distill_loss(ctypes.c_void_p(logits.data_ptr()),
                                              ctypes.c_void_p(teachers.data_ptr()), n_teachers,
                                              ctypes.byref(d), ctypes.c_void_p(loss.data_ptr()),
                                              ctypes.c_void_p(grad.data_ptr()),
                                              idxc._stream(None)))
    ms = events_ms(call, 5)
    pairs = causal_pairs(q_pos0, Lq)
    nbytes = pairs * 4 * (2 + n_teachers)
    del logits, teachers, grad
    torch.cuda.empty_cache()
    return {"Lq": Lq, "Lk": Lk, "n_teachers": n_teachers, "ms": ms,
            "algorithmic_bytes": nbytes, "GBs": nbytes / (ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}


def overlap_rate(Lq=32768, Lk=32768, k=2048, seed=0):
    """idxc_overlap on two [1, Lq, k] index tensors of one prefill layer's
    shape (row t holds k causal positions drawn from [0, t], repeats
    allowed); algorithmic bytes = both tensors read once (4 B per entry each)
    + the three per-row outputs (12 B per row)."""
    import torch
    import dsa_lightning_indexer_score_amd as idxc
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    t = (torch.arange(Lq, device="cuda") + (Lk - Lq)).view(1, Lq, 1).float()
    a = (torch.rand((1, Lq, k), generator=g, device="cuda") * (t + 1)).int()
    b = (torch.rand((1, Lq, k), generator=g, device="cuda") * (t + 1)).int()
    ms = events_ms(lambda: idxc.idxc_overlap(a, b, Lk), 5)
    nbytes = 2 * Lq * k * 4 + Lq * 12
    del a, b
    torch.cuda.empty_cache()
    return {"Lq": Lq, "Lk": Lk, "k": k, "ms": ms, "algorithmic_bytes": nbytes,
            "GBs": nbytes / (ms * 1e-3) / 1e9, "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}


def standalone_topk(B, Lq, Lk, q_pos0, k, seed=0, order="score"):
    """idxc_topk on materialised fp32 scores, in score order (sorted output)
    or position order (the index cache's order, no sort); algorithmic bytes =
    valid scores read (4 B each) + indices written (4 B each)."""
    import torch
    import dsa_lightning_indexer_score_amd as idxc
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    s = torch.randn((B, Lq, Lk), generator=g, device="cuda")
    ws_n = idxc.idxc_topk_workspace_bytes(B, Lq, Lk, q_pos0, k)
    ws = torch.empty((max(ws_n, 256),), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Lq, k), dtype=torch.int32, device="cuda")
    ms = events_ms(lambda: idxc.idxc_topk(s, k, q_pos0=q_pos0, workspace=ws, out=out,
                                          order=order), 5)
    nbytes = B * causal_pairs(q_pos0, Lq) * 4 + B * Lq * k * 4
    del s
    return {"shape": [B, Lq, Lk], "k": k, "order": order, "ms": ms,
            "GBs": nbytes / (ms * 1e-3) / 1e9,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}


# --------------------------------------------------------------------------- #
# CPU oracle baseline on bounded samples (the only leg that runs the oracle)
# --------------------------------------------------------------------------- #
def host_info():
    """Host cores, CPU model and the BLAS build numpy runs on."""
    info = {"nproc": os.cpu_count()}
    try:
        info["affinity_cpus"] = len(os.sched_getaffinity(0))
    except Exception:
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
                break
    except Exception:
        pass
    try:
        import numpy as np
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            info["blas"] = "%s %s (%s), %d threads" % (
                blas[0].get("internal_api"), blas[0].get("version"),
                blas[0].get("architecture"), int(blas[0].get("num_threads", 1)))
            info["blas_threads"] = int(blas[0].get("num_threads", 1))
        info["numpy"] = np.__version__
    except Exception:
        pass
    return info


def _oracle_row_times(q_idx, k_idx, w, Q, K, V, rows, k, scale, q_pos0, attn=True):
    """Oracle time per sampled query row (indexer + top-k, and attention), and
    the oracle's index sets of those rows. Row j of q_idx / w / Q is query
    position q_pos0 + rows[j] of keys k_idx / K / V (all fp64, batch 1)."""
    import oracle
    t_idx = t_att = 0.0
    sets = []
    for j, i in enumerate(rows):
        t = q_pos0 + int(i)
        t0 = time.perf_counter()
        sc = oracle.indexer_scores(q_idx[:, j:j + 1], k_idx, w[:, j:j + 1], t)
        idx = oracle.topk(sc, k, t)
        t1 = time.perf_counter()
        if attn:
            oracle.sparse_attention(Q[:, j:j + 1], K, V, idx, scale)
        t2 = time.perf_counter()
        t_idx += t1 - t0
        t_att += t2 - t1
        sets.append(idx[0, 0])
    n = max(1, len(rows))
    return t_idx / n, t_att / n, sets


def _gpu_overlap(gpu_rows, oracle_rows):
    import oracle
    import numpy as np
    ovs = [oracle.overlap(g, w) for g, w in zip(gpu_rows, oracle_rows)]
    return {"rows": len(ovs), "mean": float(np.mean(ovs)), "min": float(np.min(ovs))}


def cpu_baseline(cfg, n_rows=4096):
    """Time the oracle (as it stands) on n_rows query rows of one F layer and
    one S layer of the prefill stack, then compose the 47-layer stack time.
    The same rows give the GPU-against-oracle top-k overlap of that layer (the
    GPU runs on copies of the same inputs)."""
    import numpy as np
    import torch
    import idxc_inputs as gen
    import dsa_lightning_indexer_score_amd as idxc
    host = host_info()
    L = gen.layer_inputs(cfg, 0, device="cpu")
    rows = np.unique(np.linspace(0, cfg.Lq - 1, n_rows).astype(int))
    f = gen.to_f64
    t_idx, t_att, sets = _oracle_row_times(
        f(L["q_idx"][:, rows]), f(L["k_idx"]), f(L["w"][:, rows]), f(L["q"][:, rows]), f(L["k"]),
        f(L["v"]), rows, cfg.k, cfg.scale, cfg.q_pos0)
    # per-row times of rows spread evenly over the positions, times Lq, give a layer
    nF = cfg.pattern.count("F")
    stack_s = cfg.B * cfg.Lq * (nF * t_idx + cfg.n_layers * t_att)
    allf_s = cfg.B * cfg.Lq * cfg.n_layers * (t_idx + t_att)
    # GPU selection of the same layer (same tensors) on the same rows
    gi = idxc.idxc_indexer_topk(L["q_idx"].cuda(), L["k_idx"].cuda(), L["w"].cuda(), cfg.k,
                                q_pos0=cfg.q_pos0)
    ov = _gpu_overlap(gi[0, rows].cpu().numpy(), sets)
    del gi
    torch.cuda.empty_cache()
    cores = host.get("blas_threads") or os.cpu_count() or 1
    return dict(value=cfg.B * cfg.Lq / stack_s, unit="tokens/s", cores=int(cores), kind="oracle",
                sample="%d query rows (evenly spaced over positions 0..%d) of one F layer "
                       "(indexer+top-k+attention) and attention of one S layer of %s; "
                       "per-row times composed to the 47-layer stack (%d F, %d layers); "
                       "measured %.1f s" % (len(rows), cfg.Lq - 1, cfg.name, nF, cfg.n_layers,
                                           len(rows) * (t_idx + t_att)),
                composed_stack_seconds=stack_s,
                allF_tokens_per_s_composed=cfg.B * cfg.Lq / allf_s,
                host=host, gpu_vs_oracle_topk_overlap=ov)


def cpu_baselines_other():
    """The oracle on the other configurations: the single 8192-token layer
    in full (median of three runs),
    the 47-layer decode step (8 sequences of 65536 cached tokens, composed per
    sequence to 64 sequences and 47 layers, 12-F and all-F), and the
    196608-token indexer + top-k in 4096-query chunks (8 rows of the first and
    8 of the last chunk; the per-row cost, linear in the row's keys, is fitted
    and summed over all rows: extrapolated). GPU-against-oracle top-k overlap
    on the same rows of the single layer and the decode batch."""
    import numpy as np
    import torch
    import idxc_inputs as gen
    import dsa_lightning_indexer_score_amd as idxc
    f = gen.to_f64
    out = {}
    # ---- single layer, L = 8192: the whole layer, median of three runs
    import oracle
    c2 = gen.C2
    L = gen.layer_inputs(c2, 0, device="cpu")
    F = {n: f(t) for n, t in L.items()}
    times = []
    t_all = time.perf_counter()
    for _ in range(3):
        t0 = time.perf_counter()
        sc = oracle.indexer_scores(F["q_idx"], F["k_idx"], F["w"], 0)
        want = oracle.topk(sc, c2.k, 0)
        oracle.sparse_attention(F["q"], F["k"], F["v"], want, c2.scale)
        times.append(time.perf_counter() - t0)
        del sc
    layer_s = float(np.median(times))
    gi = idxc.idxc_indexer_topk(L["q_idx"].cuda(), L["k_idx"].cuda(), L["w"].cuda(), c2.k)
    out[c2.name] = {"tokens_per_s": c2.Lq / layer_s, "kind": "full",
                    "sample": "the whole layer (%d query rows: indexer, top-k, attention), "
                              "median of 3 runs" % c2.Lq,
                    "run_s": [round(x, 3) for x in times],
                    "measured_s": time.perf_counter() - t_all,
                    "gpu_vs_oracle_topk_overlap": _gpu_overlap(gi[0].cpu().numpy(), want[0])}
    del gi, L, F, want
    # ---- decode step: 8 sequences of the 64 (same distributions, own seeds)
    c4 = gen.C4_12F
    nb = 8
    q, kk, w = gen.indexer_inputs(nb, 1, c4.Lk, c4.H_I, c4.d_I, kind="normal", seed=100)
    Q, K, V = gen.attn_inputs(nb, 1, c4.Lk, c4.H, c4.D, seed=101)
    t0 = time.perf_counter()
    ti = ta = 0.0
    sets = []
    for b in range(nb):
        a, bb, st = _oracle_row_times(f(q[b:b + 1]), f(kk[b:b + 1]), f(w[b:b + 1]),
                                      f(Q[b:b + 1]), f(K[b:b + 1]), f(V[b:b + 1]), [0], c4.k,
                                      c4.scale, c4.q_pos0)
        ti += a / nb
        ta += bb / nb
        sets.append(st[0])
    step12 = c4.B * (12 * ti + 47 * ta)
    stepF = c4.B * 47 * (ti + ta)
    gi = idxc.idxc_indexer_topk(q.cuda(), kk.cuda(), w.cuda(), c4.k, q_pos0=c4.q_pos0)
    out["stack47-decode-B64-Lk65536"] = {
        "tokens_per_s_12F": c4.B / step12, "tokens_per_s_allF": c4.B / stepF,
        "kind": "composed",
        "sample": "%d sequences; per-sequence F-layer (indexer+top-k+attention) and S-layer "
                  "(attention) times composed to 64 sequences x 47 layers" % nb,
        "measured_s": time.perf_counter() - t0,
        "gpu_vs_oracle_topk_overlap": _gpu_overlap(gi[:, 0].cpu().numpy(), sets)}
    del q, kk, w, Q, K, V, gi
    # ---- long context: rows of the first and the last 4096-query chunk
    Lc, chunk = gen.C5_L, gen.C5_CHUNK
    kf = f(gen.indexer_inputs(1, 1, Lc, 64, 128, kind="normal", seed=200)[1])
    t0 = time.perf_counter()
    pts = []
    for c0 in (0, Lc - chunk):
        rows = np.linspace(0, chunk - 1, 8).astype(int)
        qq, _, ww = gen.indexer_inputs(1, len(rows), Lc, 64, 128, kind="normal", seed=201 + c0)
        ti, _, _ = _oracle_row_times(f(qq), kf, f(ww), None, None, None, rows, 2048, 0.0, c0,
                                     attn=False)
        pts.append((c0 + chunk / 2.0, ti))
    (x0, y0), (x1, y1) = pts
    slope = (y1 - y0) / (x1 - x0)
    inter = y0 - slope * x0
    total = Lc * inter + slope * Lc * (Lc + 1) / 2.0
    out["long-context-L196608-indexer-topk"] = {
        "tokens_per_s": Lc / total, "kind": "extrapolated", "seconds": total,
        "sample": "8 rows of the first and 8 of the last 4096-query chunk; per-row time "
                  "fitted linear in the row position and summed over all %d rows" % Lc,
        "measured_s": time.perf_counter() - t0}
    return out


def overlap_records():
    """Cross-layer agreement of the layers' own selections (what an S layer
    would keep of its own top-k if it reused another layer's), for the 7
    distinct synthetic layers the benchmark cycles: idxc_overlap_matrix over
    each layer's own top-k of the last 1024 prefill rows (L = 32768) and of
    the 64 decode rows. Synthetic layers are independent draws, so these
    measure the chance agreement of i.i.d. layers (about k / t), not the
    pages' trained-model overlap."""
    import numpy as np
    import torch
    import idxc_inputs as gen
    import dsa_lightning_indexer_score_amd as idxc
    res = {}
    for cfg, nrows in ((gen.C3_12F, 1024), (gen.C4_12F, None)):
        sel = []
        for s in range(N_SETS):
            L = gen.layer_inputs(cfg, s, device="cuda")
            if nrows:
                q0 = cfg.Lq - nrows
                sel.append(idxc.idxc_indexer_topk(L["q_idx"][:, q0:], L["k_idx"], L["w"][:, q0:],
                                                  cfg.k, q_pos0=q0, order="position"))
            else:
                sel.append(idxc.idxc_indexer_topk(L["q_idx"], L["k_idx"], L["w"], cfg.k,
                                                  q_pos0=cfg.q_pos0, order="position"))
            del L
        sel = torch.stack(sel).contiguous()
        m = idxc.idxc_overlap_matrix(sel, cfg.Lk).cpu().numpy()
        order = [l % N_SETS for l in range(cfg.n_layers)]
        adj = [float(m[order[l], order[l + 1]]) for l in range(cfg.n_layers - 1)
               if order[l] != order[l + 1]]
        res[cfg.name.rsplit("-", 1)[0]] = {
            "rows": int(sel.shape[1] * sel.shape[2]), "layers": N_SETS,
            "adjacent_layer_overlap_mean": float(np.mean(adj)),
            "matrix": [[round(float(x), 5) for x in r] for r in m]}
        del sel
        torch.cuda.empty_cache()
    return res


# --------------------------------------------------------------------------- #
# counter passes: rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) -- python3 bench.py --only pmc
# --------------------------------------------------------------------------- #
CAL_BYTES = 1 << 30         # the calibration kernels read / write exactly this much
TRAFFIC_SOURCES = {
    "attention_prefill": ["attn.hip", "common.hpp", "kernels.hpp"],
    "indexer_topk_prefill": ["indexer.hip", "topk.hip", "radix_topk.hpp", "select.hpp",
                             "common.hpp", "kernels.hpp", "api.hip"],
    "indexer_topk_decode": ["indexer.hip", "topk.hip", "radix_topk.hpp", "select.hpp",
                            "common.hpp", "kernels.hpp", "api.hip"],
}


def calibration_launches():
    """The counter-scaling kernels: a fill that writes CAL_BYTES and an
    elementwise negation that reads CAL_BYTES (and writes CAL_BYTES)."""
    import torch
    src = torch.ones(CAL_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def topk_launches():
    """Standalone idxc_topk for a kernel trace or a counter pass: the
    calibration kernels, then 8192 causal rows of 8192 scores and 64 decode
    rows of 65536 (k = 2048), each in position and in score order, twice,
    each launch between synchronisations."""
    import torch
    import dsa_lightning_indexer_score_amd as idxc
    calibration_launches()
    for name, (B, Lq, Lk, q0) in (("8192 causal rows of 8192", (1, 8192, 8192, 0)),
                                  ("64 decode rows of 65536", (64, 1, 65536, 65535))):
        g = torch.Generator(device="cuda")
        g.manual_seed(0)
        s = torch.randn((B, Lq, Lk), generator=g, device="cuda")
        ws_n = idxc.idxc_topk_workspace_bytes(B, Lq, Lk, q0, 2048)
        ws = torch.empty((max(ws_n, 256),), dtype=torch.uint8, device="cuda")
        out = torch.empty((B, Lq, 2048), dtype=torch.int32, device="cuda")
        for order in ("position", "score"):
            for _ in range(2):
                torch.cuda.synchronize()
                idxc.idxc_topk(s, 2048, q_pos0=q0, workspace=ws, out=out, order=order)
                torch.cuda.synchronize()
            log("topk launches: %s, %s order done" % (name, order))
        del s, ws, out
        torch.cuda.empty_cache()


def pmc_launches():
    """Launches for a counter pass: a fill that writes CAL_BYTES, an
    elementwise negation that reads CAL_BYTES and writes CAL_BYTES, then one
    F layer (indexer + top-k, then attention) of the prefill and of the
    decode stack on their first input set, each bracketed by synchronisations."""
    import torch
    import idxc_inputs as gen
    import dsa_lightning_indexer_score_amd as idxc
    calibration_launches()
    for cfg in (gen.C3_12F, gen.C4_12F):
        L = gen.layer_inputs(cfg, 0, device="cuda")
        ws = torch.empty(idxc.idxc_workspace_bytes(cfg.B, cfg.Lq, cfg.Lk, cfg.q_pos0, cfg.H_I,
                                                   cfg.d_I, cfg.k, cfg.H, cfg.D),
                         dtype=torch.uint8, device="cuda")
        cache = torch.empty((cfg.B, cfg.Lq, cfg.k), dtype=torch.int32, device="cuda")
        out = torch.empty_like(L["q"])
        torch.cuda.synchronize()
        idxc.idxc_indexer_topk(L["q_idx"], L["k_idx"], L["w"], cfg.k, q_pos0=cfg.q_pos0,
                               workspace=ws, out=cache, order="position")
        torch.cuda.synchronize()
        idxc.idxc_sparse_attn(L["q"], L["k"], L["v"], cache, cfg.scale, workspace=ws, out=out)
        torch.cuda.synchronize()
        log("pmc launches of %s done" % cfg.name)
        del L, ws, cache, out
        torch.cuda.empty_cache()


def pmc_summary(fetch_csv, write_csv, command_fetch, command_write):
    """Write profiles/hbm_traffic.md from the two counter CSVs of --only pmc.

    Counter values are KiB per dispatch. Each is scaled by the ratio of the
    calibration kernels' known bytes to what the same counter reads for them
    (FETCH_SIZE: the negation reads CAL_BYTES; WRITE_SIZE: the fill writes
    CAL_BYTES)."""
    import csv
    import hashlib

    def rows(path, counter):
        out = []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Grid_Size"]),
                            float(r["Counter_Value"]) * 1024.0))
        return sorted(out)

    def short(name):
        n = name.replace("(anonymous namespace)::", "").replace("void ", "")
        return n.split("(")[0]

    f, w = rows(fetch_csv, "FETCH_SIZE"), rows(write_csv, "WRITE_SIZE")
    assert [(d, n) for d, n, _, _ in f] == [(d, n) for d, n, _, _ in w], "dispatch lists differ"
    neg = [x for x in f if "neg_kernel" in x[1] or "NegFunctor" in x[1]]
    fill = [x for x in w if "FillFunctor" in x[1]]
    assert neg and fill, "calibration kernels not found"
    cal_f = CAL_BYTES / neg[0][3]
    cal_w = CAL_BYTES / fill[0][3]
    idx = [i for i, x in enumerate(f) if short(x[1]).startswith("idxc::")]
    lines = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
             "FETCH_SIZE pass: `%s`" % command_fetch, "",
             "WRITE_SIZE pass: `%s`" % command_write, "",
             "Calibration: torch.neg over %d bytes reads FETCH_SIZE %.0f KiB (factor %.4f); "
             "torch.ones of %d bytes writes WRITE_SIZE %.0f KiB (factor %.4f)."
             % (CAL_BYTES, neg[0][3] / 1024, cal_f, CAL_BYTES, fill[0][3] / 1024, cal_w), "",
             "| dispatch | kernel | grid | FETCH KiB | WRITE KiB | scaled read MB | "
             "scaled write MB |", "|---|---|---|---|---|---|---|"]
    for i in idx:
        d, n, g, fb = f[i]
        wb = w[i][3]
        lines.append("| %d | %s | %d | %.0f | %.0f | %.1f | %.1f |"
                     % (d, short(n), g, fb / 1024, wb / 1024, fb * cal_f / 1e6, wb * cal_w / 1e6))
    # the pmc launches run, in order: prefill indexer (+ top-k), prefill
    # attention, decode indexer (+ top-k), decode attention
    groups, cur = [], []
    for i in idx:
        nm = short(f[i][1])
        if "attn" in nm and "merge" not in nm:
            groups.append(("indexer", cur))
            groups.append(("attention", [i]))
            cur = []
        elif "merge" in nm:
            groups[-1][1].append(i)
        else:
            cur.append(i)
    names = ["indexer_topk_prefill", "attention_prefill", "indexer_topk_decode",
             "attention_decode"]
    rec = {}
    csrc = os.path.join("dsa_lightning_indexer_score_amd", "csrc")
    for name, (_, members) in zip(names, groups):
        srcs = [os.path.join(csrc, x) for x in TRAFFIC_SOURCES.get(name, ["attn.hip",
                                                                          "common.hpp",
                                                                          "kernels.hpp"])]
        h = hashlib.sha256()
        for x in srcs:
            h.update(open(os.path.join(ROOT, x), "rb").read())
        tot = sum(f[i][3] * cal_f + w[i][3] * cal_w for i in members)
        rec[name] = {"sources": srcs, "sha": h.hexdigest()[:16], "bytes": round(tot),
                     "kernels": [short(f[i][1]) for i in members]}
    lines += ["", "Per launch (read + write, scaled); bench.py reports these as `traffic` "
              "while the listed sources hash to `sha`:", "",
              "traffic-json: " + json.dumps(rec, sort_keys=True), ""]
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    open(path, "w").write("\n".join(lines))
    print("\n".join(lines))


# --------------------------------------------------------------------------- #
# dispatch counts: rocprofv3 --kernel-trace --output-format csv -- python3 bench.py --only dispatch
# --------------------------------------------------------------------------- #
DISPATCH_PHASES = ["prefill 12-F step", "prefill all-F step", "decode 12-F step",
                   "decode all-F step", "long-context pass (48 chunks of 4096)"]


def dispatch_launches():
    """One step of each stack configuration and one long-context pass, each
    preceded by a marker kernel (a fill), for a kernel trace that counts the
    indexer dispatches per step."""
    import torch
    import idxc_inputs as gen
    import dsa_lightning_indexer_score_amd as idxc

    def mark(i):
        torch.cuda.synchronize()
        torch.full((1024 * (i + 1),), float(i), device="cuda")
        torch.cuda.synchronize()

    steps = []
    for c12, cF in ((gen.C3_12F, gen.C3_ALLF), (gen.C4_12F, gen.C4_ALLF)):
        layers, sets = build_stack(c12, N_SETS)
        ws = torch.empty(idxc.idxc_workspace_bytes(c12.B, c12.Lq, c12.Lk, c12.q_pos0, c12.H_I,
                                                   c12.d_I, c12.k, c12.H, c12.D),
                         dtype=torch.uint8, device="cuda")
        cache = torch.empty((c12.B, c12.Lq, c12.k), dtype=torch.int32, device="cuda")
        for c in (c12, cF):
            call = idxc.StackCall(c.pattern, layers, c.k, c.scale, c.q_pos0, index_cache=cache,
                                  workspace=ws)
            call()  # warm-up (not traced apart: the markers delimit the counted step)
            steps.append((call, layers, sets, ws, cache))
    Lc, chunk = gen.C5_L, gen.C5_CHUNK
    q, kk, w = gen.indexer_inputs(1, Lc, Lc, 64, 128, kind="normal", seed=0, device="cuda")
    wsl = torch.empty(idxc.idxc_workspace_bytes(1, chunk, Lc, Lc - chunk, 64, 128, 2048),
                      dtype=torch.uint8, device="cuda")
    outl = torch.empty((1, chunk, 2048), dtype=torch.int32, device="cuda")

    def long_pass():
        for c in range(Lc // chunk):
            idxc.idxc_indexer_topk(q[:, c * chunk:(c + 1) * chunk], kk[:, :(c + 1) * chunk],
                                   w[:, c * chunk:(c + 1) * chunk], 2048, q_pos0=c * chunk,
                                   workspace=wsl, out=outl)
    long_pass()
    calls = [st[0] for st in steps]
    for i, fn in enumerate(calls + [long_pass]):
        mark(i)
        n = fn()
        torch.cuda.synchronize()
        log("dispatch phase %d (%s) done%s" % (i, DISPATCH_PHASES[i],
                                              "" if n is None else ", indexer_calls=%d" % n))
    mark(len(calls) + 1)


def dispatch_summary(trace_csv, command):
    """Write profiles/dispatch_counts.md from the kernel trace of --only dispatch."""
    import csv
    import idxc_inputs as gen
    rows = list(csv.DictReader(open(trace_csv)))
    key = lambda r: int(r.get("Dispatch_Id") or r.get("Correlation_Id") or 0)
    rows.sort(key=key)
    names = [r["Kernel_Name"] for r in rows]
    marks = [i for i, n in enumerate(names) if "FillFunctor" in n]
    # the last len(DISPATCH_PHASES)+1 fills delimit the phases
    marks = marks[-(len(DISPATCH_PHASES) + 1):]
    assert len(marks) == len(DISPATCH_PHASES) + 1, "markers not found"

    def kind(n):
        n = n.replace("(anonymous namespace)::", "")
        if "indexer_" in n:
            return "indexer"
        if "topk_" in n:
            return "top-k selection"
        if "attn_merge" in n:
            return "attention merge"
        if "attn" in n:
            return "attention"
        return None

    expect_f = [gen.C3_12F.pattern.count("F"), 47, gen.C4_12F.pattern.count("F"), 47,
                gen.C5_L // gen.C5_CHUNK]
    lines = ["# Indexer dispatches per step (rocprofv3 kernel trace)", "",
             "Command: `%s`" % command, "",
             "Each phase is one step of the stack (or one pass of the long context) between "
             "two marker kernels; S layers launch no indexer work, so the indexer dispatches "
             "of a step equal its F layers (12 of 47 for the 12-F pattern, 47 for all-F), "
             "and a 196608-token pass in 4096-query chunks dispatches one indexer launch per "
             "chunk (48).", "",
             "| phase | F layers (or chunks) | indexer | top-k selection | attention | "
             "attention merge | indexer = F |", "|---|---|---|---|---|---|---|"]
    ok_all = True
    rec = {}
    for p in range(len(DISPATCH_PHASES)):
        cnt = {}
        for n in names[marks[p] + 1:marks[p + 1]]:
            k = kind(n)
            if k:
                cnt[k] = cnt.get(k, 0) + 1
        ok = cnt.get("indexer", 0) == expect_f[p]
        ok_all &= ok
        rec[DISPATCH_PHASES[p]] = cnt
        lines.append("| %s | %d | %d | %d | %d | %d | %s |" % (
            DISPATCH_PHASES[p], expect_f[p], cnt.get("indexer", 0), cnt.get("top-k selection", 0),
            cnt.get("attention", 0), cnt.get("attention merge", 0), "yes" if ok else "NO"))
    lines += ["", "All phases: indexer dispatches = F layers (chunks): %s" % ("yes" if ok_all
                                                                             else "NO"),
              "", "dispatch-json: " + json.dumps(rec, sort_keys=True), ""]
    path = os.path.join(ROOT, "profiles", "dispatch_counts.md")
    open(path, "w").write("\n".join(lines))
    print("\n".join(lines))


# --------------------------------------------------------------------------- #
def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.dispatch_summary:
        dispatch_summary(*args.dispatch_summary)
        return
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
    if args.only == "pmc":
        pmc_launches()
        return
    if args.only == "dispatch":
        dispatch_launches()
        return
    if args.only == "topk":
        topk_launches()
        return
    if args.only == "sweep":
        print(json.dumps({"context_sweep": context_sweep(), "distill_loss": distill_rate()}),
              flush=True)
        return

    res = {}
    extra = {}
    # ----------------------------------------------------------------- prefill
    idx_ms = att_ms = pass_ms = None
    if args.only not in ("decode",):
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
        # per-kernel durations: HIP events around every launch of a layer-by-layer
        # pass over the same 12-F stack
        idx_ms, att_ms, pass_ms = kernel_pass(cfg12, layers, ws, cache, args.steps)
        log("prefill per layer: indexer+top-k %.3f ms, attention %.3f ms (layer-by-layer pass "
            "%.2f ms/step)" % (idx_ms, att_ms, pass_ms))
        del layers, sets, call12, callF, ws, cache
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
        # the same decode steps replayed from captured HIP graphs (no host
        # launch work inside a step)
        graphs = {}
        for name, call in (("12F", dc12), ("allF", dcF)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                call()
            graphs[name] = g
        torch.cuda.synchronize()
        for name, g in graphs.items():
            dec["graph_" + name] = time_steps(g.replay, args.decode_steps, args.warmup)
        log("decode from graphs: 12-F %.3f ms/step, all-F %.3f ms/step"
            % (dec["graph_12F"] * 1e3, dec["graph_allF"] * 1e3))
        del graphs
        dec_idx_ms, dec_att_ms, dec_pass_ms = kernel_pass(d12, dlayers, dws, dcache,
                                                          args.decode_steps)
        log("decode: 12-F %.3f ms/step, all-F %.3f ms/step; per layer indexer+top-k %.3f ms, "
            "attention %.3f ms" % (dec["decode_12F"] * 1e3, dec["decode_allF"] * 1e3,
                                   dec_idx_ms, dec_att_ms))
        extra["decode_per_layer_ms"] = {"indexer_topk": dec_idx_ms, "attention": dec_att_ms}
        extra["decode_layer_by_layer_ms_per_step"] = dec_pass_ms
        extra["decode_indexer_hbm_gbs"] = indexer_bytes(d12) / (dec_idx_ms * 1e-3) / 1e9
        extra["decode_attention_gbs"] = attn_bytes(d12) / (dec_att_ms * 1e-3) / 1e9
        del dlayers, dsets, dc12, dcF, dws, dcache
        torch.cuda.empty_cache()

    # ------------------------------------------------- long context, top-k
    if not args.skip_decode and args.only == "":
        import idxc_inputs as gen
        lc = long_context(gen.C5_L, gen.C5_CHUNK)
        log("long context L=%d in %d chunks: %.1f ms, %.0f TFLOP/s indexer"
            % (lc["L"], lc["chunks"], lc["ms"], lc["TFLOPs"]))
        extra["long_context_indexer_topk"] = lc
        torch.cuda.empty_cache()
        extra["context_sweep"] = context_sweep()
        torch.cuda.empty_cache()
        dl = distill_rate()
        log("distillation loss (4 teachers, 2048 x 32768 chunk): %.3f ms, %.0f GB/s"
            % (dl["ms"], dl["GBs"]))
        extra["distill_loss"] = dl
        dll = distill_rate(Lq=512, Lk=131072)
        log("distillation loss (4 teachers, 512 x 131072 chunk, streamed rows): %.3f ms, %.0f GB/s"
            % (dll["ms"], dll["GBs"]))
        extra["distill_loss_long_rows"] = dll
        ov = overlap_rate()
        log("cross-layer overlap (two 32768 x 2048 index tensors): %.3f ms, %.0f GB/s"
            % (ov["ms"], ov["GBs"]))
        extra["overlap_rate"] = ov
        tk = {"decode_rows": standalone_topk(64, 1, 65536, 65535, 2048),
              "prefill_rows": standalone_topk(1, 8192, 8192, 0, 2048),
              "decode_rows_position_order": standalone_topk(64, 1, 65536, 65535, 2048,
                                                            order="position"),
              "prefill_rows_position_order": standalone_topk(1, 8192, 8192, 0, 2048,
                                                             order="position")}
        log("standalone top-k: %.0f GB/s (64 x 65536), %.0f GB/s (8192 x 8192 causal); "
            "position order %.0f / %.0f GB/s"
            % (tk["decode_rows"]["GBs"], tk["prefill_rows"]["GBs"],
               tk["decode_rows_position_order"]["GBs"], tk["prefill_rows_position_order"]["GBs"]))
        extra["standalone_topk"] = tk
        torch.cuda.empty_cache()
        extra["cross_layer_overlap"] = overlap_records()
        log("cross-layer overlap of the 7 synthetic layers' own selections: prefill %.4f, "
            "decode %.4f (adjacent layers, mean)"
            % (extra["cross_layer_overlap"]["stack47-prefill-L32768"]["adjacent_layer_overlap_mean"],
               extra["cross_layer_overlap"]["stack47-decode-B64-Lk65536"]["adjacent_layer_overlap_mean"]))
        torch.cuda.empty_cache()

    # ------------------------------------------------------------------ report
    cfg = gen.C3_12F
    s12 = res.get("prefill_12F")
    sF = res.get("prefill_allF")
    value = cfg.B * cfg.Lq / s12 if s12 else None
    dominant = None
    if idx_ms is not None:
        idx_tflops = indexer_flops(cfg) / (idx_ms * 1e-3) / 1e12
        att_gbs = attn_bytes(cfg) / (att_ms * 1e-3) / 1e9
        nF = cfg.pattern.count("F")
        # dominant kernel of the headline workload by total time per step
        idx_total, att_total = nF * idx_ms, cfg.n_layers * att_ms
        att_tflops = attn_flops(cfg) / (att_ms * 1e-3) / 1e12
        roof_idx = {"kernel": "indexer_rows_kernel + topk_pairs_kernel (fused indexer + top-k of one F "
                              "layer, idxc_indexer_topk)",
                    "bound": "mfma", "achieved": idx_tflops, "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": idx_tflops / PEAK_BF16_TFLOPS,
                    "traffic": hbm_traffic("indexer_topk_prefill"),
                    "algorithmic": "%.4g flop per launch = causal pairs %d x 2*H_I*d_I"
                                   % (indexer_flops(cfg), causal_pairs(cfg.q_pos0, cfg.Lq)),
                    "launch_ms": idx_ms}
        # QK^T and PV over the gathered rows are dense bf16 MFMA contractions; the
        # gathered K/V rows (2*D*2 bytes per selected pair) come mostly from L2 and
        # the last-level cache (one layer's K and V are 16 MB), not from HBM
        roof_att = {"kernel": "sparse_attn_kernel (one layer, idxc_sparse_attn)",
                    "bound": "mfma", "achieved": att_tflops, "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": att_tflops / PEAK_BF16_TFLOPS,
                    "traffic": hbm_traffic("attention_prefill"),
                    "algorithmic": "%.4g flop per launch = selected pairs %d x 4*H*D"
                                   % (attn_flops(cfg), cfg.B * selected_pairs(cfg.q_pos0, cfg.Lq,
                                                                               cfg.k)),
                    "gathered_GBs": att_gbs,
                    "gathered_bytes": attn_bytes(cfg),
                    "launch_ms": att_ms}
        dominant, other = (roof_idx, roof_att) if idx_total >= att_total else (roof_att, roof_idx)
        # idealised stack: every F layer's indexer and every layer's attention
        # at the bf16 MFMA peak
        t_roof = (nF * indexer_flops(cfg) + cfg.n_layers * attn_flops(cfg)) / (
            PEAK_BF16_TFLOPS * 1e12) * 1e3
        extra.update({
            "stack_roofline_ms_12F": t_roof,
            "stack_roofline_frac_12F": (t_roof / (s12 * 1e3)) if s12 else None,
            "prefill_allF_tokens_per_s": cfg.B * cfg.Lq / sF if sF else None,
            "prefill_allF_ms_per_step": sF * 1e3 if sF else None,
            "prefill_speedup_12F_vs_allF": (sF / s12) if (sF and s12) else None,
            "prefill_per_layer_ms": {"indexer_topk": idx_ms, "attention": att_ms},
            "prefill_layer_by_layer_ms_per_step": pass_ms,
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
            "decode_graph_12F_tokens_per_s": gen.C4_12F.B / dec["graph_12F"],
            "decode_graph_allF_tokens_per_s": gen.C4_ALLF.B / dec["graph_allF"],
            "decode_graph_12F_ms_per_step": dec["graph_12F"] * 1e3,
            "decode_graph_allF_ms_per_step": dec["graph_allF"] * 1e3,
        })
    cpu = None
    if not args.skip_cpu:
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(cfg)
        log("cpu oracle: %.3g tokens/s on %d threads; GPU-vs-oracle overlap on %d rows: mean "
            "%.5f min %.5f" % (cpu["value"], cpu["cores"], cpu["gpu_vs_oracle_topk_overlap"]["rows"],
                               cpu["gpu_vs_oracle_topk_overlap"]["mean"],
                               cpu["gpu_vs_oracle_topk_overlap"]["min"]))
        if args.only == "":
            extra["cpu_baseline_other"] = cpu_baselines_other()
            log("cpu oracle, other configurations: %s" % json.dumps(
                {k: v.get("tokens_per_s", v.get("tokens_per_s_12F"))
                 for k, v in extra["cpu_baseline_other"].items()}))
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
