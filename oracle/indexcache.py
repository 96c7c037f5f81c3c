"""CPU oracle for the IndexCache hot path (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module. The HIP library never calls it and shares
no code with it. It is plain numpy: inputs are exact fp64 copies of the bf16
tensors, every sum is taken in fp64, and results are rounded once to fp32.

Sources (web pages; cited by title and section):
  [W] "IndexCache：跨层复用稀疏注意力的索引" (wineandchord.com/llm/landscape/works/indexcache)
      - "从 DSA 的成本分解开始" (starting from DSA's cost decomposition): the
        C_indexer cost, the F/S roles, I_l = TopK(s_l, k), first layer must be F,
        and the refresh -> share -> refresh state machine with its FSSF, k=2
        worked example.
      - "相邻层重叠很高，但“重叠率”不是搜索目标" (high overlap is not the search
        objective): the Overlap(l, j) = |I_l ∩ I_j| / k equation.
      - "Training-free：直接用语言模型损失选择 Full 层": greedy selection with an
        injectable loss, its toy example and the forward-count sum.
  [J] "NLP——IndexCache" notes (joezjh.github.io): section "IndexCache 方法"
      (T_t^(l) <- T_t^(f(l)), f(l) = max{j < l : c_j = F}); section
      "背景 & 问题提出" (the indexer picks the top-k, k = 2048, from all previous
      tokens; core attention runs on those k only).
  [S] skillsmp.com skill card "indexcache-sparse-attention-acceleration",
      section "Step 1" (Jaccard overlap of consecutive layers' top-k sets) and
      the IndexCacheManager (an S layer with no cache is an error).

Readings where the pages are silent (each is listed in the design doc):
  * Indexer score (the pages name it but never write it): per indexer head h,
    ReLU(q_I[t,h,:] . k_I[s,:]), times a per-query head weight w[t,h], summed
    over heads. One indexer key vector per token, shared by all indexer heads.
  * Candidates of query position t are s in [0, t] (the query itself included).
  * Order: higher score first, then lower position; -0.0 counts as +0.0.
    Output sorted in that order, min(k, t+1) entries, padded with -1.
  * Core attention: softmax(scale * Q[t,h] . K[s]) over the selected s, then
    the weighted sum of V[s]; one shared K/V head (MQA); scale passed in
    (1/sqrt(D) in every configuration); -1 entries are skipped.
  * Layers are independent apart from the index cache (no model is defined).

Parity pins: every function here is pinned in tests/test_oracle_*.py against
closed forms, brute force, library special cases or the pages' worked examples.
"""
from __future__ import annotations

from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

PAD = -1


# --------------------------------------------------------------------------- #
# a1: pattern validation and the nearest-F rule  ([W] cost decomposition;
#     [J] "IndexCache 方法" equation f(l) = max{j < l : c_j = F})
# --------------------------------------------------------------------------- #
def validate_pattern(pattern: str, n_layers: int) -> None:
    """Raise ValueError unless pattern has n_layers chars in {F,S} with c_0 = F."""
    if not isinstance(pattern, str):
        raise ValueError("pattern must be a string")
    if len(pattern) != n_layers:
        raise ValueError("pattern length %d != number of layers %d"
                         % (len(pattern), n_layers))
    if n_layers < 1:
        raise ValueError("need at least one layer")
    for c in pattern:
        if c not in ("F", "S"):
            raise ValueError("unknown layer role %r (only 'F' and 'S' exist)" % c)
    if pattern[0] != "F":
        raise ValueError("layer 0 has no earlier F layer to share from; it has to be 'F'")


def nearest_full(pattern: str) -> List[int]:
    """source[l] = l for F layers, f(l) = max{j < l : c_j = F} for S layers."""
    validate_pattern(pattern, len(pattern))
    src = []
    for l, c in enumerate(pattern):
        if c == "F":
            src.append(l)
        else:
            src.append(max(j for j in range(l) if pattern[j] == "F"))
    return src


# --------------------------------------------------------------------------- #
# a2 + a3: lightning-indexer scores  ([J] background; [W] cost decomposition,
#          s_l is the score whose top-k is I_l)
# --------------------------------------------------------------------------- #
def _canon_zero(x: np.ndarray) -> np.ndarray:
    """Map -0.0 to +0.0 (keeps every other value bit-identical)."""
    x = np.array(x, copy=True)
    x[x == 0] = 0.0
    return x


def row_position(b: int, i: int, q_pos0: int, q_pos: Optional[np.ndarray], Lk: int) -> int:
    """Absolute position t of query row (b, i): q_pos0 + i, or q_pos[b, i] for
    per-row (ragged) positions, where a negative entry means "no candidates"
    (-1) and entries past the last key are read as Lk - 1."""
    if q_pos is None:
        return q_pos0 + i
    t = int(np.asarray(q_pos)[b, i])
    return -1 if t < 0 else min(t, Lk - 1)


def indexer_scores(q_idx: np.ndarray, k_idx: np.ndarray, w: np.ndarray,
                   q_pos0: int, Lk: Optional[int] = None,
                   q_pos: Optional[np.ndarray] = None) -> np.ndarray:
    """score[b,i,s] = fp32( sum_h w[b,i,h] * max(0, q_idx[b,i,h,:] . k_idx[b,s,:]) ).

    Shapes: q_idx [B,Lq,H_I,d_I], k_idx [B,Lk,d_I], w [B,Lq,H_I] (exact fp64
    values of the bf16 inputs). Row i is query position t = q_pos0 + i (or
    q_pos[b, i], see row_position); only s <= t are candidates, the rest are
    returned as -inf. Sums in fp64, one rounding to fp32, then -0.0 -> +0.0.
    """
    q_idx = np.asarray(q_idx, dtype=np.float64)
    k_idx = np.asarray(k_idx, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, Lq, H_I, d_I = q_idx.shape
    if Lk is None:
        Lk = k_idx.shape[1]
    if q_pos is None and q_pos0 + Lq > Lk:
        raise ValueError("query rows exceed the key range")
    out = np.full((B, Lq, Lk), -np.inf, dtype=np.float32)
    for b in range(B):
        for i in range(Lq):
            t = row_position(b, i, q_pos0, q_pos, Lk)
            if t < 0:
                continue
            keys = k_idx[b, : t + 1, :]                  # [t+1, d_I]
            dots = keys @ q_idx[b, i].T                   # [t+1, H_I], fp64
            relu = np.maximum(dots, 0.0)
            s64 = relu @ w[b, i]                          # [t+1]
            out[b, i, : t + 1] = _canon_zero(s64.astype(np.float32))
    return out


# --------------------------------------------------------------------------- #
# a4: per-query top-k  ([W] I_l = TopK(s_l, k); [J] k most relevant of all
#     previous tokens)
# --------------------------------------------------------------------------- #
def topk_row(scores_row: np.ndarray, n_cand: int, k: int) -> np.ndarray:
    """Top-k of candidates 0..n_cand-1 of one fp32 score row.

    Strict total order: higher score first, then lower position (-0.0 == +0.0).
    Returns int32 [k]: the first min(k, n_cand) positions in that order, then -1.
    """
    vals = _canon_zero(np.asarray(scores_row[:n_cand], dtype=np.float32))
    pos = np.arange(n_cand, dtype=np.int64)
    # lexsort: last key is primary -> score descending, then position ascending
    order = np.lexsort((pos, -vals.astype(np.float64)))
    m = min(k, n_cand)
    out = np.full(k, PAD, dtype=np.int32)
    out[:m] = pos[order[:m]].astype(np.int32)
    return out


def topk(scores: np.ndarray, k: int, q_pos0: int,
         q_pos: Optional[np.ndarray] = None) -> np.ndarray:
    """indices[b,i,:] = topk_row(scores[b,i], t+1, k) with t = q_pos0 + i (or
    q_pos[b, i], see row_position)."""
    B, Lq, Lk = scores.shape
    out = np.empty((B, Lq, k), dtype=np.int32)
    for b in range(B):
        for i in range(Lq):
            out[b, i] = topk_row(scores[b, i], row_position(b, i, q_pos0, q_pos, Lk) + 1, k)
    return out


# --------------------------------------------------------------------------- #
# a6: gathered sparse core attention  ([J] background: core attention only on
#     the k selected tokens, O(Lk); [F] abstract)
# --------------------------------------------------------------------------- #
def sparse_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray,
                     indices: np.ndarray, scale: float) -> np.ndarray:
    """O[b,i,h] = sum_{s in S} p_s V[b,s],  p = softmax_s(scale * Q[b,i,h].K[b,s]).

    S = the entries of indices[b,i] that are not -1. Q [B,Lq,H,D], K/V
    [B,Lk,D] (one shared KV head), indices [B,Lq,k]. fp64 throughout, fp32 out.
    A row with no valid entry yields zeros.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, Lq, H, D = Q.shape
    out = np.zeros((B, Lq, H, D), dtype=np.float32)
    for b in range(B):
        for i in range(Lq):
            sel = indices[b, i]
            sel = sel[sel != PAD].astype(np.int64)
            if sel.size == 0:
                continue
            z = scale * (Q[b, i] @ K[b, sel].T)          # [H, n]
            z = z - z.max(axis=1, keepdims=True)
            p = np.exp(z)
            p = p / p.sum(axis=1, keepdims=True)
            out[b, i] = (p @ V[b, sel]).astype(np.float32)
    return out


# --------------------------------------------------------------------------- #
# a5 + a7: index cache and the F/S layer loop  ([W] "从 DSA 的成本分解开始": an
#          F layer's top-k replaces the single cached index tensor, an S layer
#          reuses it; [J] "IndexCache 方法": the f(l) rule)
# --------------------------------------------------------------------------- #
def schedule(layer_scores: Sequence[np.ndarray], pattern: str, k: int,
             q_pos0: int) -> Tuple[List[np.ndarray], int]:
    """Index sets of every layer of a stack from precomputed per-layer scores.

    layer_scores[l] is [B,Lq,Lk] fp32 (only F layers' entries are read).
    By definition an F layer l selects I_l = TopK(s_l, k) and an S layer l
    uses I_{f(l)}, f(l) the nearest earlier F layer ([J] "IndexCache 方法");
    the indexer therefore runs once per F layer. Returns (I_l for every
    layer, number of indexer evaluations).
    """
    validate_pattern(pattern, len(layer_scores))
    src = nearest_full(pattern)
    own = {l: topk(np.asarray(layer_scores[l]), k, q_pos0)
           for l in range(len(pattern)) if pattern[l] == "F"}
    selected = [own[src[l]].copy() for l in range(len(pattern))]
    return selected, len(own)


def layer_stack(pattern: str, layers: Sequence[Dict[str, np.ndarray]], k: int,
                scale: float, q_pos0: int, Lk: Optional[int] = None,
                q_pos: Optional[np.ndarray] = None):
    """Full hot path over a stack: per layer {indexer + top-k if F} + attention.

    layers[l] holds fp64 arrays q_idx, k_idx, w (read on F layers only) and
    q, k, v. Every layer attends over I_{src(l)}, src(l) = l on F layers and
    f(l) on S layers. Returns dict(indices=[per layer], out=[per layer],
    calls=int, scores=[per F layer or None]).
    """
    validate_pattern(pattern, len(layers))
    src = nearest_full(pattern)
    scores_all: List[Optional[np.ndarray]] = [None] * len(pattern)
    own: Dict[int, np.ndarray] = {}
    for l in range(len(pattern)):
        if pattern[l] == "F":
            L = layers[l]
            scores_all[l] = indexer_scores(L["q_idx"], L["k_idx"], L["w"], q_pos0, Lk, q_pos)
            own[l] = topk(scores_all[l], k, q_pos0, q_pos)
    sel_all = [own[src[l]].copy() for l in range(len(pattern))]
    out_all = [sparse_attention(layers[l]["q"], layers[l]["k"], layers[l]["v"], sel_all[l],
                                scale) for l in range(len(pattern))]
    return dict(indices=sel_all, out=out_all, calls=len(own), scores=scores_all)


# --------------------------------------------------------------------------- #
# Metrics  ([W] Overlap(l, j) = |I_l ∩ I_j| / k; [S] "Step 1" Jaccard)
# --------------------------------------------------------------------------- #
def position_order(indices: np.ndarray) -> np.ndarray:
    """The same top-k sets with each row's valid positions in increasing order
    and the PAD entries last: the order in which a layer stack's index cache
    holds them (the selection, a set, is unchanged; attention over the set
    does not depend on its order)."""
    ix = np.asarray(indices)
    key = np.where(ix == PAD, np.iinfo(np.int64).max, ix.astype(np.int64))
    return np.take_along_axis(ix, np.argsort(key, axis=-1, kind="stable"), axis=-1)


def _valid_set(row: np.ndarray) -> set:
    return set(int(x) for x in np.asarray(row).ravel() if int(x) != PAD)


def overlap(a_row: np.ndarray, b_row: np.ndarray) -> float:
    """|A ∩ B| / |A| over the valid (non -1) entries; equals the pages' /k when
    |A| = k. Two empty sets give 1.0."""
    A, Bs = _valid_set(a_row), _valid_set(b_row)
    if not A:
        return 1.0 if not Bs else 0.0
    return len(A & Bs) / len(A)


def jaccard(a_row: np.ndarray, b_row: np.ndarray) -> float:
    """|A ∩ B| / |A ∪ B| over the valid entries (the union is never empty for a
    real row, so no epsilon is added). Two empty sets give 1.0."""
    A, Bs = _valid_set(a_row), _valid_set(b_row)
    U = A | Bs
    if not U:
        return 1.0
    return len(A & Bs) / len(U)


def mean_overlap(a: np.ndarray, b: np.ndarray) -> Tuple[float, float]:
    """(mean, min) of overlap over all rows of two [...,k] index tensors."""
    a2 = np.asarray(a).reshape(-1, a.shape[-1])
    b2 = np.asarray(b).reshape(-1, b.shape[-1])
    vals = [overlap(x, y) for x, y in zip(a2, b2)]
    return float(np.mean(vals)), float(np.min(vals))


def overlap_matrix(sel: np.ndarray) -> np.ndarray:
    """M[a, b] = mean over rows of overlap(sel[a], sel[b]) for index tensors
    sel [n_layers, ..., k]: the pages' Overlap(l, j) for every pair of layers
    ([W] "相邻层重叠很高，但“重叠率”不是搜索目标", Overlap equation), in fp64."""
    sel = np.asarray(sel)
    n = sel.shape[0]
    m = np.empty((n, n), dtype=np.float64)
    for a in range(n):
        for b in range(n):
            m[a, b] = mean_overlap(sel[a], sel[b])[0]
    return m


def overlap_proxy_loss(pattern: str, matrix: np.ndarray) -> float:
    """Stand-in loss for the greedy search when no language model is at hand
    (the pages use the LM loss): (1/n) * sum over S layers l of
    (1 - M[l, f(l)]), f(l) the latest F layer before l ([J] "IndexCache 方法")."""
    validate_pattern(pattern, len(pattern))
    src = nearest_full(pattern)
    n = len(pattern)
    total = sum(1.0 - float(matrix[l][src[l]]) for l in range(n) if pattern[l] == "S")
    return total / n


# --------------------------------------------------------------------------- #
# Multi-layer distillation loss ([J] "方法二：Training-Aware IndexCache":
# L_multi = sum_j 1/(m+1) sum_t KL(p_t^(l+j) || q_t^(l)), q = Softmax(I_t);
# Proposition 1: its gradient equals that of KL against the mean teacher)
# --------------------------------------------------------------------------- #
def distill_loss(logits: np.ndarray, teachers: np.ndarray, q_pos0: int,
                 q_pos: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row multi-teacher KL and its gradient with respect to the logits.

    logits [B,Lq,Lk] are the indexer scores I_t of row (b,i) over keys
    0..t (t from row_position; entries past t are ignored); teachers
    [n,B,Lq,Lk] are n distributions over the same keys (entries past t
    ignored). Returns (loss [B,Lq] = (1/n) sum_j sum_s p_j log(p_j / q),
    grad [B,Lq,Lk] = dloss/dlogits = q - mean_j p_j on 0..t, 0 beyond), fp64,
    with 0 log 0 = 0 and q = softmax over 0..t.
    """
    I = np.asarray(logits, dtype=np.float64)
    P = np.asarray(teachers, dtype=np.float64)
    n = P.shape[0]
    B, Lq, Lk = I.shape
    loss = np.zeros((B, Lq))
    grad = np.zeros((B, Lq, Lk))
    for b in range(B):
        for i in range(Lq):
            t = row_position(b, i, q_pos0, q_pos, Lk)
            if t < 0:
                continue
            x = I[b, i, : t + 1]
            logq = x - (x.max() + np.log(np.exp(x - x.max()).sum()))
            total = 0.0
            for j in range(n):
                p = P[j, b, i, : t + 1]
                nz = p > 0
                total += float(np.sum(p[nz] * (np.log(p[nz]) - logq[nz])))
            loss[b, i] = total / n
            grad[b, i, : t + 1] = np.exp(logq) - P[:, b, i, : t + 1].mean(axis=0)
    return loss, grad


# --------------------------------------------------------------------------- #
# Greedy layer selection with an injectable loss ([W] "Training-free：直接用语言
# 模型损失选择 Full 层"; [J] "核心算法：Greedy Layer Selection", Algorithm 1)
# --------------------------------------------------------------------------- #
def greedy_pattern(n_layers: int, removals: int,
                   loss: Callable[[str], float]) -> Tuple[str, int]:
    """Best-improvement greedy F->S flips, layer 0 pinned to F.

    Each step tries every remaining F layer (except layer 0) as S, evaluates
    ``loss`` on the trial pattern and commits the lowest; ties go to the lower
    layer index. Returns (pattern, number of loss evaluations).
    """
    if removals < 0 or removals > n_layers - 1:
        raise ValueError("removals must be in [0, n_layers-1]")
    pat = ["F"] * n_layers
    evals = 0
    for _ in range(removals):
        best = None
        for layer in range(1, n_layers):
            if pat[layer] != "F":
                continue
            trial = pat.copy()
            trial[layer] = "S"
            v = loss("".join(trial))
            evals += 1
            if best is None or v < best[0]:
                best = (v, layer)
        pat[best[1]] = "S"
    return "".join(pat), evals
