"""Seeded synthetic inputs shared by the HIP path's tests/bench and the CPU oracle.

This module only draws random tensors. It holds none of the method's arithmetic:
no scoring, no selection, no attention. Both sides receive the very same tensors
(the HIP path as device bf16/fp32/int32 tensors, the oracle as exact fp64/int
numpy copies).

Workload shapes follow the synthetic configurations of the IndexCache hot path
(lightning-indexer scoring -> per-query top-k -> index cache -> gathered sparse
attention). The pages measure a 30B, 47-layer DSA model at up to 200K context
("IndexCache：跨层复用稀疏注意力的索引", wineandchord.com, section
"速度数字应该怎样读" / how to read the speed numbers); no weights or datasets are
available, so seeded random tensors of those shapes stand in for them.

Draw order inside one generator call is fixed and documented per function, so a
given (seed, shape) always yields the same tensors on every machine for CPU
generation. Device generation (``device='cuda'``) uses torch's seeded device
generator and is only reproducible on the same device type; tests that compare
against the oracle always copy the drawn device tensors to the host.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch


# --------------------------------------------------------------------------- #
# Configurations
# --------------------------------------------------------------------------- #
@dataclasses.dataclass(frozen=True)
class StackConfig:
    name: str
    n_layers: int
    pattern: str
    B: int
    Lq: int
    Lk: int
    q_pos0: int
    H_I: int
    d_I: int
    H: int
    D: int
    k: int
    kind: str  # "int" (integer-valued indexer inputs) or "normal"
    idx_std: float = 1.0  # std of q_I / k_I for kind == "normal"
    w_kind: str = "normal"  # "quarter" -> {0.25,0.5,1}; "normal" -> N(0,1)
    seed: int = 0

    @property
    def scale(self) -> float:
        return float(self.D) ** -0.5


def twelve_f_pattern(n_layers: int = 47) -> str:
    """F at layers 0, 4, 8, ... (every 4th layer, first layer F)."""
    return "".join("F" if l % 4 == 0 else "S" for l in range(n_layers))


C1 = StackConfig("tiny-fssf-L256", 4, "FSSF", 1, 256, 256, 0, 4, 32, 4, 64, 16,
                 "int", w_kind="quarter")
C2 = StackConfig("single-layer-prefill-L8192", 1, "F", 1, 8192, 8192, 0, 64, 128,
                 64, 128, 2048, "normal", idx_std=128 ** -0.5, w_kind="normal")
C3_12F = StackConfig("stack47-prefill-L32768-12F", 47, twelve_f_pattern(47), 1,
                     32768, 32768, 0, 64, 128, 64, 128, 2048, "normal")
C3_ALLF = dataclasses.replace(C3_12F, name="stack47-prefill-L32768-allF",
                              pattern="F" * 47)
C4_12F = StackConfig("stack47-decode-B64-Lk65536-12F", 47, twelve_f_pattern(47), 64,
                     1, 65536, 65535, 64, 128, 64, 128, 2048, "normal")
C4_ALLF = dataclasses.replace(C4_12F, name="stack47-decode-B64-Lk65536-allF",
                              pattern="F" * 47)
C5_L = 196608
C5_CHUNK = 4096


# --------------------------------------------------------------------------- #
# Generators
# --------------------------------------------------------------------------- #
def _gen(seed: int, device: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def indexer_inputs(B: int, Lq: int, Lk: int, H_I: int, d_I: int, *, kind: str,
                   seed: int, idx_std: float = 1.0, w_kind: str = "normal",
                   device: str = "cpu"):
    """Draw (q_I [B,Lq,H_I,d_I], k_I [B,Lk,d_I], w [B,Lq,H_I]) as bf16.

    Draw order: q_I, then k_I, then w, from one generator seeded with ``seed``.
    kind == "int": q_I, k_I integers uniform in [-4, 4] (inclusive, 9 values).
    kind == "normal": q_I, k_I ~ N(0, idx_std^2).
    w_kind == "quarter": w uniform over {0.25, 0.5, 1}; "normal": N(0,1);
    "neg-quarter": uniform over {-1, -0.5, -0.25, 0.25, 0.5, 1}.
    """
    g = _gen(seed, device)
    if kind == "int":
        q = torch.randint(-4, 5, (B, Lq, H_I, d_I), generator=g, device=device)
        kk = torch.randint(-4, 5, (B, Lk, d_I), generator=g, device=device)
        q = q.to(torch.bfloat16)
        kk = kk.to(torch.bfloat16)
    elif kind == "normal":
        q = (torch.randn((B, Lq, H_I, d_I), generator=g, device=device) * idx_std)
        kk = (torch.randn((B, Lk, d_I), generator=g, device=device) * idx_std)
        q = q.to(torch.bfloat16)
        kk = kk.to(torch.bfloat16)
    else:
        raise ValueError(kind)
    if w_kind == "quarter":
        sel = torch.randint(0, 3, (B, Lq, H_I), generator=g, device=device)
        w = torch.tensor([0.25, 0.5, 1.0], device=device)[sel]
    elif w_kind == "neg-quarter":
        sel = torch.randint(0, 6, (B, Lq, H_I), generator=g, device=device)
        w = torch.tensor([-1.0, -0.5, -0.25, 0.25, 0.5, 1.0], device=device)[sel]
    elif w_kind == "normal":
        w = torch.randn((B, Lq, H_I), generator=g, device=device)
    else:
        raise ValueError(w_kind)
    return q.contiguous(), kk.contiguous(), w.to(torch.bfloat16).contiguous()


def attn_inputs(B: int, Lq: int, Lk: int, H: int, D: int, *, seed: int,
                device: str = "cpu"):
    """Draw (Q [B,Lq,H,D], K [B,Lk,D], V [B,Lk,D]) as bf16 N(0,1).

    Draw order: Q, K, V from one generator seeded with ``seed``.
    """
    g = _gen(seed, device)
    Q = torch.randn((B, Lq, H, D), generator=g, device=device).to(torch.bfloat16)
    K = torch.randn((B, Lk, D), generator=g, device=device).to(torch.bfloat16)
    V = torch.randn((B, Lk, D), generator=g, device=device).to(torch.bfloat16)
    return Q.contiguous(), K.contiguous(), V.contiguous()


def layer_inputs(cfg: StackConfig, layer: int, device: str = "cpu"):
    """All six inputs of one layer of a stack config.

    Indexer inputs use seed ``cfg.seed + 2*layer``; attention inputs use
    ``cfg.seed + 2*layer + 1``. Indexer inputs are drawn for every layer (S
    layers never read them on the HIP path).
    """
    q_i, k_i, w = indexer_inputs(cfg.B, cfg.Lq, cfg.Lk, cfg.H_I, cfg.d_I,
                                 kind=cfg.kind, seed=cfg.seed + 2 * layer,
                                 idx_std=cfg.idx_std, w_kind=cfg.w_kind,
                                 device=device)
    Q, K, V = attn_inputs(cfg.B, cfg.Lq, cfg.Lk, cfg.H, cfg.D,
                          seed=cfg.seed + 2 * layer + 1, device=device)
    return dict(q_idx=q_i, k_idx=k_i, w=w, q=Q, k=K, v=V)


def score_rows(B: int, Lq: int, Lk: int, *, kind: str, seed: int,
               device: str = "cpu") -> torch.Tensor:
    """fp32 score matrices [B,Lq,Lk] used to drive a stand-alone top-k.

    kind == "normal": N(0,1) fp32.  kind == "ties": integers in [-3, 3] (heavy
    ties, includes zeros).  kind == "signed-zero": values in {-0.0, +0.0, 1.0}.
    kind == "const": all 0.5.  Entries above the causal diagonal are left as
    drawn; a top-k must never read them.
    """
    g = _gen(seed, device)
    if kind == "normal":
        return torch.randn((B, Lq, Lk), generator=g, device=device)
    if kind == "ties":
        return torch.randint(-3, 4, (B, Lq, Lk), generator=g,
                             device=device).to(torch.float32)
    if kind == "signed-zero":
        sel = torch.randint(0, 3, (B, Lq, Lk), generator=g, device=device)
        return torch.tensor([-0.0, 0.0, 1.0], device=device)[sel]
    if kind == "const":
        return torch.full((B, Lq, Lk), 0.5, device=device)
    raise ValueError(kind)


def index_sets(B: int, Lq: int, q_pos0: int, k: int, *, seed: int,
               pad_frac: float = 0.0, device: str = "cpu") -> torch.Tensor:
    """Random valid index lists [B,Lq,k] int32 for driving sparse attention.

    Row i (absolute position t = q_pos0 + i) holds min(k, t+1) distinct
    positions drawn uniformly without replacement from [0, t], in random order,
    followed by -1 padding. With pad_frac > 0 a further random fraction of each
    row's tail is replaced by -1 (at least one valid entry is kept).
    """
    g = _gen(seed, "cpu")
    out = torch.full((B, Lq, k), -1, dtype=torch.int32)
    for b in range(B):
        for i in range(Lq):
            t = q_pos0 + i
            n = min(k, t + 1)
            if t + 1 <= 4 * k:
                perm = torch.randperm(t + 1, generator=g)[:n]
            else:
                # rejection-free: sample a few more than needed, dedupe, trim
                perm = torch.empty(0, dtype=torch.int64)
                while perm.numel() < n:
                    cand = torch.randint(0, t + 1, (2 * n,), generator=g)
                    perm = torch.unique(torch.cat([perm, cand]))
                    perm = perm[torch.randperm(perm.numel(), generator=g)]
                perm = perm[:n]
            if pad_frac > 0.0 and n > 1:
                keep = max(1, int(round(n * (1.0 - pad_frac))))
                perm = perm[:keep]
            out[b, i, : perm.numel()] = perm.to(torch.int32)
    return out.to(device)


def to_f64(t: torch.Tensor):
    """Exact host fp64 numpy copy of a bf16/fp32 tensor (for the oracle)."""
    return t.detach().to("cpu").to(torch.float64).numpy()
