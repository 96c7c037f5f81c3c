"""IndexCache hot path on AMD MI355X: Python binding of libidxc.so.

Each function marshals torch tensors (device memory and the current stream)
into one call of the C ABI of the same name (include/idxc.h); every step of
the computation runs in the library's HIP kernels. Nothing here computes.
"""
from __future__ import annotations

import ctypes
from typing import Dict, List, Optional, Sequence

import torch

from . import _lib
from ._lib import IdxcDims, IdxcError, IdxcLayer

__all__ = ["idxc_version", "idxc_validate_pattern", "idxc_schedule", "idxc_indexer_scores",
           "idxc_topk", "idxc_topk_workspace_bytes", "idxc_workspace_bytes", "idxc_indexer_topk", "idxc_sparse_attn", "idxc_sparse_attn_workspace_bytes", "idxc_overlap",
           "idxc_layer_stack_forward", "idxc_overlap_matrix", "idxc_greedy_pattern",
           "idxc_overlap_proxy_loss", "idxc_indexer_topk_ragged",
           "idxc_layer_stack_forward_ragged", "idxc_layer_stack_forward_noalloc",
           "idxc_distill_loss", "make_dims", "IdxcError",
           "StackCall"]


def _stream(stream=None) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None) -> ctypes.c_void_p:
    if t is None:
        return ctypes.c_void_p(0)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return ctypes.c_void_p(t.data_ptr())


def make_dims(B, Lq, Lk, q_pos0=0, H_I=0, d_I=0, H=0, D=0, k=0) -> IdxcDims:
    return IdxcDims(int(B), int(Lq), int(Lk), int(q_pos0), int(H_I), int(d_I), int(H),
                    int(D), int(k))


def _idx_dims(q_idx, k_idx, q_pos0, k=0) -> IdxcDims:
    B, Lq, H_I, d_I = q_idx.shape
    return make_dims(B, Lq, k_idx.shape[1], q_pos0, H_I, d_I, 0, 0, k)


def idxc_version() -> str:
    return _lib.load().idxc_version().decode()


def idxc_validate_pattern(pattern: str) -> int:
    """Returns the number of F layers; raises IdxcError for a bad pattern."""
    lib = _lib.load()
    nf = ctypes.c_int32(0)
    _lib.check(lib.idxc_validate_pattern(pattern.encode(), len(pattern), ctypes.byref(nf)))
    return nf.value


def idxc_schedule(pattern: str) -> List[int]:
    """source[l] = l for F layers, f(l) for S layers (host only)."""
    lib = _lib.load()
    arr = (ctypes.c_int32 * max(1, len(pattern)))()
    _lib.check(lib.idxc_schedule(pattern.encode(), len(pattern), arr))
    return list(arr[: len(pattern)])


def idxc_indexer_scores(q_idx, k_idx, w, q_pos0: int = 0, out=None, stream=None):
    lib = _lib.load()
    d = _idx_dims(q_idx, k_idx, q_pos0)
    if out is None:
        out = torch.empty((d.B, d.Lq, d.Lk), dtype=torch.float32, device=q_idx.device)
    _lib.check(lib.idxc_indexer_scores(_ptr(q_idx, "q_idx", torch.bfloat16),
                                       _ptr(k_idx, "k_idx", torch.bfloat16),
                                       _ptr(w, "w", torch.bfloat16), ctypes.byref(d),
                                       _ptr(out, "scores", torch.float32), _stream(stream)))
    return out


def idxc_topk_workspace_bytes(B, Lq, Lk, q_pos0, k) -> int:
    lib = _lib.load()
    d = make_dims(B, Lq, Lk, q_pos0, k=k)
    n = ctypes.c_size_t(0)
    _lib.check(lib.idxc_topk_workspace_bytes(ctypes.byref(d), ctypes.byref(n)))
    return n.value


_ORDERS = {"score": _lib.IDXC_ORDER_SCORE, "position": _lib.IDXC_ORDER_POSITION}


def _order(order) -> int:
    if order not in _ORDERS:
        raise ValueError("order must be 'score' or 'position', not %r" % (order,))
    return _ORDERS[order]


def idxc_topk(scores, k: int, q_pos0: int = 0, workspace=None, out=None, stream=None,
              order: str = "score"):
    lib = _lib.load()
    B, Lq, Lk = scores.shape
    d = make_dims(B, Lq, Lk, q_pos0, k=k)
    if workspace is None:
        nb = idxc_topk_workspace_bytes(B, Lq, Lk, q_pos0, k)
        workspace = _workspace(nb, scores.device) if nb else None
    if out is None:
        out = torch.empty((B, Lq, k), dtype=torch.int32, device=scores.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _lib.check(lib.idxc_topk(_ptr(scores, "scores", torch.float32), ctypes.byref(d),
                             _order(order), _ptr(workspace, "workspace"), nbytes,
                             _ptr(out, "indices", torch.int32), _stream(stream)))
    return out


def idxc_workspace_bytes(B, Lq, Lk, q_pos0, H_I, d_I, k, H=0, D=0) -> int:
    lib = _lib.load()
    d = make_dims(B, Lq, Lk, q_pos0, H_I, d_I, H, D, k)
    n = ctypes.c_size_t(0)
    _lib.check(lib.idxc_workspace_bytes(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty((max(nbytes, 256),), dtype=torch.uint8, device=device)


def _indexer_topk(q_idx, k_idx, w, k, q_pos0, q_pos, workspace, out, stream, order):
    lib = _lib.load()
    d = _idx_dims(q_idx, k_idx, q_pos0, k)
    if workspace is None:
        workspace = _workspace(idxc_workspace_bytes(d.B, d.Lq, d.Lk, q_pos0, d.H_I, d.d_I, k),
                               q_idx.device)
    if out is None:
        out = torch.empty((d.B, d.Lq, k), dtype=torch.int32, device=q_idx.device)
    args = [_ptr(q_idx, "q_idx", torch.bfloat16), _ptr(k_idx, "k_idx", torch.bfloat16),
            _ptr(w, "w", torch.bfloat16), ctypes.byref(d)]
    tail = [_order(order), _ptr(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _ptr(out, "indices", torch.int32),
            _stream(stream)]
    if q_pos is None:
        _lib.check(lib.idxc_indexer_topk(*args, *tail))
    else:
        _lib.check(lib.idxc_indexer_topk_ragged(*args, _ptr(q_pos, "q_pos", torch.int32), *tail))
    return out


def idxc_indexer_topk(q_idx, k_idx, w, k: int, q_pos0: int = 0, workspace=None, out=None,
                      stream=None, order: str = "score"):
    return _indexer_topk(q_idx, k_idx, w, k, q_pos0, None, workspace, out, stream, order)


def idxc_indexer_topk_ragged(q_idx, k_idx, w, k: int, q_pos, workspace=None, out=None,
                             stream=None, order: str = "score"):
    """Row r = b*Lq + i at absolute position q_pos[b, i] (int32 [B, Lq] on the
    device; negative = no candidates); keys padded to the longest sequence."""
    return _indexer_topk(q_idx, k_idx, w, k, 0, q_pos, workspace, out, stream, order)


def idxc_sparse_attn_workspace_bytes(B, Lq, Lk, H, D, k) -> int:
    lib = _lib.load()
    d = make_dims(B, Lq, Lk, 0, 0, 0, H, D, k)
    n = ctypes.c_size_t(0)
    _lib.check(lib.idxc_sparse_attn_workspace_bytes(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def idxc_sparse_attn(q, k, v, indices, scale: float, workspace="auto", out=None, stream=None):
    """workspace: "auto" (allocate what a split needs), None (no split) or a tensor."""
    lib = _lib.load()
    B, Lq, H, D = q.shape
    d = make_dims(B, Lq, k.shape[1], 0, 0, 0, H, D, indices.shape[-1])
    if isinstance(workspace, str):
        nb = idxc_sparse_attn_workspace_bytes(B, Lq, k.shape[1], H, D, indices.shape[-1])
        workspace = _workspace(nb, q.device) if nb else None
    if out is None:
        out = torch.empty_like(q)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _lib.check(lib.idxc_sparse_attn(_ptr(q, "q", torch.bfloat16), _ptr(k, "k", torch.bfloat16),
                                    _ptr(v, "v", torch.bfloat16),
                                    _ptr(indices, "indices", torch.int32), ctypes.byref(d),
                                    float(scale), _ptr(workspace, "workspace"), nbytes,
                                    _ptr(out, "out", torch.bfloat16), _stream(stream)))
    return out


def idxc_layer_stack_forward(pattern: str, layers: Sequence[Dict[str, torch.Tensor]], k: int,
                             scale: float, q_pos0: int = 0, index_cache=None, workspace=None,
                             debug_indices: bool = False, stream=None):
    """Run the stack. layers[l] holds q_idx, k_idx, w (F layers), q, k, v and
    optionally out. Returns dict(out=[...], indexer_calls=int,
    index_cache=tensor, debug_indices=tensor or None)."""
    return _stack(pattern, layers, k, scale, q_pos0, None, index_cache, workspace,
                  debug_indices, stream)


def idxc_layer_stack_forward_ragged(pattern: str, layers: Sequence[Dict[str, torch.Tensor]],
                                    k: int, scale: float, q_pos, index_cache=None,
                                    workspace=None, debug_indices: bool = False, stream=None):
    """The stack with per-row query positions q_pos (int32 [B, Lq] on the device)."""
    return _stack(pattern, layers, k, scale, 0, q_pos, index_cache, workspace, debug_indices,
                  stream)


def idxc_layer_stack_forward_noalloc(pattern: str, layers: Sequence[Dict[str, torch.Tensor]],
                                     k: int, scale: float, q_pos0: int = 0, index_cache=None,
                                     debug_indices: bool = False, stream=None):
    """The stack without a workspace: its scratch is the library's static
    per-GPU array (sizes beyond it raise IdxcError). Same return value as
    idxc_layer_stack_forward."""
    return _stack(pattern, layers, k, scale, q_pos0, None, index_cache, None, debug_indices,
                  stream, noalloc=True)


def _stack(pattern, layers, k, scale, q_pos0, q_pos, index_cache, workspace, debug_indices,
           stream, noalloc=False):
    lib = _lib.load()
    n = len(layers)
    ref = next(L for L in layers if L.get("q") is not None)
    B, Lq, H, D = ref["q"].shape
    Lk = ref["k"].shape[1]
    f0 = next((L for L in layers if L.get("q_idx") is not None), None)
    H_I, d_I = (f0["q_idx"].shape[2], f0["q_idx"].shape[3]) if f0 is not None else (0, 0)
    d = make_dims(B, Lq, Lk, q_pos0, H_I, d_I, H, D, k)
    dev = ref["q"].device
    if index_cache is None:
        index_cache = torch.empty((B, Lq, k), dtype=torch.int32, device=dev)
    if workspace is None and not noalloc:
        workspace = _workspace(idxc_workspace_bytes(B, Lq, Lk, q_pos0, H_I, d_I, k, H, D), dev)
    dbg = torch.empty((n, B, Lq, k), dtype=torch.int32, device=dev) if debug_indices else None
    arr = (IdxcLayer * n)()
    outs = []
    for l, L in enumerate(layers):
        o = L.get("out")
        if o is None:
            o = torch.empty_like(L["q"])
        outs.append(o)
        arr[l] = IdxcLayer(_ptr(L.get("q_idx"), "q_idx", torch.bfloat16).value,
                           _ptr(L.get("k_idx"), "k_idx", torch.bfloat16).value,
                           _ptr(L.get("w"), "w", torch.bfloat16).value,
                           _ptr(L["q"], "q", torch.bfloat16).value,
                           _ptr(L["k"], "k", torch.bfloat16).value,
                           _ptr(L["v"], "v", torch.bfloat16).value,
                           _ptr(o, "out", torch.bfloat16).value)
    calls = ctypes.c_int32(-1)
    head = [pattern.encode(), n, arr, ctypes.byref(d)]
    if noalloc:
        _lib.check(lib.idxc_layer_stack_forward_noalloc(
            *head, float(scale), _ptr(index_cache, "index_cache"), ctypes.byref(calls),
            _ptr(dbg, "debug_indices"), _stream(stream)))
        return dict(out=outs, indexer_calls=calls.value, index_cache=index_cache,
                    debug_indices=dbg)
    tail = [float(scale), _ptr(index_cache, "index_cache"), _ptr(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), ctypes.byref(calls),
            _ptr(dbg, "debug_indices"), _stream(stream)]
    if q_pos is None:
        _lib.check(lib.idxc_layer_stack_forward(*head, *tail))
    else:
        _lib.check(lib.idxc_layer_stack_forward_ragged(*head, _ptr(q_pos, "q_pos", torch.int32),
                                                       *tail))
    return dict(out=outs, indexer_calls=calls.value, index_cache=index_cache,
                debug_indices=dbg)


def idxc_overlap(a, b, Lk: int, stream=None):
    """Per-row |A ∩ B|, overlap |A ∩ B| / |A| and Jaccard |A ∩ B| / |A ∪ B| of two
    [B, Lq, k] int32 index tensors (valid entries as sets, -1 ignored).
    Returns (inter int32 [B, Lq], overlap fp32 [B, Lq], jaccard fp32 [B, Lq])."""
    lib = _lib.load()
    if a.shape != b.shape or a.dim() != 3:
        raise ValueError("a and b must be [B, Lq, k] tensors of one shape")
    B, Lq, k = a.shape
    d = make_dims(B, Lq, Lk, Lk - Lq, k=k)
    dev = a.device
    inter = torch.empty((B, Lq), dtype=torch.int32, device=dev)
    ov = torch.empty((B, Lq), dtype=torch.float32, device=dev)
    jac = torch.empty((B, Lq), dtype=torch.float32, device=dev)
    _lib.check(lib.idxc_overlap(_ptr(a, "a", torch.int32), _ptr(b, "b", torch.int32),
                                ctypes.byref(d), _ptr(inter, "inter"), _ptr(ov, "overlap"),
                                _ptr(jac, "jaccard"), _stream(stream)))
    return inter, ov, jac


def idxc_overlap_matrix(sel, Lk: int, workspace=None, stream=None):
    """Mean overlap of every pair of layers: sel is an int32 [n_layers, B, Lq, k]
    tensor (for instance every layer's own top-k); returns fp32 [n_layers,
    n_layers] on the device with M[a, b] = mean over rows of |A ∩ B| / |A|."""
    lib = _lib.load()
    if sel.dim() != 4:
        raise ValueError("sel must be an [n_layers, B, Lq, k] tensor")
    n, B, Lq, k = sel.shape
    d = make_dims(B, Lq, Lk, Lk - Lq, k=k)
    need = int(lib.idxc_overlap_matrix_workspace_bytes(n))
    if workspace is None:
        workspace = _workspace(max(need, 16), sel.device)
    m = torch.empty((n, n), dtype=torch.float32, device=sel.device)
    _lib.check(lib.idxc_overlap_matrix(_ptr(sel, "sel", torch.int32), n, ctypes.byref(d),
                                       _ptr(workspace, "workspace"),
                                       workspace.numel() * workspace.element_size(),
                                       _ptr(m, "matrix"), _stream(stream)))
    return m


def idxc_greedy_pattern(n_layers: int, removals: int, loss):
    """Greedy F->S search of the C driver; loss(pattern: str) -> float is
    called for every trial. Returns (pattern, number of loss calls)."""
    lib = _lib.load()
    errors = []

    def call(pattern, _user):
        try:
            return float(loss(pattern.decode("ascii")))
        except Exception as e:  # surfaced after the C call returns
            errors.append(e)
            return float("nan")

    fn = _lib.LOSS_FN(call)
    buf = ctypes.create_string_buffer(n_layers + 1)
    evals = ctypes.c_int64(0)
    code = lib.idxc_greedy_pattern(n_layers, removals, fn, None, buf, ctypes.byref(evals))
    if errors:
        raise errors[0]
    _lib.check(code)
    return buf.value.decode("ascii"), int(evals.value)


def idxc_overlap_proxy_loss(pattern: str, matrix) -> float:
    """(1 / n) * sum over S layers l of (1 - M[l, f(l)]) for a host copy of an
    idxc_overlap_matrix result (numpy array or tensor, [n, n])."""
    lib = _lib.load()
    if isinstance(matrix, torch.Tensor):
        matrix = matrix.detach().to("cpu", torch.float32).numpy()
    import numpy as np
    m = np.ascontiguousarray(np.asarray(matrix, dtype=np.float32))
    n = len(pattern)
    if m.shape != (n, n):
        raise ValueError("matrix must be [n_layers, n_layers]")
    out = ctypes.c_double(0.0)
    _lib.check(lib.idxc_overlap_proxy_loss(pattern.encode("ascii"), n,
                                           m.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                                           ctypes.byref(out)))
    return float(out.value)


def idxc_distill_loss(logits, teachers, q_pos0: int = 0, grad: bool = True, stream=None):
    """Multi-teacher distillation loss per query row and its gradient with
    respect to the logits. logits fp32 [B, Lq, Lk]; teachers fp32 [n, B, Lq,
    Lk]. Returns (row_loss [B, Lq], grad [B, Lq, Lk] or None)."""
    lib = _lib.load()
    if logits.dim() != 3 or teachers.dim() != 4 or teachers.shape[1:] != logits.shape:
        raise ValueError("logits [B, Lq, Lk] and teachers [n, B, Lq, Lk] expected")
    B, Lq, Lk = logits.shape
    d = make_dims(B, Lq, Lk, q_pos0)
    loss = torch.empty((B, Lq), dtype=torch.float32, device=logits.device)
    g = torch.empty_like(logits) if grad else None
    _lib.check(lib.idxc_distill_loss(_ptr(logits, "logits", torch.float32),
                                     _ptr(teachers, "teachers", torch.float32),
                                     teachers.shape[0], ctypes.byref(d), _ptr(loss, "row_loss"),
                                     _ptr(g, "grad"), _stream(stream)))
    return loss, g


class StackCall:
    """idxc_layer_stack_forward with its arguments marshalled once.

    Holds references to every tensor it points at; calling it runs the whole
    stack on the given stream and returns the number of indexer launches.
    """

    def __init__(self, pattern: str, layers: Sequence[Dict[str, torch.Tensor]], k: int,
                 scale: float, q_pos0: int = 0, index_cache=None, workspace=None):
        self._lib = _lib.load()
        self.layers = layers
        n = len(layers)
        ref = next(L for L in layers if L.get("q") is not None)
        B, Lq, H, D = ref["q"].shape
        Lk = ref["k"].shape[1]
        f0 = next(L for L in layers if L.get("q_idx") is not None)
        H_I, d_I = f0["q_idx"].shape[2], f0["q_idx"].shape[3]
        dev = ref["q"].device
        self.dims = make_dims(B, Lq, Lk, q_pos0, H_I, d_I, H, D, k)
        self.index_cache = index_cache if index_cache is not None else torch.empty(
            (B, Lq, k), dtype=torch.int32, device=dev)
        self.workspace = workspace if workspace is not None else _workspace(
            idxc_workspace_bytes(B, Lq, Lk, q_pos0, H_I, d_I, k, H, D), dev)
        self.arr = (IdxcLayer * n)()
        for l, L in enumerate(layers):
            self.arr[l] = IdxcLayer(_ptr(L.get("q_idx"), "q_idx", torch.bfloat16).value,
                                    _ptr(L.get("k_idx"), "k_idx", torch.bfloat16).value,
                                    _ptr(L.get("w"), "w", torch.bfloat16).value,
                                    _ptr(L["q"], "q", torch.bfloat16).value,
                                    _ptr(L["k"], "k", torch.bfloat16).value,
                                    _ptr(L["v"], "v", torch.bfloat16).value,
                                    _ptr(L["out"], "out", torch.bfloat16).value)
        self.pattern = pattern.encode()
        self.n = n
        self.scale = float(scale)
        self.calls = ctypes.c_int32(-1)
        self.cache_ptr = _ptr(self.index_cache, "index_cache")
        self.ws_ptr = _ptr(self.workspace, "workspace")
        self.ws_bytes = self.workspace.numel() * self.workspace.element_size()

    def __call__(self, stream=None) -> int:
        _lib.check(self._lib.idxc_layer_stack_forward(
            self.pattern, self.n, self.arr, ctypes.byref(self.dims), self.scale,
            self.cache_ptr, self.ws_ptr, self.ws_bytes, ctypes.byref(self.calls), None,
            _stream(stream)))
        return self.calls.value
