"""ctypes loader for libidxc.so (the C ABI declared in include/idxc.h).

The library is built in-tree by ``dsa_lightning_indexer_score_amd.build``.
There is no fallback: if the shared library is missing or cannot be loaded,
every entry point raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libidxc.so")

IDXC_OK = 0
IDXC_ERR_INVALID_ARG = 1
IDXC_ERR_PATTERN = 2
IDXC_ERR_UNSUPPORTED = 3
IDXC_ERR_HIP = 4
IDXC_ORDER_SCORE = 0
IDXC_ORDER_POSITION = 1

STATUS_NAMES = {
    IDXC_OK: "IDXC_OK",
    IDXC_ERR_INVALID_ARG: "IDXC_ERR_INVALID_ARG",
    IDXC_ERR_PATTERN: "IDXC_ERR_PATTERN",
    IDXC_ERR_UNSUPPORTED: "IDXC_ERR_UNSUPPORTED",
    IDXC_ERR_HIP: "IDXC_ERR_HIP",
}

# Every symbol declared in include/idxc.h.
EXPORTED = (
    "idxc_last_error", "idxc_version", "idxc_validate_pattern", "idxc_schedule",
    "idxc_indexer_scores", "idxc_topk", "idxc_topk_workspace_bytes", "idxc_workspace_bytes",
    "idxc_indexer_topk", "idxc_sparse_attn", "idxc_sparse_attn_workspace_bytes",
    "idxc_layer_stack_forward", "idxc_overlap", "idxc_overlap_matrix_workspace_bytes",
    "idxc_overlap_matrix", "idxc_greedy_pattern", "idxc_overlap_proxy_loss",
    "idxc_indexer_topk_ragged", "idxc_layer_stack_forward_ragged", "idxc_distill_loss",
    "idxc_layer_stack_forward_noalloc",
)

# bytes of the device-resident scratch of idxc_layer_stack_forward_noalloc
# (IDXC_NOALLOC_SCRATCH_BYTES in include/idxc.h)
NOALLOC_SCRATCH_BYTES = 64 << 20

# double loss(const char* pattern, void* user)
LOSS_FN = ctypes.CFUNCTYPE(ctypes.c_double, ctypes.c_char_p, ctypes.c_void_p)


class IdxcDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "Lq", "Lk", "q_pos0", "H_I", "d_I", "H", "D", "k")]


class IdxcLayer(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("q_idx", "k_idx", "w", "q", "k", "v", "out")]


class IdxcError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("%s: %s" % (STATUS_NAMES.get(code, str(code)), msg))
        self.code = code


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libidxc.so is not built (%s); run `python -m "
            "dsa_lightning_indexer_score_amd.build` first" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    P = ctypes.POINTER
    sigs = {
        "idxc_last_error": ([], ctypes.c_char_p),
        "idxc_version": ([], ctypes.c_char_p),
        "idxc_validate_pattern": ([ctypes.c_char_p, i32, P(i32)], ctypes.c_int),
        "idxc_schedule": ([ctypes.c_char_p, i32, P(i32)], ctypes.c_int),
        "idxc_indexer_scores": ([vp, vp, vp, P(IdxcDims), vp, vp], ctypes.c_int),
        "idxc_topk": ([vp, P(IdxcDims), ctypes.c_int32, vp, sz, vp, vp], ctypes.c_int),
        "idxc_topk_workspace_bytes": ([P(IdxcDims), P(sz)], ctypes.c_int),
        "idxc_workspace_bytes": ([P(IdxcDims), P(sz)], ctypes.c_int),
        "idxc_indexer_topk": ([vp, vp, vp, P(IdxcDims), ctypes.c_int32, vp, sz, vp, vp],
                              ctypes.c_int),
        "idxc_sparse_attn": ([vp, vp, vp, vp, P(IdxcDims), ctypes.c_float, vp, sz, vp, vp],
                             ctypes.c_int),
        "idxc_sparse_attn_workspace_bytes": ([P(IdxcDims), P(sz)], ctypes.c_int),
        "idxc_layer_stack_forward": ([ctypes.c_char_p, i32, P(IdxcLayer), P(IdxcDims),
                                      ctypes.c_float, vp, vp, sz, P(i32), vp, vp],
                                     ctypes.c_int),
        "idxc_overlap": ([vp, vp, P(IdxcDims), vp, vp, vp, vp], ctypes.c_int),
        "idxc_indexer_topk_ragged": ([vp, vp, vp, P(IdxcDims), vp, ctypes.c_int32, vp, sz, vp,
                                      vp], ctypes.c_int),
        "idxc_layer_stack_forward_ragged": ([ctypes.c_char_p, i32, P(IdxcLayer), P(IdxcDims), vp,
                                             ctypes.c_float, vp, vp, sz, P(i32), vp, vp],
                                            ctypes.c_int),
        "idxc_layer_stack_forward_noalloc": ([ctypes.c_char_p, i32, P(IdxcLayer), P(IdxcDims),
                                              ctypes.c_float, vp, P(i32), vp, vp],
                                             ctypes.c_int),
        "idxc_overlap_matrix_workspace_bytes": ([i32], sz),
        "idxc_distill_loss": ([vp, vp, i32, P(IdxcDims), vp, vp, vp], ctypes.c_int),
        "idxc_overlap_matrix": ([vp, i32, P(IdxcDims), vp, sz, vp, vp], ctypes.c_int),
        "idxc_greedy_pattern": ([i32, i32, LOSS_FN, vp, ctypes.c_char_p, P(ctypes.c_int64)],
                                ctypes.c_int),
        "idxc_overlap_proxy_loss": ([ctypes.c_char_p, i32, P(ctypes.c_float),
                                     P(ctypes.c_double)], ctypes.c_int),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def check(code: int) -> None:
    if code != IDXC_OK:
        msg = load().idxc_last_error().decode("utf-8", "replace")
        raise IdxcError(code, msg)
