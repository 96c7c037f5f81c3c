"""CPU-side tests of libidxc.so: it loads, exports every symbol that
include/idxc.h declares, and its host-only logic and argument checks work
without a GPU (every error path returns before any HIP call)."""
import ctypes
import itertools
import os
import re

import pytest

import oracle
from dsa_lightning_indexer_score_amd import _lib
from dsa_lightning_indexer_score_amd._lib import IdxcDims, IdxcLayer

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "idxc.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libidxc.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(idxc_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    decl = declared_functions()
    assert set(decl) == set(_lib.EXPORTED)
    for name in decl:
        assert hasattr(lib, name), name
    assert lib.idxc_version().decode().startswith("idxc")


def test_validate_pattern_matches_oracle(lib):
    for n in range(1, 7):
        for pat in itertools.product("FSX", repeat=n):
            p = "".join(pat)
            nf = ctypes.c_int32(-1)
            code = lib.idxc_validate_pattern(p.encode(), n, ctypes.byref(nf))
            try:
                oracle.validate_pattern(p, n)
                want_ok = True
            except ValueError:
                want_ok = False
            assert (code == 0) == want_ok, p
            if want_ok:
                assert nf.value == p.count("F")
            else:
                assert code == _lib.IDXC_ERR_PATTERN
                assert lib.idxc_last_error().decode() != ""
    # length mismatch and NULL
    assert lib.idxc_validate_pattern(b"FSS", 4, None) == _lib.IDXC_ERR_PATTERN
    assert lib.idxc_validate_pattern(None, 4, None) == _lib.IDXC_ERR_INVALID_ARG


def test_schedule_matches_oracle_nearest_full(lib):
    for n in range(1, 11):
        for tail in itertools.product("FS", repeat=n - 1):
            p = "F" + "".join(tail)
            arr = (ctypes.c_int32 * n)()
            assert lib.idxc_schedule(p.encode(), n, arr) == 0
            assert list(arr) == oracle.nearest_full(p)


def _dims(**kw):
    base = dict(B=1, Lq=64, Lk=64, q_pos0=0, H_I=4, d_I=32, H=4, D=64, k=16)
    base.update(kw)
    return IdxcDims(*[base[n] for n, _ in IdxcDims._fields_])


FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails its checks first


def P(x=FAKE):
    return ctypes.c_void_p(x)


def test_indexer_scores_argument_errors(lib):
    f = lib.idxc_indexer_scores
    ok = _dims()
    assert f(None, P(), P(), ctypes.byref(ok), P(), None) == _lib.IDXC_ERR_INVALID_ARG
    assert f(P(FAKE + 2), P(), P(), ctypes.byref(ok), P(), None) == _lib.IDXC_ERR_INVALID_ARG
    assert f(P(), P(), P(), None, P(), None) == _lib.IDXC_ERR_INVALID_ARG
    for bad, code in ((dict(Lq=0), 1), (dict(q_pos0=1), 1), (dict(Lk=10, Lq=11), 1),
                      (dict(d_I=48), 3), (dict(H_I=65), 3), (dict(H_I=0), 1),
                      (dict(q_pos0=-1), 1)):
        assert f(P(), P(), P(), ctypes.byref(_dims(**bad)), P(), None) == code, bad


def test_topk_argument_errors(lib):
    f = lambda s, d, ws, nb, out, st, order=0: lib.idxc_topk(s, d, order, ws, nb, out, st)
    assert f(P(), ctypes.byref(_dims(k=0)), None, 0, P(), None) == _lib.IDXC_ERR_INVALID_ARG
    assert f(P(), ctypes.byref(_dims(k=4096)), None, 0, P(), None) == _lib.IDXC_ERR_UNSUPPORTED
    assert f(None, ctypes.byref(_dims()), None, 0, P(), None) == _lib.IDXC_ERR_INVALID_ARG
    assert f(P(), ctypes.byref(_dims()), None, 0, P(FAKE + 4), None) == _lib.IDXC_ERR_INVALID_ARG
    for bad in (-1, 2, 7):
        assert f(P(), ctypes.byref(_dims()), None, 0, P(), None, bad) == _lib.IDXC_ERR_INVALID_ARG
        assert "order" in lib.idxc_last_error().decode()
    # rows of up to 65536 scores take one launch and no workspace; longer
    # ones need the chunked selection's
    n = ctypes.c_size_t(0)
    for Lk in (8193, 16384, 65536):
        fits = _dims(Lq=1, Lk=Lk, q_pos0=Lk - 1, k=2048)
        assert lib.idxc_topk_workspace_bytes(ctypes.byref(fits), ctypes.byref(n)) == 0
        assert n.value == 0
    long_rows = _dims(Lq=1, Lk=65537, q_pos0=65536, k=2048)
    assert lib.idxc_topk_workspace_bytes(ctypes.byref(long_rows), ctypes.byref(n)) == 0
    # one 2048-bin histogram of 16-bit counts per 8192-score chunk, and a
    # list of 16384 (key, position) pairs and a count per row
    assert n.value == 9 * 4096 + 16384 * 8 + 4
    assert f(P(), ctypes.byref(long_rows), None, 0, P(), None) == _lib.IDXC_ERR_INVALID_ARG
    assert f(P(), ctypes.byref(long_rows), P(), n.value - 1, P(), None) == _lib.IDXC_ERR_INVALID_ARG
    # rows of any length up to Lk = 2^24 are supported given the workspace
    longest = _dims(B=2, Lq=3, Lk=1 << 24, q_pos0=(1 << 24) - 3, k=2048)
    assert lib.idxc_topk_workspace_bytes(ctypes.byref(longest), ctypes.byref(n)) == 0
    assert n.value == 6 * 2048 * 4096 + 6 * (16384 * 8 + 4)
    assert f(P(), ctypes.byref(longest), P(), n.value - 16, P(), None) == _lib.IDXC_ERR_INVALID_ARG
    short = _dims(Lq=1, Lk=8192, q_pos0=8191, k=2048)
    assert lib.idxc_topk_workspace_bytes(ctypes.byref(short), ctypes.byref(n)) == 0
    assert n.value == 0


def test_sparse_attn_argument_errors(lib):
    f = lib.idxc_sparse_attn
    for bad, code in ((dict(D=96), 3), (dict(H=65), 3), (dict(k=0), 1), (dict(B=0), 1)):
        assert f(P(), P(), P(), P(), ctypes.byref(_dims(**bad)), 0.125, None, 0, P(), None) == code
    assert f(P(), None, P(), P(), ctypes.byref(_dims()), 0.125, None, 0, P(), None) == 1
    for bad_scale in (float("nan"), float("inf"), float("-inf"), 0.0, -0.0, -0.125):
        assert f(P(), P(), P(), P(), ctypes.byref(_dims()), bad_scale, None, 0, P(), None) == 1
        assert "scale" in lib.idxc_last_error().decode()
    # few rows: a split needs a workspace; a short one is rejected
    dec = _dims(B=64, Lq=1, Lk=65536, q_pos0=65535, H=64, D=128, k=2048)
    n = ctypes.c_size_t(0)
    assert lib.idxc_sparse_attn_workspace_bytes(ctypes.byref(dec), ctypes.byref(n)) == 0
    assert n.value > 64 * 64 * 128 * 2
    assert f(P(), P(), P(), P(), ctypes.byref(dec), 0.1, P(), 64, P(), None) == 1
    many = _dims(B=1, Lq=32768, Lk=32768, H=64, D=128, k=2048)
    assert lib.idxc_sparse_attn_workspace_bytes(ctypes.byref(many), ctypes.byref(n)) == 0
    assert n.value == 0


def test_workspace_and_fused_errors(lib):
    n = ctypes.c_size_t(0)
    assert lib.idxc_workspace_bytes(ctypes.byref(_dims()), ctypes.byref(n)) == 0
    assert n.value >= 64 * (8 * (16 + 64) + 4)
    f = lib.idxc_indexer_topk
    assert f(P(), P(), P(), ctypes.byref(_dims()), 0, P(), 16, P(), None) == \
        _lib.IDXC_ERR_INVALID_ARG
    assert "workspace" in lib.idxc_last_error().decode()
    assert f(P(), P(), P(), ctypes.byref(_dims()), 3, P(), 1 << 30, P(), None) == \
        _lib.IDXC_ERR_INVALID_ARG
    assert "order" in lib.idxc_last_error().decode()


def test_stack_errors_before_launch(lib):
    f = lib.idxc_layer_stack_forward
    layers = (IdxcLayer * 4)()
    for l in range(4):
        layers[l] = IdxcLayer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    d = _dims()
    calls = ctypes.c_int32(-7)
    args = lambda pat, n, ly=layers, dd=d, ws=1 << 30: (
        pat, n, ly, ctypes.byref(dd), 0.125, P(), P(), ws, ctypes.byref(calls), None, None)
    assert f(*args(b"SFSF", 4)) == _lib.IDXC_ERR_PATTERN
    assert f(*args(b"FSS", 4)) == _lib.IDXC_ERR_PATTERN
    assert f(*args(b"FSQF", 4)) == _lib.IDXC_ERR_PATTERN
    assert f(*args(None, 4)) == _lib.IDXC_ERR_INVALID_ARG
    assert f(*args(b"FSSF", 4, ws=8)) == _lib.IDXC_ERR_INVALID_ARG
    assert f(*args(b"FSSF", 4, dd=_dims(k=0))) == _lib.IDXC_ERR_INVALID_ARG
    for bad_scale in (float("nan"), float("inf"), 0.0, -1.0):
        a = list(args(b"FSSF", 4))
        a[4] = bad_scale
        assert f(*a) == _lib.IDXC_ERR_INVALID_ARG
        assert "scale" in lib.idxc_last_error().decode()
    # an F layer without indexer inputs is rejected, an S layer's are never read
    layers[3] = IdxcLayer(0, 0, 0, FAKE, FAKE, FAKE, FAKE)
    assert f(*args(b"FSSF", 4)) == _lib.IDXC_ERR_INVALID_ARG
    assert "layers[3].q_idx" in lib.idxc_last_error().decode()
    layers[2] = IdxcLayer(0, 0, 0, 0, FAKE, FAKE, FAKE)
    assert f(*args(b"FSSS", 4)) == _lib.IDXC_ERR_INVALID_ARG
    assert "layers[2].q" in lib.idxc_last_error().decode()
    assert calls.value == -7  # nothing ran


def test_overlap_argument_errors(lib):
    f = lib.idxc_overlap
    d = ctypes.byref(_dims(Lq=8, Lk=64, k=16))
    assert f(None, P(), d, P(), None, None, None) == _lib.IDXC_ERR_INVALID_ARG
    assert f(P(), P(FAKE + 2), d, P(), None, None, None) == _lib.IDXC_ERR_INVALID_ARG
    assert f(P(), P(), ctypes.byref(_dims(k=0)), P(), None, None, None) == \
        _lib.IDXC_ERR_INVALID_ARG
    big = ctypes.byref(_dims(Lq=1, Lk=262145, q_pos0=262144, k=16))
    assert f(P(), P(), big, P(), None, None, None) == _lib.IDXC_ERR_UNSUPPORTED
    # nothing requested: no launch
    assert f(P(), P(), d, None, None, None, None) == _lib.IDXC_OK


def _golden(name):
    import json
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        return json.load(f)


def test_greedy_driver_toy_example_and_forward_count():
    import dsa_lightning_indexer_score_amd as idxc
    g = _golden("greedy_toy.json")
    imp = g["importance"]
    pat, evals = idxc.idxc_greedy_pattern(
        g["n_layers"], g["removals"], lambda p: sum(v for r, v in zip(p, imp) if r == "S"))
    assert pat == g["expected_pattern"] and evals == 7
    for N, K, want in g["forward_count_cases"]:
        _, evals = idxc.idxc_greedy_pattern(N, K, lambda p: 0.0)
        assert evals == want


def test_greedy_driver_matches_oracle_on_proxy_losses():
    import numpy as np
    import dsa_lightning_indexer_score_amd as idxc
    rng = np.random.default_rng(7)
    for trial in range(20):
        n = int(rng.integers(2, 13))
        K = int(rng.integers(0, n))
        m = rng.random((n, n)).astype(np.float32)
        np.fill_diagonal(m, 1.0)
        if trial % 4 == 0:
            m[:] = np.round(m * 4) / 4  # many ties: the lower layer must win
        c_loss = lambda p: idxc.idxc_overlap_proxy_loss(p, m)
        o_loss = lambda p: oracle.overlap_proxy_loss(p, m.astype(np.float64))
        assert idxc.idxc_greedy_pattern(n, K, c_loss) == oracle.greedy_pattern(n, K, o_loss)
        for _ in range(5):
            p = "F" + "".join(rng.choice(["F", "S"], n - 1))
            assert idxc.idxc_overlap_proxy_loss(p, m) == pytest.approx(o_loss(p), abs=1e-12)


def test_greedy_and_proxy_errors(lib):
    import numpy as np
    import dsa_lightning_indexer_score_amd as idxc
    with pytest.raises(_lib.IdxcError):
        idxc.idxc_greedy_pattern(5, 5, lambda p: 0.0)
    with pytest.raises(_lib.IdxcError):
        idxc.idxc_greedy_pattern(5, -1, lambda p: 0.0)
    with pytest.raises(_lib.IdxcError):
        idxc.idxc_greedy_pattern(5, 2, lambda p: float("nan"))
    with pytest.raises(ZeroDivisionError):
        idxc.idxc_greedy_pattern(5, 2, lambda p: 1 / 0)
    buf = ctypes.create_string_buffer(6)
    fn = _lib.LOSS_FN(lambda p, u: 0.0)
    assert lib.idxc_greedy_pattern(5, 1, _lib.LOSS_FN(), None, buf, None) == \
        _lib.IDXC_ERR_INVALID_ARG
    assert lib.idxc_greedy_pattern(5, 1, fn, None, None, None) == _lib.IDXC_ERR_INVALID_ARG
    assert lib.idxc_greedy_pattern(5, 1, fn, None, buf, None) == _lib.IDXC_OK
    m = np.eye(3, dtype=np.float32)
    with pytest.raises(_lib.IdxcError):
        idxc.idxc_overlap_proxy_loss("SFF", m)
    out = ctypes.c_double(0.0)
    mp = m.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    assert lib.idxc_overlap_proxy_loss(b"FSF", 3, None, ctypes.byref(out)) == \
        _lib.IDXC_ERR_INVALID_ARG
    assert lib.idxc_overlap_proxy_loss(b"FSF", 4, mp, ctypes.byref(out)) == _lib.IDXC_ERR_PATTERN


def test_overlap_matrix_argument_errors(lib):
    f = lib.idxc_overlap_matrix
    d = ctypes.byref(_dims(Lq=8, Lk=64, k=16))
    assert lib.idxc_overlap_matrix_workspace_bytes(0) == 0
    assert lib.idxc_overlap_matrix_workspace_bytes(65) == 0
    assert lib.idxc_overlap_matrix_workspace_bytes(47) >= 47 * 47 * 8
    ws = lib.idxc_overlap_matrix_workspace_bytes(4)
    assert f(P(), 0, d, P(), ws, P(), None) == _lib.IDXC_ERR_INVALID_ARG
    assert f(P(), 65, d, P(), 1 << 20, P(), None) == _lib.IDXC_ERR_UNSUPPORTED
    assert f(None, 4, d, P(), ws, P(), None) == _lib.IDXC_ERR_INVALID_ARG
    assert f(P(), 4, d, P(), ws, None, None) == _lib.IDXC_ERR_INVALID_ARG
    assert f(P(), 4, d, P(FAKE + 8), ws, P(), None) == _lib.IDXC_ERR_INVALID_ARG
    assert f(P(FAKE + 2), 4, d, P(), ws, P(), None) == _lib.IDXC_ERR_INVALID_ARG
    assert f(P(), 4, d, P(), ws - 8, P(), None) == _lib.IDXC_ERR_INVALID_ARG
    big = ctypes.byref(_dims(Lq=1, Lk=262145, q_pos0=262144, k=16))
    assert f(P(), 4, big, P(), ws, P(), None) == _lib.IDXC_ERR_UNSUPPORTED
    assert f(P(), 4, ctypes.byref(_dims(k=0)), P(), ws, P(), None) == _lib.IDXC_ERR_INVALID_ARG


def test_ragged_argument_errors(lib):
    f = lib.idxc_indexer_topk_ragged
    d = ctypes.byref(_dims(Lq=8, Lk=64, k=16))
    # q_pos NULL or misaligned; then the usual checks of the uniform call
    assert f(P(), P(), P(), d, None, 0, P(), 1 << 30, P(), None) == _lib.IDXC_ERR_INVALID_ARG
    assert f(P(), P(), P(), d, P(FAKE + 4), 0, P(), 1 << 30, P(), None) == \
        _lib.IDXC_ERR_INVALID_ARG
    assert f(P(), P(), P(), d, P(), 7, P(), 1 << 30, P(), None) == _lib.IDXC_ERR_INVALID_ARG
    assert f(P(), P(), P(), d, P(), 0, P(), 16, P(), None) == _lib.IDXC_ERR_INVALID_ARG
    assert f(P(), P(), P(), ctypes.byref(_dims(d_I=48)), P(), 0, P(), 1 << 30, P(), None) == \
        _lib.IDXC_ERR_UNSUPPORTED
    g = lib.idxc_layer_stack_forward_ragged
    calls = ctypes.c_int32(0)
    layer = (IdxcLayer * 1)(IdxcLayer(*([FAKE] * 7)))
    assert g(b"F", 1, layer, d, None, 1.0, P(), P(), 1 << 30, ctypes.byref(calls), None,
             None) == _lib.IDXC_ERR_INVALID_ARG
    assert g(b"S", 1, layer, d, P(), 1.0, P(), P(), 1 << 30, ctypes.byref(calls), None,
             None) == _lib.IDXC_ERR_PATTERN


def test_distill_argument_errors(lib):
    f = lib.idxc_distill_loss
    d = ctypes.byref(_dims(Lq=8, Lk=64))
    assert f(P(), P(), 0, d, P(), P(), None) == _lib.IDXC_ERR_INVALID_ARG
    assert f(P(), P(), 65, d, P(), P(), None) == _lib.IDXC_ERR_UNSUPPORTED
    assert f(None, P(), 2, d, P(), P(), None) == _lib.IDXC_ERR_INVALID_ARG
    assert f(P(), None, 2, d, P(), P(), None) == _lib.IDXC_ERR_INVALID_ARG
    assert f(P(), P(), 2, d, P(FAKE + 4), P(), None) == _lib.IDXC_ERR_INVALID_ARG
    assert f(P(), P(), 2, d, P(), P(FAKE + 8), None) == _lib.IDXC_ERR_INVALID_ARG
    assert f(P(), P(), 2, ctypes.byref(_dims(Lq=8, Lk=4)), P(), P(), None) == \
        _lib.IDXC_ERR_INVALID_ARG
    assert f(P(), P(), 2, d, None, None, None) == _lib.IDXC_OK   # nothing requested: no launch


def test_noalloc_scratch_constant_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define\s+IDXC_NOALLOC_SCRATCH_BYTES\s+\(\(size_t\)(\d+)\s*<<\s*(\d+)\)", text)
    assert m, "IDXC_NOALLOC_SCRATCH_BYTES not found"
    assert int(m.group(1)) << int(m.group(2)) == _lib.NOALLOC_SCRATCH_BYTES


def test_noalloc_stack_checks_before_any_device_use(lib):
    f = lib.idxc_layer_stack_forward_noalloc
    layers = (IdxcLayer * 4)()
    for l in range(4):
        layers[l] = IdxcLayer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    calls = ctypes.c_int32(-7)

    def call(pat=b"FSSF", n=4, dd=None, scale=0.125, cache=P(), dbg=None):
        dd = dd if dd is not None else _dims()
        return f(pat, n, layers, ctypes.byref(dd), scale, cache, ctypes.byref(calls), dbg, None)

    assert call(pat=b"SFSF") == _lib.IDXC_ERR_PATTERN
    assert call(pat=b"FSS") == _lib.IDXC_ERR_PATTERN
    assert call(scale=0.0) == _lib.IDXC_ERR_INVALID_ARG
    assert call(cache=None) == _lib.IDXC_ERR_INVALID_ARG
    assert call(dbg=P(FAKE + 4)) == _lib.IDXC_ERR_INVALID_ARG
    # a 32768-token prefill needs far more scratch than the static array
    big = _dims(B=1, Lq=32768, Lk=32768, H_I=64, d_I=128, H=64, D=128, k=2048)
    assert call(dd=big) == _lib.IDXC_ERR_UNSUPPORTED
    msg = lib.idxc_last_error().decode()
    assert "scratch" in msg and str(_lib.NOALLOC_SCRATCH_BYTES) in msg
    # just above the limit: the smallest workspace is one byte too large
    n = ctypes.c_size_t(0)
    dec = _dims(B=64, Lq=1, Lk=65536, q_pos0=65535, H_I=64, d_I=128, H=64, D=128, k=2048)
    assert lib.idxc_workspace_bytes(ctypes.byref(dec), ctypes.byref(n)) == 0
    assert n.value <= _lib.NOALLOC_SCRATCH_BYTES  # the decode batch of the benchmark fits
    layers[1] = IdxcLayer(0, 0, 0, FAKE, FAKE, FAKE, FAKE)
    assert call(pat=b"FFSF") == _lib.IDXC_ERR_INVALID_ARG
    assert "layers[1].q_idx" in lib.idxc_last_error().decode()
    assert calls.value == -7  # nothing ran
