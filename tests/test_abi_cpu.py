"""C ABI checks that need no GPU: exports, status codes, validation, workspace sizes.

Every call here fails validation, and validation precedes the first HIP call,
so nothing touches a device.
"""
import ctypes
import math
import os
import re

import pytest

from muon_step_03_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon.h")
ES = {_lib.MUON_DTYPE_F32: 4, _lib.MUON_DTYPE_BF16: 2}

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libmuon.so not built")


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(muon_[a-z_]+)\s*\(", text)))


def test_header_declares_what_binding_expects():
    assert header_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for name in header_functions():
        assert hasattr(L, name), name


def test_status_strings(L):
    names = {0: "ok", 1: "invalid argument", 2: "invalid shape", 3: "unsupported dtype",
             4: "workspace too small", 5: "HIP runtime error"}
    for code, text in names.items():
        assert _lib.status_string(code) == text
    assert _lib.status_string(99) == "unknown status"
    assert L.muon_last_hip_error() == 0


def ws_formula(count, rows, cols, dtype):
    """Workspace size from the layout the library documents (X0, X1, A, B,
    head/tail partials, per-matrix scalars (10), row/column partials, norms
    and per-256-row/column chunk statistics (5); 256-byte aligned regions)."""
    tile_p, tile_q = (128, 256) if dtype == _lib.MUON_DTYPE_BF16 else (64, 64)
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    p, q = min(rows, cols), max(rows, cols)
    pp = -(-p // tile_p) * tile_p
    if dtype == _lib.MUON_DTYPE_BF16 and pp == 512:
        tile_q = 128          # the 512x128 update tiles: long side padded to 128
    qp = -(-q // tile_q) * tile_q
    es = ES[dtype]
    head = (pp // 64) * (qp // 64)
    tail = math.ceil(rows / 64) * math.ceil(cols / 64)
    chunks = math.ceil(rows / 256) + math.ceil(cols / 256)
    return (2 * al(count * pp * qp * es) + 2 * al(count * pp * pp * es) + al(count * head * 8)
            + al(count * tail * 24) + al(count * 10 * 4) + al(count * tail * 128 * 4)
            + al(count * (rows + cols) * 4) + al(count * chunks * 5 * 4) + 256)


@pytest.mark.parametrize("shape", [(256, 512), (768, 3072), (3072, 768), (100, 300), (1, 1),
                                   (1408, 512), (512, 1408), (450, 777), (2048, 5632)])
@pytest.mark.parametrize("dtype", [_lib.MUON_DTYPE_F32, _lib.MUON_DTYPE_BF16])
@pytest.mark.parametrize("count", [1, 7])
def test_workspace_bytes(L, shape, dtype, count):
    assert L.muon_workspace_bytes(count, *shape, dtype) == ws_formula(count, *shape, dtype)


def test_workspace_bytes_invalid(L):
    assert L.muon_workspace_bytes(1, 0, 5, 0) == 0
    assert L.muon_workspace_bytes(1, 5, _lib.MUON_MAX_DIM + 1, 0) == 0
    assert L.muon_workspace_bytes(-1, 5, 5, 0) == 0
    assert L.muon_workspace_bytes(1, 5, 5, 7) == 0
    assert L.muon_workspace_bytes(0, 5, 5, 0) == 0


def test_workspace_bytes_grouped_is_sum(L):
    shapes = [(3, 768, 768), (2, 768, 3072), (2, 3072, 768)]
    arr = (_lib.MuonGroup * 3)(*[_lib.MuonGroup(c, r, k, None, None, None, 1, 2, 3)
                                 for c, r, k in shapes])
    got = L.muon_workspace_bytes_grouped(arr, 3, _lib.MUON_DTYPE_BF16)
    want = sum(ws_formula(c, r, k, _lib.MUON_DTYPE_BF16) - 256 for c, r, k in shapes) + 256
    assert got == want


# Fake device addresses: never dereferenced, since every call below fails
# validation first.
W, G, M, WS = 0x10000000, 0x20000000, 0x30000000, 0x40000000
OKARGS = dict(lr=0.02, mom=0.95, wd=0.1, ns=5, a=3.4445, b=-4.775, c=2.0315, variant=0)


def call_step(L, W=W, G=G, M=M, rows=64, cols=128, dtype=0, ws=WS, wsb=1 << 30, stats=None,
              **kw):
    k = dict(OKARGS, **kw)
    return L.muon_step(W, G, M, rows, cols, dtype, k["lr"], k["mom"], k["wd"], k["ns"], k["a"],
                       k["b"], k["c"], k["variant"], ws, wsb, stats, None)


@pytest.mark.parametrize("kw,status", [
    (dict(W=None), 1), (dict(G=None), 1), (dict(M=None), 1),
    (dict(rows=0), 2), (dict(cols=0), 2), (dict(rows=-3), 2),
    (dict(cols=_lib.MUON_MAX_DIM + 1), 2),
    (dict(dtype=2), 3), (dict(dtype=-1), 3),
    (dict(ns=-1), 1), (dict(ns=_lib.MUON_MAX_NS_STEPS + 1), 1),
    (dict(lr=float("nan")), 1), (dict(mom=float("inf")), 1), (dict(wd=float("-inf")), 1),
    (dict(a=float("nan")), 1), (dict(b=float("inf")), 1), (dict(c=float("nan")), 1),
    (dict(variant=5), 1), (dict(variant=-1), 1), (dict(variant=0x200), 1),
    (dict(variant=0x105), 1),
    (dict(ws=None), 1), (dict(wsb=1000), 4),
    (dict(G=W), 1),                          # W and G alias
    (dict(M=W + 64), 1),                     # M overlaps W
    (dict(ws=G - 1024, wsb=1 << 20), 1),     # workspace overlaps G
])
def test_step_validation(L, kw, status):
    assert call_step(L, **kw) == status


@pytest.mark.parametrize("variant", [0, 1, 2, 3, 4, 0x100, 0x101, 0x102, 0x103, 0x104])
def test_valid_variants_pass_validation(L, variant):
    """Valid variants get past argument checks (to the workspace check here)."""
    assert call_step(L, variant=variant, wsb=16) == _lib.MUON_ERR_WORKSPACE_TOO_SMALL


def test_workspace_exact_size_boundary(L):
    need = L.muon_workspace_bytes(1, 64, 128, 0)
    assert call_step(L, wsb=need - 1) == _lib.MUON_ERR_WORKSPACE_TOO_SMALL


def test_batched_validation(L):
    P = ctypes.c_void_p
    args = (0, 0.02, 0.95, 0.1, 5, 3.4445, -4.775, 2.0315, 0, WS, 1 << 30, None, None)
    assert L.muon_step_batched(None, P(G), P(M), 4, 64, 64, *args) == 1
    assert L.muon_step_batched(P(W), P(G), P(M), -1, 64, 64, *args) == 1
    assert L.muon_step_batched(P(W), P(G), P(M), 4, 0, 64, *args) == 2
    # Empty batch: a no-op, no workspace needed, nothing enqueued.
    assert L.muon_step_batched(None, None, None, 0, 64, 64, *args) == 0


def test_grouped_validation(L):
    args = (0, 0.02, 0.95, 0.1, 5, 3.4445, -4.775, 2.0315, 0, WS, 1 << 34, None, None)
    def grp(**kw):
        d = dict(count=2, rows=64, cols=64, W_table=None, G_table=None, M_table=None,
                 W=None, G=None, M=None)
        d.update(kw)
        return _lib.MuonGroup(**d)
    arr = lambda *g: (_lib.MuonGroup * len(g))(*g)  # noqa: E731
    # neither pointer form / both forms / a partial form
    assert L.muon_step_grouped(arr(grp()), 1, *args) == 1
    assert L.muon_step_grouped(arr(grp(W=W, G=G, M=M, W_table=1, G_table=2, M_table=3)), 1,
                               *args) == 1
    assert L.muon_step_grouped(arr(grp(W_table=1, G_table=2)), 1, *args) == 1
    assert L.muon_step_grouped(arr(grp(W=W, G=G)), 1, *args) == 1
    # stacks that overlap: 2 x 64 x 64 floats starting 1 KiB apart
    assert L.muon_step_grouped(arr(grp(W=W, G=W + 1024, M=M)), 1, *args) == 1
    assert L.muon_step_grouped(None, 1, *args) == 1
    assert L.muon_step_grouped(None, -1, *args) == 1
    # bad shape in a later group is still caught before any work
    good = grp(W=W, G=G, M=M)
    assert L.muon_step_grouped(arr(good, grp(rows=0, W=W, G=G, M=M)), 2, *args) == 2
    # empty: no groups, or only count-0 groups
    assert L.muon_step_grouped(None, 0, *args) == 0
    assert L.muon_step_grouped(arr(grp(count=0)), 1, *args) == 0
    # too many blocks for one launch
    huge = grp(count=1 << 20, rows=4096, cols=4096, W=W, G=G + (1 << 50), M=M + (1 << 52))
    assert L.muon_step_grouped(arr(huge), 1, *args) == 2


def test_phase_names_and_profile_args(L):
    names = [L.muon_phase_name(i).decode() for i in range(_lib.MUON_NUM_PHASES)]
    assert names == ["head", "norm_finalize", "gram", "poly", "update", "tail_reduce",
                     "tail_finalize", "tail_apply", "adamw", "update_tail"]
    assert L.muon_phase_name(10) == b"?" and L.muon_phase_name(-1) == b"?"
    assert L.muon_profile_read(None, None, 8) == 1
    ms = (ctypes.c_double * 8)()
    n = (ctypes.c_int64 * 8)()
    assert L.muon_profile_read(ms, n, 0) == 1
    # nothing recorded yet: reads back zeros without touching a device
    assert L.muon_profile_read(ms, n, 8) == 0 and sum(n) == 0


def test_python_binding_rejects_non_2d():
    torch = pytest.importorskip("torch")
    from muon_step_03_amd import MuonStep, muon_step
    with pytest.raises(ValueError):
        MuonStep([torch.nn.Parameter(torch.zeros(8))])
    with pytest.raises(ValueError):
        muon_step(torch.zeros(4, 4, 4), torch.zeros(4, 4, 4), torch.zeros(4, 4, 4))


# ------------------------------------------------------------ AdamW entry points
P_, G_, MM, VV = 0x50000000, 0x60000000, 0x70000000, 0x80000000
ADAM_OK = dict(lr=0.015, b1=0.8, b2=0.95, eps=1e-10, wd=1e-3, step=1)


def call_adamw(L, P=P_, G=G_, m=MM, v=VV, n=1000, dtype=1, **kw):
    k = dict(ADAM_OK, **kw)
    return L.muon_adamw_step(P, G, m, v, n, dtype, k["lr"], k["b1"], k["b2"], k["eps"], k["wd"],
                             k["step"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), 3), (dict(dtype=-1), 3),
    (dict(b1=1.0), 1), (dict(b1=-0.1), 1), (dict(b2=1.0), 1), (dict(b2=float("nan")), 1),
    (dict(eps=-1e-10), 1), (dict(eps=float("inf")), 1), (dict(step=0), 1), (dict(step=-3), 1),
    (dict(lr=float("nan")), 1), (dict(wd=float("inf")), 1),
    (dict(n=-1), 2), (dict(n=(1 << 40) + 1), 2),
    (dict(P=None), 1), (dict(G=None), 1), (dict(m=None), 1), (dict(v=None), 1),
    # overlapping buffers: G inside P (bf16: 2000 bytes), v inside m (4000 bytes)
    (dict(G=P_ + 1998), 1), (dict(v=MM + 3996), 1), (dict(m=G_), 1),
])
def test_adamw_validation(L, kw, status):
    assert call_adamw(L, **kw) == status


def test_adamw_empty_is_noop(L):
    """n == 0 (any pointers) and an empty group enqueue nothing."""
    assert call_adamw(L, n=0, P=None, G=None, m=None, v=None) == 0
    assert L.muon_adamw_step_grouped(None, 0, 1, 0.8, 0.95, 1e-10, 1, None) == 0


def test_adamw_grouped_validation(L):
    T = _lib.AdamwTensor
    arr = lambda *t: (T * len(t))(*t)  # noqa: E731
    a = T(P_, G_, MM, VV, 1000, 0.7, 1e-3)
    b = T(P_ + 4096, G_ + 4096, MM + 8192, VV + 8192, 1000, 0.004, 1e-3)
    args = (1, 0.8, 0.95, 1e-10, 1, None)
    assert L.muon_adamw_step_grouped(None, 2, *args) == 1
    assert L.muon_adamw_step_grouped(arr(a, b), -1, *args) == 1
    # one tensor's v overlaps the other's m
    c = T(P_ + 4096, G_ + 4096, MM + 8192, MM + 100, 1000, 0.004, 1e-3)
    assert L.muon_adamw_step_grouped(arr(a, c), 2, *args) == 1
    # the same tensor twice aliases every buffer
    assert L.muon_adamw_step_grouped(arr(a, a), 2, *args) == 1
    bad = T(P_ + 4096, G_ + 4096, MM + 8192, VV + 8192, 1000, float("nan"), 1e-3)
    assert L.muon_adamw_step_grouped(arr(a, bad), 2, *args) == 1
    # disjoint tensors with n == 0 entries: only the scalars fail here
    z = T(None, None, None, None, 0, 0.1, 0.0)
    assert L.muon_adamw_step_grouped(arr(z, a, b), 3, 1, 1.5, 0.95, 1e-10, 1, None) == 1
    assert L.muon_adamw_step_grouped(arr(z, a, b), 3, 7, 0.8, 0.95, 1e-10, 1, None) == 3


def test_adamw_python_binding_checks():
    torch = pytest.importorskip("torch")
    from muon_step_03_amd import AdamWStep, adamw_tensor
    with pytest.raises(ValueError):   # CPU tensors are rejected before any library call
        adamw_tensor(torch.zeros(4), torch.zeros(4), torch.zeros(4), torch.zeros(4), lr=0.1)
    with pytest.raises(ValueError):
        AdamWStep([dict(params=[torch.nn.Parameter(torch.zeros(4))], lr=0.1)])


def test_aux_workload_matches_page_hyperparameters():
    """The binding's AdamW defaults are the oracle's (pinned to the pages)."""
    import oracle
    from muon_step_03_amd import api
    assert api.AUX_BETAS == oracle.AUX_BETAS and api.AUX_EPS == oracle.AUX_EPS
    assert api.AUX_WEIGHT_DECAY == oracle.AUX_WEIGHT_DECAY and api.AUX_LR == oracle.AUX_LR


# ------------------------------------------ chunking a model under a budget
def _need(shapes, c):
    import torch
    from muon_step_03_amd import workspace_bytes_grouped
    return workspace_bytes_grouped([_lib.MuonGroup(min(c, n), r, k, None, None, None, None,
                                                   None, None) for n, r, k in shapes],
                                   torch.bfloat16)


@pytest.mark.parametrize("budget_gib", [0.5, 4, 16, 32, 48, 200])
def test_chunk_size_fewest_even_calls(budget_gib):
    """The chunk fits the budget, no smaller number of calls would, and the
    chunks are as even as that number of calls allows."""
    import torch
    from muon_step_03_amd import chunk_size
    shapes = [(1024, 2048, 5632), (1024, 5632, 2048)]
    budget = int(budget_gib * 2**30)
    c = chunk_size(shapes, torch.bfloat16, budget)
    calls = math.ceil(1024 / c)
    assert _need(shapes, c) <= budget
    assert c == math.ceil(1024 / calls)
    if calls > 1:
        assert _need(shapes, math.ceil(1024 / (calls - 1))) > budget
    else:
        assert c == 1024


def test_chunk_size_whole_model_and_errors():
    import torch
    from muon_step_03_amd import chunk_size
    shapes = [(48, 768, 768), (12, 768, 3072), (12, 3072, 768)]
    assert chunk_size(shapes, torch.bfloat16, 1 << 40) == 48
    assert chunk_size(shapes, torch.bfloat16, _need(shapes, 48)) == 48
    assert chunk_size(shapes, torch.bfloat16, _need(shapes, 48) - 1) == 24
    with pytest.raises(ValueError):
        chunk_size(shapes, torch.bfloat16, _need(shapes, 1) - 1)
    with pytest.raises(ValueError):
        chunk_size([], torch.bfloat16, 1 << 30)


def test_stats_buffer_checks():
    """The binding refuses a statistics buffer the library would write past
    (MUON_STATS_PER_MATRIX floats per matrix, no bounds on the device), of the
    wrong dtype, non-contiguous or on the host."""
    import torch
    from muon_step_03_amd.api import check_stats
    check_stats(None, 7)
    with pytest.raises(ValueError, match="needed"):
        check_stats(torch.zeros(2 * _lib.MUON_STATS_PER_MATRIX - 1), 2)
    with pytest.raises(ValueError, match="float32"):
        check_stats(torch.zeros(10, dtype=torch.float64), 2)
    with pytest.raises(ValueError, match="contiguous"):
        check_stats(torch.zeros(20)[::2], 2)
    with pytest.raises(ValueError, match="GPU"):
        check_stats(torch.zeros(10), 2)
    with pytest.raises(TypeError):
        check_stats([0.0] * 10, 2)


def test_noalloc_validation(L):
    """muon_step_grouped_noalloc validates like muon_step_grouped and refuses
    groups whose workspace exceeds its static array, before any HIP call."""
    def call(groups, dtype=1, ns=5, variant=0):
        arr = (_lib.MuonGroup * max(1, len(groups)))(*groups)
        return L.muon_step_grouped_noalloc(arr, len(groups), dtype, 0.02, 0.95, 0.1, ns,
                                           3.4445, -4.775, 2.0315, variant, None, None)
    big = _lib.MuonGroup(8, 1024, 4096, None, None, None, W, G, M)
    assert L.muon_workspace_bytes_grouped((_lib.MuonGroup * 1)(big), 1, 1) > \
        _lib.MUON_NOALLOC_WORKSPACE_BYTES
    assert call([big]) == _lib.MUON_ERR_WORKSPACE_TOO_SMALL
    assert call([big], dtype=7) == _lib.MUON_ERR_UNSUPPORTED_DTYPE
    assert call([big], ns=-1) == _lib.MUON_ERR_INVALID_ARGUMENT
    assert call([_lib.MuonGroup(1, 0, 5, None, None, None, W, G, M)]) == _lib.MUON_ERR_INVALID_SHAPE
    assert call([_lib.MuonGroup(0, 5, 5, None, None, None, None, None, None)]) == _lib.MUON_OK
    assert call([]) == _lib.MUON_OK


def test_trace_ranges_load_roctx_and_keep_validation():
    """MUON_TRACE=1 opens roctx ranges around each call: the library finds
    roctx at run time, and the calls still validate and fail as without it
    (a fresh process, since the switch is read once per process)."""
    code = (
        "import ctypes\n"
        "from muon_step_03_amd import _lib\n"
        "L = _lib.lib()\n"
        "print(L.muon_step(None, None, None, 64, 64, 0, 0.02, 0.95, 0.1, 5, 3.4445, -4.775,"
        " 2.0315, 0, None, 0, None, None))\n"
        "print(L.muon_adamw_step(None, None, None, None, 16, 7, 1e-3, 0.9, 0.95, 1e-8, 0.1, 1,"
        " None))\n"
        "print(int('rocprofiler-sdk-roctx' in open('/proc/self/maps').read()))\n"
    )
    import subprocess
    import sys
    out = {}
    for trace in ("0", "1"):
        env = dict(os.environ, MUON_TRACE=trace)
        r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                           text=True, timeout=120)
        assert r.returncode == 0, r.stderr
        assert "no roctx library" not in r.stderr
        out[trace] = r.stdout.split()
    assert out["1"][:2] == out["0"][:2] and "0" not in out["1"][:2]
    assert out["0"][2] == "0" and out["1"][2] == "1"     # loaded only when tracing
