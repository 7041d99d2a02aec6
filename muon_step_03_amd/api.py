"""PyTorch-facing binding of libmuon.so: tensor checks and argument marshalling.

Every arithmetic step of the Muon step runs in the library's HIP kernels;
PyTorch only provides device memory (weights, gradients, momentum, workspace,
pointer tables) and the current stream.

Defaults follow the pages: lr 0.02, momentum 0.95 with Nesterov, 5
Newton-Schulz steps with (3.4445, -4.7750, 2.0315) ("LLM Pretraining Loss
Spike 진단과 처방 ... Muon 전환 판단", section "Muon head의 실체는 하이브리드
옵티마이저다"), weight decay 0.1 (the torch.optim.Muon example of "[Deep
Learning] Muon — 행렬 업데이트를 직교화하는 옵티마이저", section 5), and
non-2-D parameters are rejected (same section).
"""
from __future__ import annotations

import ctypes
from typing import Iterable, Sequence

import torch

from . import _lib

NS_COEFFICIENTS = (3.4445, -4.7750, 2.0315)
VARIANTS = {"muon": _lib.MUON_VARIANT_MUON, "muongs": _lib.MUON_VARIANT_MUONGS,
            "muonh": _lib.MUON_VARIANT_MUONH, "normuon": _lib.MUON_VARIANT_NORMUON,
            "meqmuon": _lib.MUON_VARIANT_MEQMUON}
SCALES = {"moonlight": 0, "keller": _lib.MUON_SCALE_KELLER}
_DTYPES = {torch.float32: _lib.MUON_DTYPE_F32, torch.bfloat16: _lib.MUON_DTYPE_BF16}


class MuonError(RuntimeError):
    """A non-zero status returned by the library."""

    def __init__(self, status: int, where: str):
        msg = f"{where}: {_lib.status_string(status)} (status {status})"
        if status == _lib.MUON_ERR_HIP:
            msg += f", hip error {_lib.lib().muon_last_hip_error()}"
        super().__init__(msg)
        self.status = status


def _check(status: int, where: str) -> None:
    if status != _lib.MUON_OK:
        raise MuonError(status, where)


def dtype_code(dtype: torch.dtype) -> int:
    try:
        return _DTYPES[dtype]
    except KeyError:
        raise TypeError(f"Muon weights must be float32 or bfloat16, got {dtype}") from None


def _variant_code(variant, scale="moonlight") -> int:
    """variant name (or raw code) OR-ed with the shape-factor flag."""
    if scale not in SCALES:
        raise ValueError(f"unknown scale {scale!r}; expected one of {sorted(SCALES)}")
    if isinstance(variant, int):
        return variant | SCALES[scale]
    try:
        return VARIANTS[variant] | SCALES[scale]
    except KeyError:
        raise ValueError(f"unknown variant {variant!r}; expected one of {sorted(VARIANTS)}") from None


def _stream_handle(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _keep_for_stream(stream, *tensors) -> None:
    """Tensors this binding allocated (on the current stream) and hands to
    kernels enqueued on ``stream``: when that is another stream, tell the
    caching allocator, so that their blocks are not given to a later
    allocation before the kernels on ``stream`` are done with them."""
    if stream is None:
        return
    cur = torch.cuda.current_stream(stream.device)
    if stream.cuda_stream == cur.cuda_stream:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def check_stats(stats, n_matrices: int, device=None) -> None:
    """A statistics buffer must be a contiguous float32 GPU tensor of at least
    ``n_matrices * MUON_STATS_PER_MATRIX`` elements (on ``device`` if given):
    the library writes that many floats and no bounds are checked on the
    device."""
    if stats is None:
        return
    if not isinstance(stats, torch.Tensor):
        raise TypeError("stats must be a torch.Tensor")
    need = int(n_matrices) * _lib.MUON_STATS_PER_MATRIX
    if stats.dtype != torch.float32:
        raise ValueError(f"stats must be float32, got {stats.dtype}")
    if stats.numel() < need:
        raise ValueError(f"stats holds {stats.numel()} floats, {need} needed "
                         f"({n_matrices} matrices x {_lib.MUON_STATS_PER_MATRIX})")
    if not stats.is_contiguous():
        raise ValueError("stats must be contiguous")
    if not stats.is_cuda:
        raise ValueError("stats must be on a GPU")
    if device is not None and stats.device != torch.device(device):
        raise ValueError(f"stats is on {stats.device}, the weights on {device}")


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _scalars(dtype, lr, momentum, weight_decay, ns_steps, ns_coefficients, variant,
             scale="moonlight"):
    a, b, c = ns_coefficients
    return [dtype, float(lr), float(momentum), float(weight_decay), int(ns_steps),
            float(a), float(b), float(c), _variant_code(variant, scale)]


def _check_matrix(name, t, shape=None, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.ndim != 2:
        raise ValueError(f"Muon updates 2-D weight matrices only; {name} has {t.ndim} dims")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


def workspace_bytes(count: int, rows: int, cols: int, dtype: torch.dtype) -> int:
    return int(_lib.lib().muon_workspace_bytes(count, rows, cols, dtype_code(dtype)))


def _groups_array(groups: Sequence[_lib.MuonGroup]):
    arr = (_lib.MuonGroup * max(1, len(groups)))()
    for i, g in enumerate(groups):
        arr[i] = g
    return arr


def workspace_bytes_grouped(groups: Sequence[_lib.MuonGroup], dtype: torch.dtype) -> int:
    arr = _groups_array(groups)
    return int(_lib.lib().muon_workspace_bytes_grouped(arr, len(groups), dtype_code(dtype)))


def _workspace(nbytes: int, device, workspace):
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} "
                             f"bytes, {nbytes} needed")
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def muon_step(W, G, M, *, lr=0.02, momentum=0.95, weight_decay=0.1, ns_steps=5,
              ns_coefficients=NS_COEFFICIENTS, variant="muon", scale="moonlight", workspace=None,
              stats=None, stream=None):
    """One Muon step on one matrix, in place on W and M.

    W, G: [rows, cols] float32 or bfloat16 on the GPU (same dtype); M float32.
    stats: optional float32 GPU tensor of 5 elements (||U||, ||W||^2, <W,O>,
    ||O||^2, ||O~||^2).
    """
    _check_matrix("W", W)
    _check_matrix("G", G, W.shape, W.dtype)
    _check_matrix("M", M, W.shape, torch.float32)
    rows, cols = W.shape
    dt = dtype_code(W.dtype)
    need = workspace_bytes(1, rows, cols, W.dtype)
    ws = _workspace(need, W.device, workspace)
    check_stats(stats, 1, W.device)
    st = _lib.lib().muon_step(
        _ptr(W), _ptr(G), _ptr(M), rows, cols,
        *_scalars(dt, lr, momentum, weight_decay, ns_steps, ns_coefficients, variant, scale),
        _ptr(ws), ws.numel() * ws.element_size(), _ptr(stats), _stream_handle(stream))
    _check(st, "muon_step")
    if workspace is None:
        _keep_for_stream(stream, ws)
    return W, M


def pointer_table(tensors: Iterable[torch.Tensor], device) -> torch.Tensor:
    """Device int64 array of the tensors' data pointers (a device pointer table)."""
    ptrs = [t.data_ptr() for t in tensors]
    return torch.tensor(ptrs, dtype=torch.int64, device=device)


def muon_step_batched(Ws, Gs, Ms, *, lr=0.02, momentum=0.95, weight_decay=0.1, ns_steps=5,
                      ns_coefficients=NS_COEFFICIENTS, variant="muon", scale="moonlight",
                      workspace=None, stats=None, stream=None, tables=None):
    """One Muon step on a list of same-shape matrices (device pointer tables).

    ``tables`` may pass prebuilt (W, G, M) pointer tables to skip rebuilding.
    """
    Ws, Gs, Ms = list(Ws), list(Gs), list(Ms)
    if not (len(Ws) == len(Gs) == len(Ms)):
        raise ValueError("W, G and M lists must have the same length")
    if not Ws:
        return
    shape, dtype = Ws[0].shape, Ws[0].dtype
    for i, (w, g, m) in enumerate(zip(Ws, Gs, Ms)):
        _check_matrix(f"W[{i}]", w, shape, dtype)
        _check_matrix(f"G[{i}]", g, shape, dtype)
        _check_matrix(f"M[{i}]", m, shape, torch.float32)
    dev = Ws[0].device
    own_tables = tables is None
    if own_tables:
        tables = (pointer_table(Ws, dev), pointer_table(Gs, dev), pointer_table(Ms, dev))
    check_stats(stats, len(Ws), dev)
    rows, cols = shape
    need = workspace_bytes(len(Ws), rows, cols, dtype)
    ws = _workspace(need, dev, workspace)
    st = _lib.lib().muon_step_batched(
        _ptr(tables[0]), _ptr(tables[1]), _ptr(tables[2]), len(Ws), rows, cols,
        *_scalars(dtype_code(dtype), lr, momentum, weight_decay, ns_steps, ns_coefficients,
                  variant, scale),
        _ptr(ws), ws.numel() * ws.element_size(), _ptr(stats), _stream_handle(stream))
    _check(st, "muon_step_batched")
    _keep_for_stream(stream, *(tables if own_tables else ()), ws if workspace is None else None)


def stacked_group(W: torch.Tensor, G: torch.Tensor, M: torch.Tensor) -> _lib.MuonGroup:
    """A group over contiguous [count, rows, cols] stacks."""
    if W.ndim != 3:
        raise ValueError("a stacked group needs [count, rows, cols] tensors")
    for name, t, dt in (("W", W, W.dtype), ("G", G, W.dtype), ("M", M, torch.float32)):
        if tuple(t.shape) != tuple(W.shape) or t.dtype != dt or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} stack must be a contiguous GPU tensor of shape "
                             f"{tuple(W.shape)} and dtype {dt}")
    n, r, c = W.shape
    return _lib.MuonGroup(n, r, c, None, None, None, W.data_ptr(), G.data_ptr(), M.data_ptr())


def chunk_size(shapes, dtype: torch.dtype, max_workspace_bytes: int) -> int:
    """Matrices per shape per grouped call: the fewest calls such that one
    call over min(c, count) matrices of every (count, rows, cols) shape needs
    at most ``max_workspace_bytes`` of workspace (which grows with c), with
    the matrices spread evenly over those calls."""
    shapes = [(int(n), int(r), int(k)) for n, r, k in shapes]
    if not shapes or min(n for n, _, _ in shapes) < 1:
        raise ValueError("chunk_size needs non-empty shape groups")

    def need(c):
        return workspace_bytes_grouped([_lib.MuonGroup(min(c, n), r, k, None, None, None,
                                                       None, None, None)
                                        for n, r, k in shapes], dtype)

    lo, hi = 1, max(n for n, _, _ in shapes)
    if need(lo) > max_workspace_bytes:
        raise ValueError(f"one matrix of each shape needs {need(lo)} workspace bytes, "
                         f"more than {max_workspace_bytes}")
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if need(mid) <= max_workspace_bytes:
            lo = mid
        else:
            hi = mid - 1
    calls = -(-max(n for n, _, _ in shapes) // lo)
    return -(-max(n for n, _, _ in shapes) // calls)   # same number of calls, even chunks


def stacked_chunks(stacks, dtype: torch.dtype, max_workspace_bytes: int):
    """Split a model given as (W, G, M) [count, rows, cols] stacks into
    successive grouped calls whose workspace fits ``max_workspace_bytes``.

    Call k takes matrices [k c, (k+1) c) of every stack, c = :func:`chunk_size`;
    a model that fits whole is one call.  Returns the list of calls (each a
    list of groups for :func:`muon_step_grouped`) and the workspace bytes the
    largest call needs.  Every matrix's step is independent of the others, so
    running the calls in order on one stream is the whole step."""
    stacks = list(stacks)
    c = chunk_size([tuple(W.shape) for W, _, _ in stacks], dtype, max_workspace_bytes)
    counts = [int(W.shape[0]) for W, _, _ in stacks]
    calls = [[stacked_group(W[k:k + c], G[k:k + c], M[k:k + c])
              for (W, G, M), n in zip(stacks, counts) if k < n]
             for k in range(0, max(counts), c)]
    return calls, max(workspace_bytes_grouped(call, dtype) for call in calls)


def table_group(count, rows, cols, W_table, G_table, M_table) -> _lib.MuonGroup:
    """A group over device pointer tables (int64 GPU tensors of data pointers)."""
    return _lib.MuonGroup(count, rows, cols, W_table.data_ptr(), G_table.data_ptr(),
                          M_table.data_ptr(), None, None, None)


def muon_step_grouped(groups: Sequence[_lib.MuonGroup], dtype: torch.dtype, *, lr=0.02,
                      momentum=0.95, weight_decay=0.1, ns_steps=5,
                      ns_coefficients=NS_COEFFICIENTS, variant="muon", scale="moonlight",
                      workspace=None, stats=None, stream=None, device=None):
    """One Muon step over several shape groups (a whole model) in one launch
    sequence.  Build groups with :func:`stacked_group` / :func:`table_group`;
    the caller keeps the tensors they point to alive."""
    groups = list(groups)
    need = workspace_bytes_grouped(groups, dtype)
    if device is None:
        device = torch.device("cuda", torch.cuda.current_device())
    check_stats(stats, sum(int(g.count) for g in groups), device)
    ws = _workspace(need, device, workspace)
    arr = _groups_array(groups)
    st = _lib.lib().muon_step_grouped(
        arr, len(groups),
        *_scalars(dtype_code(dtype), lr, momentum, weight_decay, ns_steps, ns_coefficients,
                  variant, scale),
        _ptr(ws), ws.numel() * ws.element_size(), _ptr(stats), _stream_handle(stream))
    _check(st, "muon_step_grouped")
    if workspace is None:
        _keep_for_stream(stream, ws)


def muon_step_grouped_noalloc(groups: Sequence[_lib.MuonGroup], dtype: torch.dtype, *, lr=0.02,
                              momentum=0.95, weight_decay=0.1, ns_steps=5,
                              ns_coefficients=NS_COEFFICIENTS, variant="muon", scale="moonlight",
                              stats=None, stream=None, device=None):
    """:func:`muon_step_grouped` on the library's static workspace
    (``MUON_NOALLOC_WORKSPACE_BYTES`` per GPU): nothing is allocated, here
    or in the library.  Calls that overlap in time on one GPU share that
    workspace and must be serialised by the caller."""
    groups = list(groups)
    if device is None:
        device = torch.device("cuda", torch.cuda.current_device())
    check_stats(stats, sum(int(g.count) for g in groups), device)
    arr = _groups_array(groups)
    st = _lib.lib().muon_step_grouped_noalloc(
        arr, len(groups),
        *_scalars(dtype_code(dtype), lr, momentum, weight_decay, ns_steps, ns_coefficients,
                  variant, scale),
        _ptr(stats), _stream_handle(stream))
    _check(st, "muon_step_grouped_noalloc")


class MuonStep:
    """Muon (or MuonGS) for a list of 2-D hidden weights.

    Parameters are grouped by (shape, dtype); each group keeps device pointer
    tables and fp32 momentum buffers, and :meth:`step` updates every group in
    one launch sequence per dtype from the parameters' ``.grad``, on the
    current stream.

    ``stats_order`` lists the parameter indices in the order of the rows of
    the optional ``stats`` buffer of :meth:`step` (``MUON_STATS_PER_MATRIX``
    floats per parameter): parameters grouped by dtype, then by shape (each
    in order of first appearance), then in parameter order.
    """

    def __init__(self, params, lr=0.02, momentum=0.95, weight_decay=0.1, ns_steps=5,
                 ns_coefficients=NS_COEFFICIENTS, variant="muon", scale="moonlight"):
        self.params = list(params)
        for i, p in enumerate(self.params):
            if p.ndim != 2:
                raise ValueError(f"Muon updates 2-D weight matrices only; parameter {i} has "
                                 f"{p.ndim} dims (use AdamW for it)")
            _check_matrix(f"param[{i}]", p.data)
        self.hp = dict(lr=lr, momentum=momentum, weight_decay=weight_decay, ns_steps=ns_steps,
                       ns_coefficients=tuple(ns_coefficients), variant=variant, scale=scale)
        self.momentum_buffers = [torch.zeros(p.shape, dtype=torch.float32, device=p.device)
                                 for p in self.params]
        self._by_dtype = {}
        for i, p in enumerate(self.params):
            self._by_dtype.setdefault(p.dtype, {}).setdefault(tuple(p.shape), []).append(i)
        self.stats_order = [i for shapes in self._by_dtype.values() for idx in shapes.values()
                            for i in idx]
        self._tables = {}
        self._workspaces = {}

    def _table(self, tab, slot, tensors, dev):
        """Rebuild the pointer table in ``tab[slot]`` when the tensors' data
        pointers differ from the ones it was built from (``tab[slot + 1]``):
        a parameter whose ``.data`` was rebound, or new gradient tensors."""
        ptrs = tuple(t.data_ptr() for t in tensors)
        if tab[slot + 1] != ptrs:
            tab[slot] = pointer_table(tensors, dev)
            tab[slot + 1] = ptrs
        return tab[slot]

    def _groups(self, dtype, shapes):
        groups, keep = [], []
        for shape, idx in shapes.items():
            dev = self.params[idx[0]].device
            grads, datas = [], []
            for i in idx:
                g = self.params[i].grad
                if g is None:
                    raise RuntimeError(f"parameter {i} has no gradient")
                _check_matrix(f"grad[{i}]", g, shape, dtype)
                _check_matrix(f"param[{i}]", self.params[i].data, shape, dtype)
                grads.append(g)
                datas.append(self.params[i].data)
            tab = self._tables.setdefault((dtype, shape), [None] * 6)
            w_tab = self._table(tab, 0, datas, dev)
            g_tab = self._table(tab, 2, grads, dev)
            m_tab = self._table(tab, 4, [self.momentum_buffers[i] for i in idx], dev)
            groups.append(table_group(len(idx), shape[0], shape[1], w_tab, g_tab, m_tab))
            keep.append(grads)
        return groups, keep

    @torch.no_grad()
    def step(self, stats=None):
        """One step of every parameter.  ``stats``: optional float32 GPU
        tensor of ``len(params) * MUON_STATS_PER_MATRIX`` floats, rows in
        ``stats_order``."""
        check_stats(stats, len(self.params))
        offset = 0
        for dtype, shapes in self._by_dtype.items():
            groups, _keep = self._groups(dtype, shapes)
            need = workspace_bytes_grouped(groups, dtype)
            ws = self._workspaces.get(dtype)
            if ws is None or ws.numel() < need:
                dev = self.params[next(iter(shapes.values()))[0]].device
                ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
                self._workspaces[dtype] = ws
            n = sum(len(idx) for idx in shapes.values())
            st = None if stats is None else \
                stats[offset * _lib.MUON_STATS_PER_MATRIX:(offset + n) * _lib.MUON_STATS_PER_MATRIX]
            muon_step_grouped(groups, dtype, workspace=ws, stats=st, device=ws.device, **self.hp)
            offset += n


# ---------------------------------------------------------------- AdamW half
# The hybrid optimizer's AdamW for embeddings, output head and 1-D parameters
# ("LLM Pretraining Loss Spike 진단과 처방", section "Muon head의 실체는 하이브리드
# 옵티마이저다").  Defaults from the experiments paragraph of "MuonGS:
# Pretraining LLMs with Relaxed Weight-Norm Control": betas (0.8, 0.95),
# eps 1e-10, weight decay 1e-3, peak lrs 0.7 / 0.004 / 0.015 for embedding /
# head / 1-D parameters.
AUX_BETAS = (0.8, 0.95)
AUX_EPS = 1e-10
AUX_WEIGHT_DECAY = 1e-3
AUX_LR = {"embedding": 0.7, "head": 0.004, "vector": 0.015}


def _check_flat(name, t, numel=None, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


def adamw_tensor(P, G, m, v, *, lr, weight_decay=AUX_WEIGHT_DECAY) -> _lib.AdamwTensor:
    """Descriptor of one tensor for :func:`adamw_step_grouped` (the caller
    keeps P, G, m, v alive until the step has run)."""
    _check_flat("P", P)
    dtype_code(P.dtype)
    _check_flat("G", G, P.numel(), P.dtype)
    _check_flat("m", m, P.numel(), torch.float32)
    _check_flat("v", v, P.numel(), torch.float32)
    return _lib.AdamwTensor(P.data_ptr(), G.data_ptr(), m.data_ptr(), v.data_ptr(), P.numel(),
                            float(lr), float(weight_decay))


def adamw_step(P, G, m, v, *, lr, step, betas=AUX_BETAS, eps=AUX_EPS,
               weight_decay=AUX_WEIGHT_DECAY, stream=None):
    """One AdamW step on one tensor, in place on P, m and v.  ``step`` counts
    updates from 1 (bias corrections)."""
    t = adamw_tensor(P, G, m, v, lr=lr, weight_decay=weight_decay)
    st = _lib.lib().muon_adamw_step(t.P, t.G, t.m, t.v, t.n, dtype_code(P.dtype), t.lr,
                                    float(betas[0]), float(betas[1]), float(eps),
                                    t.weight_decay, int(step), _stream_handle(stream))
    _check(st, "muon_adamw_step")


def adamw_step_grouped(tensors: Sequence[_lib.AdamwTensor], dtype: torch.dtype, *, step,
                       betas=AUX_BETAS, eps=AUX_EPS, stream=None):
    """One AdamW step on many tensors of one dtype, one launch per
    ``MUON_ADAMW_TENSORS_PER_LAUNCH`` tensors."""
    tensors = list(tensors)
    arr = (_lib.AdamwTensor * max(1, len(tensors)))()
    for i, t in enumerate(tensors):
        arr[i] = t
    st = _lib.lib().muon_adamw_step_grouped(arr, len(tensors), dtype_code(dtype),
                                            float(betas[0]), float(betas[1]), float(eps),
                                            int(step), _stream_handle(stream))
    _check(st, "muon_adamw_step_grouped")


class AdamWStep:
    """AdamW over parameter groups (dicts with ``params``, ``lr`` and optional
    ``weight_decay``), float32 moments per parameter, every parameter of one
    dtype updated by one grouped call per step from its ``.grad``."""

    def __init__(self, param_groups, betas=AUX_BETAS, eps=AUX_EPS,
                 weight_decay=AUX_WEIGHT_DECAY):
        self.betas = tuple(betas)
        self.eps = float(eps)
        self.entries = []   # (param, m, v, lr, weight_decay)
        for gi, grp in enumerate(param_groups):
            lr = grp["lr"]
            wd = grp.get("weight_decay", weight_decay)
            for p in grp["params"]:
                _check_flat(f"group {gi} param", p.data)
                dtype_code(p.dtype)
                self.entries.append((p, torch.zeros(p.numel(), dtype=torch.float32, device=p.device),
                                     torch.zeros(p.numel(), dtype=torch.float32, device=p.device),
                                     lr, wd))
        self.step_count = 0

    @torch.no_grad()
    def step(self):
        self.step_count += 1
        by_dtype = {}
        for i, (p, m, v, lr, wd) in enumerate(self.entries):
            if p.grad is None:
                raise RuntimeError(f"AdamW parameter {i} has no gradient")
            by_dtype.setdefault(p.dtype, []).append(
                adamw_tensor(p.data, p.grad, m, v, lr=lr, weight_decay=wd))
        for dtype, tensors in by_dtype.items():
            adamw_step_grouped(tensors, dtype, step=self.step_count, betas=self.betas, eps=self.eps)


class HybridMuonAdamW:
    """The hybrid the pages describe: Muon on hidden 2-D weights, AdamW on
    everything else (embedding, head, gains, biases).  ``muon_params`` go to
    :class:`MuonStep`, ``adamw_groups`` to :class:`AdamWStep`."""

    def __init__(self, muon_params, adamw_groups, *, muon_kwargs=None, adamw_kwargs=None):
        self.muon = MuonStep(muon_params, **(muon_kwargs or {}))
        self.adamw = AdamWStep(adamw_groups, **(adamw_kwargs or {}))

    def step(self, stats=None):
        self.muon.step(stats=stats)
        self.adamw.step()
