"""Python binding of libve, the MI355X RaggedShard shard-step library.

Argument marshalling only: every step of the hot path runs in the HIP
kernels behind the C ABI in ``include/ve.h``.  PyTorch supplies device memory
and streams.  Importing this module fails loudly when the library has not
been built (``python -m ragged_shard_optimizer_amd.build``); there is no
fallback implementation.

Names follow the C ABI: ``plan_load`` / ``Plan.query`` / ``Plan.slice`` /
``Plan.copy_in`` / ``Plan.step`` / ``Plan.group_op`` / ``plan_layout`` wrap
``ve_plan_load``, ``ve_plan_query``, ``ve_dbuffer_slice``,
``ve_dbuffer_copy_in``, ``ve_shard_adam8bit_step``, ``ve_dbuffer_group_op``
and ``ve_plan_layout``.
"""

from __future__ import annotations

import ctypes as C
import os
import weakref

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# VE_SANITIZED=1 selects the host-sanitized build (build --sanitize)
LIB_PATH = os.path.join(_HERE, "_build", "libve_san.so" if os.environ.get("VE_SANITIZED") == "1" else "libve.so")

VE_OK, VE_ERR_INVALID_ARG, VE_ERR_LAYOUT, VE_ERR_OOM, VE_ERR_DEVICE, VE_ERR_UNSUPPORTED = range(6)
_STATUS = {0: "VE_OK", 1: "VE_ERR_INVALID_ARG", 2: "VE_ERR_LAYOUT", 3: "VE_ERR_OOM",
           4: "VE_ERR_DEVICE", 5: "VE_ERR_UNSUPPORTED"}

# every symbol include/ve.h declares
EXPORTS = ("ve_plan_load", "ve_plan_free", "ve_plan_query", "ve_dbuffer_copy_in",
           "ve_shard_adam8bit_step", "ve_dbuffer_slice", "ve_dbuffer_group_op", "ve_plan_layout", "ve_plan_buckets",
           "ve_muon_workspace_bytes", "ve_muon_newton_schulz", "ve_muon_newton_schulz_noalloc",
           "ve_gemm_bf16_nt", "ve_stream_copy", "ve_set_option", "ve_get_option", "ve_last_error")

# ve_group_op
GROUP_ZERO, GROUP_SCALE, GROUP_ACCUMULATE = 0, 1, 2


class VeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class TensorSpec(C.Structure):
    _fields_ = [("rows", C.c_int64), ("cols", C.c_int64), ("block_rows", C.c_int64),
                ("block_cols", C.c_int64), ("offset", C.c_int64)]


class AdamHParams(C.Structure):
    _fields_ = [("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float), ("eps", C.c_float),
                ("weight_decay", C.c_float)]


# ve_shard_state: eight device pointers, in this order
STATE_FIELDS = ("grad_ptrs", "grad_shard", "master", "m_q", "v_q", "m_scale", "v_scale", "param_shard")

_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libve.so is not built ({LIB_PATH}); run "
                              "`python -m ragged_shard_optimizer_amd.build`")
        L = C.CDLL(LIB_PATH)
        P = C.c_void_p
        L.ve_last_error.restype = C.c_char_p
        L.ve_plan_load.argtypes = [P, C.c_int32, C.c_int32, C.c_int64, C.c_int32, C.POINTER(C.c_void_p)]
        L.ve_plan_free.argtypes = [P]
        L.ve_plan_query.argtypes = [P, C.c_int32, P, P, P]
        L.ve_dbuffer_copy_in.argtypes = [P, C.c_int32, P, P, P]
        L.ve_shard_adam8bit_step.argtypes = [P, C.c_int32, P, C.c_int32, P, C.c_int64, P]
        L.ve_dbuffer_slice.argtypes = [P, C.c_int32, C.c_int32, P, P, P]
        L.ve_dbuffer_group_op.argtypes = [P, C.c_int32, C.c_int32, C.c_float, P, C.c_int32, P]
        L.ve_plan_layout.argtypes = [P, C.c_int32, C.c_int32, C.c_int64, P, P]
        L.ve_plan_buckets.argtypes = [P, P, C.c_int32, C.c_int32, C.c_int64, C.c_int32, C.c_double, P, P, P]
        L.ve_muon_workspace_bytes.argtypes = [C.c_int64, C.c_int64, P]
        L.ve_muon_newton_schulz.argtypes = [P, P, C.c_int64, C.c_int64, C.c_int32, C.c_float, P, C.c_int64, P]
        L.ve_gemm_bf16_nt.argtypes = [P, C.c_int64, P, C.c_int64, P, C.c_int64, P, C.c_int64, P, C.c_int64,
                                      C.c_int64, C.c_int64, C.c_int64, C.c_float, C.c_float, C.c_int32, P]
        L.ve_stream_copy.argtypes = [P, P, C.c_int64, P]
        L.ve_set_option.argtypes = [C.c_char_p, C.c_int64]
        L.ve_get_option.argtypes = [C.c_char_p, P]
        L.ve_muon_newton_schulz_noalloc.argtypes = [P, P, C.c_int64, C.c_int64, C.c_int32, C.c_float, P]
        for name in EXPORTS[:-1]:
            getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def _check(rc: int):
    if rc != VE_OK:
        raise VeError(rc, lib().ve_last_error().decode())


def _stream_handle(stream):
    if stream is None:
        import torch
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return C.c_void_p(stream)
    return C.c_void_p(stream.cuda_stream)


class Plan:
    """A validated bucket layout (``ve_plan_load``).

    ``specs``: int64 array ``[n, 5]`` of (rows, cols, block_rows, block_cols,
    offset); ``device`` -1 gives a host-only plan (layout queries only).
    """

    def __init__(self, specs, fsdp_size: int, shard_elems: int, device: int = 0):
        spec = np.ascontiguousarray(specs, dtype=np.int64).reshape(-1, 5)
        arr = (TensorSpec * max(1, len(spec)))()
        for i, row in enumerate(spec):
            arr[i] = TensorSpec(*[int(v) for v in row])
        h = C.c_void_p()
        _check(lib().ve_plan_load(arr, len(spec), int(fsdp_size), int(shard_elems), int(device), C.byref(h)))
        self._h = h
        self.n_tensors = len(spec)
        self.fsdp_size = int(fsdp_size)
        self.shard_elems = int(shard_elems)
        self.device = int(device)
        self._pieces = {}
        self._grads_ok = {}  # rank -> gradient tables already checked for it

    def pieces(self, rank: int):
        """[(tensor, elem_end)] of every tensor ``rank`` (or the whole bucket
        for -1) holds a piece of; queried once per rank and kept (the plan is
        immutable)."""
        if rank not in self._pieces:
            got = []
            for k in range(self.n_tensors):
                sl = self.slice(rank, k)
                if sl is not None:
                    got.append((k, sl[2]))
            self._pieces[rank] = got
        return self._pieces[rank]

    def _check_grads(self, rank: int, grad_table):
        """Every tensor whose piece ``rank`` copies has a gradient reaching the
        piece's end.  A gradient table is fixed once built, so each one is
        checked once per rank (a bucket of 10,000 tensors would otherwise
        spend longer here than in the copy)."""
        ok = self._grads_ok.setdefault(int(rank), weakref.WeakSet())
        if grad_table in ok:
            return
        if len(grad_table.grads) != self.n_tensors:
            raise ValueError("grad table length != number of tensors in the plan")
        for k, end in self.pieces(rank):
            g = grad_table.grads[k]
            if g is None or g.numel() < end:
                raise ValueError(f"tensor {k} is copied on rank {rank} but its gradient is missing or short")
        ok.add(grad_table)

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            _check(lib().ve_plan_free(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h

    def query(self, rank: int):
        """(valid_elems, n_blocks, n_segments) of ``rank``."""
        v, b, s = C.c_int64(), C.c_int64(), C.c_int32()
        _check(lib().ve_plan_query(self._h, int(rank), C.byref(v), C.byref(b), C.byref(s)))
        return v.value, b.value, s.value

    def slice(self, rank: int, tensor: int):
        """(shard_offset, elem_start, elem_end), or None if ``rank`` holds none of it."""
        o, a, b = C.c_int64(), C.c_int64(), C.c_int64()
        _check(lib().ve_dbuffer_slice(self._h, int(rank), int(tensor), C.byref(o), C.byref(a), C.byref(b)))
        return None if o.value < 0 else (o.value, a.value, b.value)

    def copy_in(self, rank: int, grad_table, bucket, stream=None):
        """``ve_dbuffer_copy_in``: ``grad_table`` from :func:`grad_pointer_table`,
        ``bucket`` a contiguous 16-bit device tensor of S (or m*S for rank -1)
        elements."""
        need = self.shard_elems * (self.fsdp_size if rank < 0 else 1)
        _require_buffer(bucket, need, 2, "bucket")
        self._check_grads(rank, grad_table)
        _check(lib().ve_dbuffer_copy_in(self._h, int(rank), C.c_void_p(grad_table.table.data_ptr()),
                                        C.c_void_p(bucket.data_ptr()), _stream_handle(stream)))

    def step(self, rank: int, states, hparams: dict, step: int, stream=None):
        """``ve_shard_adam8bit_step`` over a :class:`StateTable` built for the
        same plan and ``rank`` (its scale arrays are sized to that rank's
        block count and its gradient tables checked for that rank's pieces).
        Row blocks are scheduled through counters the plan holds per rank;
        a call for a rank on another stream than the rank's previous call
        waits for it on the GPU.  Under graph capture there is no such
        ordering: replays of a captured step must not overlap other calls
        for the same plan and rank."""
        if states.plan is not self or states.rank != rank:
            raise ValueError("state table was built for another plan or rank")
        hp = AdamHParams(float(hparams["lr"]), float(hparams["beta1"]), float(hparams["beta2"]),
                         float(hparams["eps"]), float(hparams["weight_decay"]))
        _check(lib().ve_shard_adam8bit_step(self._h, int(rank), C.c_void_p(states.table.data_ptr()),
                                            len(states), C.byref(hp), int(step), _stream_handle(stream)))


    def group_op(self, rank: int, op: int, alpha: float, table, stream=None):
        """``ve_dbuffer_group_op`` over a :class:`GroupTable` built for the
        same ``rank``."""
        if table.rank != rank or table.plan is not self:
            raise ValueError("group table was built for another plan or rank")
        if op == GROUP_ACCUMULATE and not table.has_grads:
            raise ValueError("accumulate needs a gradient table for every bucket")
        _check(lib().ve_dbuffer_group_op(self._h, int(rank), int(op), float(alpha),
                                         C.c_void_p(table.table.data_ptr()), len(table),
                                         _stream_handle(stream)))


def plan_layout(shapes, fsdp_size: int, align: int = 16):
    """``ve_plan_layout``: ``shapes`` is an int array ``[n, >=3]`` of (rows,
    cols, block_rows[, block_cols]); returns ``(specs, S, lower_bound)`` with
    ``specs`` int64 ``[n, 5]`` (rows, cols, block_rows, block_cols, offset),
    ready for :class:`Plan`."""
    sh = np.asarray(shapes, dtype=np.int64)
    if sh.ndim != 2 or sh.shape[1] < 3 or len(sh) < 1:
        raise ValueError("shapes: need an [n, >=3] array of (rows, cols, block_rows[, block_cols])")
    arr = (TensorSpec * len(sh))()
    for i, row in enumerate(sh):
        bc = int(row[3]) if sh.shape[1] > 3 else int(row[1])
        arr[i] = TensorSpec(int(row[0]), int(row[1]), int(row[2]), bc, 0)
    S, lb = C.c_int64(), C.c_int64()
    _check(lib().ve_plan_layout(arr, len(sh), int(fsdp_size), int(align), C.byref(S), C.byref(lb)))
    specs = np.array([[a.rows, a.cols, a.block_rows, a.block_cols, a.offset] for a in arr], dtype=np.int64)
    return specs, S.value, lb.value


def plan_buckets(units, fsdp_size: int, align: int = 16, max_units: int = 4, tolerance: float = 0.005):
    """``ve_plan_buckets``: ``units`` is a list (model order) of int arrays
    ``[n_k, >=3]`` of (rows, cols, block_rows[, block_cols]), one per wrapper
    unit.  Returns a list of buckets, each ``(first_unit, end_unit, specs,
    S)`` with ``specs`` int64 ``[n, 5]`` (rows, cols, block_rows,
    block_cols, offset) of the bucket's tensors, ready for :class:`Plan`."""
    shapes = [np.asarray(u, dtype=np.int64).reshape(-1, np.asarray(u).shape[-1]) for u in units]
    if not shapes or any(sh.ndim != 2 or sh.shape[1] < 3 or len(sh) < 1 for sh in shapes):
        raise ValueError("units: a non-empty list of [n, >=3] arrays of (rows, cols, block_rows[, block_cols])")
    allsh = np.concatenate([sh[:, :3] for sh in shapes])
    bcols = np.concatenate([sh[:, 3] if sh.shape[1] > 3 else sh[:, 1] for sh in shapes])
    unit_of = np.concatenate([np.full(len(sh), i, dtype=np.int32) for i, sh in enumerate(shapes)])
    n = len(allsh)
    arr = (TensorSpec * n)()
    for i in range(n):
        arr[i] = TensorSpec(int(allsh[i, 0]), int(allsh[i, 1]), int(allsh[i, 2]), int(bcols[i]), 0)
    bucket_of = np.zeros(n, dtype=np.int32)
    S = np.zeros(len(shapes), dtype=np.int64)
    nb = C.c_int32()
    _check(lib().ve_plan_buckets(arr, C.c_void_p(unit_of.ctypes.data), n, int(fsdp_size), int(align),
                                 int(max_units), float(tolerance), C.c_void_p(bucket_of.ctypes.data),
                                 C.c_void_p(S.ctypes.data), C.byref(nb)))
    specs = np.array([[a.rows, a.cols, a.block_rows, a.block_cols, a.offset] for a in arr], dtype=np.int64)
    out = []
    for b in range(nb.value):
        idx = np.nonzero(bucket_of == b)[0]
        out.append((int(unit_of[idx[0]]), int(unit_of[idx[-1]]) + 1, specs[idx], int(S[b])))
    return out


def muon_workspace_bytes(rows: int, cols: int) -> int:
    n = C.c_int64()
    _check(lib().ve_muon_workspace_bytes(int(rows), int(cols), C.byref(n)))
    return n.value


def _ptr_of(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def muon_newton_schulz(G, out, steps: int = 5, eps: float = 1e-7, workspace=None, stream=None):
    """``ve_muon_newton_schulz``: ``G`` and ``out`` contiguous 2-D 16-bit
    (bf16 bits) device tensors of the same shape; ``workspace`` a uint8
    device tensor of at least :func:`muon_workspace_bytes` bytes (allocated
    here if None)."""
    import torch
    if G.dim() != 2 or tuple(out.shape) != tuple(G.shape):
        raise ValueError("G and out: 2-D tensors of the same shape")
    rows, cols = G.shape
    _require_buffer(G, rows * cols, 2, "G")
    _require_buffer(out, rows * cols, 2, "out")
    need = muon_workspace_bytes(rows, cols)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=G.device)
    _require_buffer(workspace, need, 1, "workspace")
    _check(lib().ve_muon_newton_schulz(_ptr_of(G), _ptr_of(out), rows, cols, int(steps), float(eps),
                                       _ptr_of(workspace), workspace.numel(), _stream_handle(stream)))
    return out


def muon_newton_schulz_noalloc(G, out, steps: int = 5, eps: float = 1e-7, stream=None):
    """``ve_muon_newton_schulz_noalloc``: as :func:`muon_newton_schulz`, with
    the library's static device scratch as the workspace (nothing is
    allocated, here or in the library)."""
    if G.dim() != 2 or tuple(out.shape) != tuple(G.shape):
        raise ValueError("G and out: 2-D tensors of the same shape")
    rows, cols = G.shape
    _require_buffer(G, rows * cols, 2, "G")
    _require_buffer(out, rows * cols, 2, "out")
    _check(lib().ve_muon_newton_schulz_noalloc(_ptr_of(G), _ptr_of(out), rows, cols, int(steps), float(eps),
                                               _stream_handle(stream)))
    return out


def gemm_bf16_nt(P, Q, C=None, CT=None, D=None, alpha: float = 1.0, beta: float = 0.0, symmetric: bool = False,
                 stream=None):
    """``ve_gemm_bf16_nt`` on contiguous 2-D 16-bit device tensors:
    C = bf16(alpha P Q^T + beta D), CT = C^T."""
    M, K = P.shape
    N, K2 = Q.shape
    if K2 != K:
        raise ValueError("P and Q must share the contraction length")
    for t, shape, name in ((C, (M, N), "C"), (CT, (N, M), "CT"), (D, (M, N), "D")):
        if t is not None:
            if tuple(t.shape) != shape:
                raise ValueError(f"{name}: shape {tuple(t.shape)} != {shape}")
            _require_buffer(t, shape[0] * shape[1], 2, name)
    _require_buffer(P, M * K, 2, "P")
    _require_buffer(Q, N * K, 2, "Q")
    _check(lib().ve_gemm_bf16_nt(_ptr_of(P), K, _ptr_of(Q), K, _ptr_of(D), N, _ptr_of(C), N, _ptr_of(CT), M,
                                 M, N, K, float(alpha), float(beta), int(bool(symmetric)), _stream_handle(stream)))


def stream_copy(dst, src, stream=None):
    """``ve_stream_copy``: copy device tensor ``src`` into ``dst`` (same
    number of bytes, contiguous, 16-byte aligned) -- the streaming reference."""
    nbytes = src.numel() * src.element_size()
    if not (src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst: contiguous device tensors")
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same size in bytes")
    _check(lib().ve_stream_copy(C.c_void_p(dst.data_ptr()), C.c_void_p(src.data_ptr()), nbytes,
                                _stream_handle(stream)))


def set_option(name: str, value: int):
    """``ve_set_option``: a process-wide launch option (see include/ve.h)."""
    _check(lib().ve_set_option(name.encode(), int(value)))


def get_option(name: str) -> int:
    v = C.c_int64()
    _check(lib().ve_get_option(name.encode(), C.byref(v)))
    return v.value


class options:
    """Context manager: set launch options for a block of code and restore
    the previous values afterwards, e.g. ``with options(gemm_split=0): ...``."""

    def __init__(self, **values):
        self.values = values
        self.saved = {}

    def __enter__(self):
        for k, v in self.values.items():
            self.saved[k] = get_option(k)
            set_option(k, v)
        return self

    def __exit__(self, *exc):
        for k, v in self.saved.items():
            set_option(k, v)
        return False


def plan_load(specs, fsdp_size, shard_elems, device=0) -> Plan:
    return Plan(specs, fsdp_size, shard_elems, device)


def _require_buffer(t, numel: int, itemsize: int, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous() or t.element_size() != itemsize:
        raise ValueError(f"{name}: need a contiguous tensor of {itemsize}-byte elements")
    if t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements < required {numel}")


class GradTable:
    """Device array of per-parameter gradient pointers (``grad_ptrs``).
    Keeps the tensors alive while the table exists."""

    def __init__(self, grads, device):
        import torch
        ptrs = []
        for g in grads:
            if g is None:
                ptrs.append(0)
                continue
            if not g.is_cuda or not g.is_contiguous() or g.element_size() != 2:
                raise ValueError("gradients must be contiguous 16-bit device tensors")
            ptrs.append(g.data_ptr())
        self.grads = list(grads)
        self.table = torch.tensor(ptrs if ptrs else [0], dtype=torch.int64, device=device)


def grad_pointer_table(grads, device=None) -> GradTable:
    """Per-tensor bf16 gradient tensors (flat or shaped, contiguous; None for
    tensors the call never reads), in the plan's tensor order."""
    if device is None:
        device = next(g.device for g in grads if g is not None)
    return GradTable(grads, device)


class StateTable:
    """Device array of ``ve_shard_state`` records (one per bucket)."""

    def __init__(self, plan: Plan, rank: int, states, device):
        import torch
        S = plan.shard_elems
        _, nb, _ = plan.query(rank)
        rows = []
        self.keep = []
        for st in states:
            gt = st["grad_table"]
            if len(gt.grads) != plan.n_tensors:
                raise ValueError("grad table length != number of tensors in the plan")
            for k, _end in plan.pieces(rank):
                if gt.grads[k] is None:
                    raise ValueError(f"tensor {k} has a piece on rank {rank} but no gradient")
            for k, numel in plan.pieces(-1):  # the whole bucket holds every tensor whole
                if gt.grads[k] is not None and gt.grads[k].numel() < numel:
                    raise ValueError(f"gradient {k} is smaller than the tensor")
            _require_buffer(st["grad_shard"], S, 2, "grad_shard")
            _require_buffer(st["master"], S, 4, "master")
            _require_buffer(st["m_q"], S, 1, "m_q")
            _require_buffer(st["v_q"], S, 1, "v_q")
            _require_buffer(st["m_scale"], nb, 4, "m_scale")
            _require_buffer(st["v_scale"], nb, 4, "v_scale")
            _require_buffer(st["param_shard"], S, 2, "param_shard")
            rows.append([gt.table.data_ptr()] + [st[f].data_ptr() for f in STATE_FIELDS[1:]])
            self.keep.append(st)
        self.table = torch.tensor(rows, dtype=torch.int64, device=device).reshape(-1)
        self.n = len(rows)
        self.plan, self.rank = plan, int(rank)

    def __len__(self):
        return self.n


def state_table(plan: Plan, rank: int, states, device=None) -> StateTable:
    """``states``: list of dicts with keys ``grad_table`` (a GradTable) and
    grad_shard, master, m_q, v_q, m_scale, v_scale, param_shard (device
    tensors)."""
    if device is None:
        device = states[0]["master"].device
    return StateTable(plan, rank, states, device)


class GroupTable:
    """Device array of ``ve_group_operand`` records: one bf16 bucket (rank
    chunk of S elements, or the whole bucket for rank -1) per entry, with an
    optional gradient table (needed by accumulate)."""

    def __init__(self, plan: Plan, rank: int, buckets, grad_tables, device):
        import torch
        need = plan.shard_elems * (plan.fsdp_size if rank < 0 else 1)
        if grad_tables is None:
            grad_tables = [None] * len(buckets)
        if len(grad_tables) != len(buckets):
            raise ValueError("one gradient table per bucket")
        rows = []
        for b, gt in zip(buckets, grad_tables):
            _require_buffer(b, need, 2, "bucket")
            if gt is not None:
                if len(gt.grads) != plan.n_tensors:
                    raise ValueError("grad table length != number of tensors in the plan")
                for k, end in plan.pieces(rank):
                    g = gt.grads[k]
                    if g is None or g.numel() < end:
                        raise ValueError(f"tensor {k} has elements in the range but its gradient is "
                                         "missing or short")
            rows.append([b.data_ptr(), 0 if gt is None else gt.table.data_ptr()])
        self.plan, self.rank = plan, int(rank)
        self.has_grads = all(gt is not None for gt in grad_tables)
        self.keep = (list(buckets), list(grad_tables))
        self.table = torch.tensor(rows if rows else [[0, 0]], dtype=torch.int64, device=device).reshape(-1)
        self.n = len(rows)

    def __len__(self):
        return self.n


def group_table(plan: Plan, rank: int, buckets, grad_tables=None, device=None) -> GroupTable:
    """``buckets``: contiguous 16-bit device tensors; ``grad_tables``: one
    GradTable per bucket (accumulate) or None."""
    if device is None:
        device = buckets[0].device
    return GroupTable(plan, rank, buckets, grad_tables, device)


def new_state(plan: Plan, rank: int, grad_table: GradTable, master, device=None) -> dict:
    """Allocate one bucket's state around an fp32 master shard (codes and
    scales zero, outputs zero)."""
    import torch
    device = device or master.device
    S = plan.shard_elems
    _, nb, _ = plan.query(rank)
    return dict(grad_table=grad_table,
                grad_shard=torch.zeros(S, dtype=torch.int16, device=device),
                master=master,
                m_q=torch.zeros(S, dtype=torch.int8, device=device),
                v_q=torch.zeros(S, dtype=torch.int8, device=device),
                m_scale=torch.zeros(max(nb, 1), dtype=torch.float32, device=device),
                v_scale=torch.zeros(max(nb, 1), dtype=torch.float32, device=device),
                param_shard=torch.zeros(S, dtype=torch.int16, device=device))
