"""CPU oracle for the RaggedShard shard step -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path never does: it has
its own GPU library and fails loudly when that library is missing.

``ve_oracle.c`` holds the arithmetic (plain C, fp64 updates; see its header
for the method and the readings taken where the pages are silent).  This
module only builds it with gcc and marshals numpy arrays through ctypes.
``bruteforce.py`` is a second, unsharded numpy formulation used to pin the
C oracle's layout logic.
"""

from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ve_oracle.c")
_PLAIN = os.path.join(_HERE, "_build", "libve_oracle.so")
_SAN = os.path.join(_HERE, "_build", "libve_oracle_san.so")
# VE_SANITIZED=1 selects the AddressSanitizer + UBSan build (same runtime as
# the library's sanitized build, so both can share one process)
_LIB = _SAN if os.environ.get("VE_SANITIZED") == "1" else _PLAIN


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile the oracle with gcc (no FMA contraction, IEEE semantics); with
    ``sanitize``, with clang and AddressSanitizer + UBSan."""
    out = _SAN if sanitize else _PLAIN
    if force or not os.path.exists(out):
        os.makedirs(os.path.dirname(out), exist_ok=True)
        tmp = out + f".tmp{os.getpid()}"
        if sanitize:
            cmd = ["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
                   "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                   "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        else:
            cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
                   "-fno-fast-math", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, out)
    return out


class _Tensor(C.Structure):
    _fields_ = [("rows", C.c_int64), ("cols", C.c_int64), ("block_rows", C.c_int64),
                ("block_cols", C.c_int64), ("offset", C.c_int64)]


class _HParams(C.Structure):
    _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double),
                ("eps", C.c_double), ("wd", C.c_double)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(sanitize=_LIB == _SAN)
        L = C.CDLL(_LIB)
        P = C.c_void_p
        L.ora_last_error.restype = C.c_char_p
        L.ora_validate.argtypes = [P, C.c_int, C.c_int, C.c_int64]
        L.ora_rank_blocks.restype = C.c_int64
        L.ora_rank_blocks.argtypes = [P, C.c_int, C.c_int64, C.c_int64, P]
        L.ora_slice.argtypes = [P, C.c_int, C.c_int, C.c_int64, C.c_int64, C.c_int, P, P, P]
        L.ora_copy_in.restype = None
        L.ora_copy_in.argtypes = [P, C.c_int, C.c_int, C.c_int64, C.c_int64, P, P, P]
        L.ora_group_op.argtypes = [P, C.c_int, C.c_int, C.c_int64, C.c_int64, C.c_int, C.c_float, P, P, P]
        L.ora_plan_min_shard.restype = C.c_int64
        L.ora_plan_min_shard.argtypes = [P, P, P, C.c_int, C.c_int64, C.c_int64, C.c_int64]
        L.ora_plan_min_shard_any_order.restype = C.c_int64
        L.ora_plan_min_shard_any_order.argtypes = [P, P, C.c_int, C.c_int64, C.c_int64, C.c_int64]
        L.ora_quantize.restype = None
        L.ora_quantize.argtypes = [P, C.c_int64, P, P]
        L.ora_shard_step.argtypes = [P, C.c_int, C.c_int, C.c_int64, C.c_int64, P, P,
                                     P, P, P, P, P, P, P, P, C.c_int64, P, C.c_int64]
        _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


_spec_cache: dict = {}


def _specs(spec: np.ndarray):
    spec = np.ascontiguousarray(spec, dtype=np.int64).reshape(-1, 5)
    key = spec.tobytes()
    hit = _spec_cache.get(key)
    if hit is not None:
        return hit
    arr = (_Tensor * max(1, len(spec))).from_buffer_copy(spec.tobytes() if len(spec) else bytes(40))
    if len(_spec_cache) > 64:
        _spec_cache.clear()
    _spec_cache[key] = (arr, len(spec))
    return arr, len(spec)


def _ptr(a):
    return a.ctypes.data_as(C.c_void_p) if a is not None else None


def quantize(x) -> tuple:
    """The oracle's block quantiser on one fp32 block: (int8 codes, fp32 scale)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    q = np.zeros(x.size, dtype=np.int8)
    s = np.zeros(1, dtype=np.float32)
    lib().ora_quantize(_ptr(x), x.size, _ptr(q), _ptr(s))
    return q, np.float32(s[0])


def validate(spec, m: int, S: int) -> None:
    arr, n = _specs(spec)
    if lib().ora_validate(arr, n, m, S) != 0:
        raise OracleError(lib().ora_last_error().decode())


def rank_blocks(spec, S: int, rank: int):
    """(number of quantisation blocks, number of valid elements) on ``rank``."""
    arr, n = _specs(spec)
    v = C.c_int64(0)
    nb = lib().ora_rank_blocks(arr, n, S, rank, C.byref(v))
    return int(nb), int(v.value)


def slice_(spec, m: int, S: int, rank: int, k: int):
    """(shard_offset, elem_start, elem_end) of tensor k on ``rank``, or None."""
    arr, n = _specs(spec)
    a, b, c = C.c_int64(), C.c_int64(), C.c_int64()
    ok = lib().ora_slice(arr, n, m, S, rank, k, C.byref(a), C.byref(b), C.byref(c))
    return (a.value, b.value, c.value) if ok else None


def _grad_table(grads, bases, n):
    ptrs = (C.c_void_p * max(1, n))()
    base = np.zeros(max(1, n), dtype=np.int64)
    keep = []
    for k in range(n):
        g = grads[k]
        if g is None:
            ptrs[k] = None
            continue
        g = np.ascontiguousarray(g, dtype=np.uint16)
        keep.append(g)
        ptrs[k] = g.ctypes.data
        base[k] = 0 if bases is None else int(bases[k])
    return ptrs, base, keep


def copy_in(spec, m: int, S: int, rank: int, grads, bases=None) -> np.ndarray:
    """Group copy-in of ``rank``'s chunk (rank -1: the whole bucket)."""
    arr, n = _specs(spec)
    ptrs, base, keep = _grad_table(grads, bases, n)
    out = np.empty(m * S if rank < 0 else S, dtype=np.uint16)
    lib().ora_copy_in(arr, n, m, S, rank, ptrs, _ptr(base), _ptr(out))
    return out


GROUP_ZERO, GROUP_SCALE, GROUP_ACCUMULATE = 0, 1, 2


def group_op(spec, m: int, S: int, rank: int, op: int, alpha: float, bucket: np.ndarray, grads=None,
             bases=None) -> np.ndarray:
    """DBuffer group operation on ``bucket`` (uint16 bf16 bits, length S for
    ``rank`` >= 0, m*S for ``rank`` = -1), updated in place.  ``op`` is
    GROUP_ZERO, GROUP_SCALE or GROUP_ACCUMULATE; ``alpha`` is rounded to fp32
    first; ``grads`` (accumulate only) are the per-parameter bf16 gradients,
    as for ``copy_in``."""
    arr, n = _specs(spec)
    if grads is None:
        grads = [None] * n
    ptrs, base, keep = _grad_table(grads, bases, n)
    if bucket.dtype != np.uint16 or not bucket.flags.c_contiguous:
        raise TypeError("bucket: need contiguous uint16")
    rc = lib().ora_group_op(arr, n, m, S, rank, int(op), float(np.float32(alpha)), ptrs, _ptr(base),
                            _ptr(bucket))
    if rc != 0:
        raise OracleError(lib().ora_last_error().decode())
    return bucket


def plan_min_shard(sizes, units, m: int, align: int, s_max: int, order=None) -> int:
    """Exhaustive search: the smallest S (multiple of ``align``, <= s_max) at
    which tensors of ``sizes`` elements and shard ``units`` fit in m chunks,
    in ``order`` (default: as given), or over every order when ``order`` is
    "any" (at most 8 tensors).  0 if no S up to s_max works.  Tiny inputs
    only: the search is exponential."""
    n = np.ascontiguousarray(sizes, dtype=np.int64)
    u = np.ascontiguousarray(units, dtype=np.int64)
    if n.shape != u.shape or n.ndim != 1 or len(n) < 1:
        raise ValueError("sizes and units: equal-length 1-D arrays")
    if isinstance(order, str) and order == "any":
        r = lib().ora_plan_min_shard_any_order(_ptr(n), _ptr(u), len(n), m, align, s_max)
        if r < 0:
            raise OracleError(lib().ora_last_error().decode())
        return int(r)
    o = np.arange(len(n), dtype=np.intc) if order is None else np.ascontiguousarray(order, dtype=np.intc)
    return int(lib().ora_plan_min_shard(_ptr(n), _ptr(u), _ptr(o), len(n), m, align, s_max))


def shard_step(spec, m: int, S: int, rank: int, grads, state: dict, hp: dict, t: int,
               bases=None, blocks=None) -> dict:
    """One fused step on ``rank``; ``state`` arrays are updated in place.

    ``state`` keys: grad_shard (uint16[S]), master (float32[S]), m_q, v_q
    (int8[S]), m_scale, v_scale (float32[B_r]), param_shard (uint16[S]).
    ``hp`` values are rounded to fp32 first (the step's hyper-parameters are
    fp32 numbers).
    ``blocks``: optional list of block indices to process (the rest is
    untouched).
    """
    arr, n = _specs(spec)
    ptrs, base, keep = _grad_table(grads, bases, n)
    want = {"grad_shard": np.uint16, "master": np.float32, "m_q": np.int8, "v_q": np.int8,
            "m_scale": np.float32, "v_scale": np.float32, "param_shard": np.uint16}
    for key, dt in want.items():
        a = state[key]
        if a.dtype != dt or not a.flags.c_contiguous:
            raise TypeError(f"{key}: need contiguous {np.dtype(dt)}")
    # the step's hyper-parameters are fp32 quantities; the oracle works on
    # exactly those values, widened to double
    f = lambda key: float(np.float32(hp[key]))
    h = _HParams(f("lr"), f("beta1"), f("beta2"), f("eps"), f("weight_decay"))
    sel = None if blocks is None else np.unique(np.asarray(blocks, dtype=np.int64))
    rc = lib().ora_shard_step(arr, n, m, S, rank, ptrs, _ptr(base),
                              _ptr(state["grad_shard"]), _ptr(state["master"]), _ptr(state["m_q"]),
                              _ptr(state["v_q"]), _ptr(state["m_scale"]), _ptr(state["v_scale"]),
                              _ptr(state["param_shard"]), C.byref(h), int(t),
                              _ptr(sel), 0 if sel is None else len(sel))
    if rc != 0:
        raise OracleError(lib().ora_last_error().decode())
    return state


def shard_step_threads(spec, m: int, S: int, rank: int, grads, state: dict, hp: dict, t: int, bases=None,
                       threads: int = 1) -> dict:
    """The same step as :func:`shard_step`, with the rank's blocks split into
    ``threads`` contiguous ranges stepped by that many host threads at once
    (each C call releases the interpreter lock; blocks touch disjoint
    elements and scales).  Padding is zeroed afterwards as the full step
    does.  Every block is still computed by the same serial code, so the
    result does not depend on ``threads``."""
    nb, _ = rank_blocks(spec, S, rank)
    if threads <= 1 or nb < 2:
        return shard_step(spec, m, S, rank, grads, state, hp, t, bases=bases)
    lib()
    cuts = np.linspace(0, nb, min(threads, nb) + 1).astype(np.int64)
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=len(cuts) - 1) as ex:
        futs = [ex.submit(shard_step, spec, m, S, rank, grads, state, hp, t, bases, np.arange(a, b))
                for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
        for f in futs:
            f.result()
    covered = np.zeros(S, dtype=bool)
    for k in range(len(np.asarray(spec).reshape(-1, 5))):
        sl = slice_(spec, m, S, rank, k)
        if sl is not None:
            covered[sl[0]:sl[0] + sl[2] - sl[1]] = True
    state["grad_shard"][~covered] = 0
    state["param_shard"][~covered] = 0
    return state


def new_state(spec, S: int, rank: int, master: np.ndarray) -> dict:
    """Zero optimizer state (codes and scales 0) around an fp32 master shard."""
    nb, _ = rank_blocks(spec, S, rank)
    return dict(grad_shard=np.zeros(S, np.uint16), master=np.array(master, np.float32, copy=True),
                m_q=np.zeros(S, np.int8), v_q=np.zeros(S, np.int8),
                m_scale=np.zeros(nb, np.float32), v_scale=np.zeros(nb, np.float32),
                param_shard=np.zeros(S, np.uint16))
