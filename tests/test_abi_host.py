"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every symbol ve.h declares, validates layouts, and its layout queries agree
with the oracle's."""

from __future__ import annotations

import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle
import ragged_shard_optimizer_amd as ve
from synth import CONFIGS, plan_p0

from helpers import layout_of

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "ve.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ve_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_symbols()
    assert set(names) == set(ve.EXPORTS)
    L = C.CDLL(ve.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_last_error_after_bad_call():
    rc = ve.lib().ve_plan_query(None, 0, None, None, None)
    assert rc == ve.VE_ERR_INVALID_ARG
    assert b"plan is NULL" in ve.lib().ve_last_error()


@pytest.mark.parametrize("name", list(CONFIGS))
def test_host_plan_matches_oracle_layout(name):
    cfg, lay = layout_of(name)
    spec = lay.spec_array()
    plan = ve.Plan(spec, lay.fsdp, lay.shard, device=-1)
    ranks = range(lay.fsdp) if lay.fsdp <= 64 else sorted({0, 1, lay.fsdp // 2, lay.largest_rank(), lay.fsdp - 1})
    rng = np.random.default_rng(0)
    for r in ranks:
        nb, nv = oracle.rank_blocks(spec, lay.shard, r)
        v, b, nseg = plan.query(r)
        assert (v, b) == (nv, nb), (r, v, b, nv, nb)
        on_rank = [k for k, *_ in lay.chunk_intervals(r)]
        assert nseg == len(on_rank)
        ks = range(len(lay.tensors))
        if len(lay.tensors) > 300:   # large buckets: the rank's tensors plus a sample of the rest
            ks = sorted(set(on_rank) | set(rng.choice(len(lay.tensors), 200, replace=False).tolist()))
        for k in ks:
            got = plan.slice(r, k)
            want = oracle.slice_(spec, lay.fsdp, lay.shard, r, k)
            assert got == want, (r, k, got, want)
    for k in range(0, len(lay.tensors), max(1, len(lay.tensors) // 50)):
        assert plan.slice(-1, k) == oracle.slice_(spec, lay.fsdp, lay.shard, -1, k)
    plan.close()


@pytest.mark.parametrize("spec,m,S,status", [
    ([[4, 8, 2, 8, 0], [4, 8, 2, 8, 30]], 2, 32, ve.VE_ERR_LAYOUT),     # overlap
    ([[4, 8, 2, 8, 0]], 2, 24, ve.VE_ERR_LAYOUT),                      # cut inside a unit
    ([[4, 8, 1, 8, 40]], 2, 32, ve.VE_ERR_LAYOUT),                     # outside the bucket
    ([[4, 8, 1, 3, 0]], 1, 32, ve.VE_ERR_LAYOUT),                      # block_cols does not divide
    ([[0, 8, 1, 8, 0]], 1, 32, ve.VE_ERR_LAYOUT),                      # empty tensor
    ([[4, 8, 1, 8, -1]], 1, 32, ve.VE_ERR_LAYOUT),                     # negative offset
    ([[4, 8, 1, 8, 0]], 0, 32, ve.VE_ERR_INVALID_ARG),                 # no ranks
    ([[4, 8, 1, 8, 0]], 1, 0, ve.VE_ERR_INVALID_ARG),                  # empty chunk
    ([[1 << 16, 1 << 15, 1 << 16, 1 << 15, 0]], 1, 1 << 31, ve.VE_ERR_UNSUPPORTED),  # 2^31-element block
])
def test_plan_rejects(spec, m, S, status):
    with pytest.raises(ve.VeError) as e:
        ve.Plan(np.array(spec), m, S, device=-1)
    assert e.value.status == status
    # the oracle agrees on what is a layout error
    if status == ve.VE_ERR_LAYOUT:
        with pytest.raises(oracle.OracleError):
            oracle.validate(np.array(spec), m, S)


def test_plan_accepts_partial_panels_and_empty_bucket():
    p = ve.Plan(np.array([[10, 4, 4, 4, 0]]), 3, 16, device=-1)
    assert p.query(2) == (8, 1, 1)
    assert p.slice(2, 0) == (0, 32, 40)
    e = ve.Plan(np.zeros((0, 5), np.int64), 2, 16, device=-1)
    assert e.query(1) == (0, 0, 0)


def test_host_plan_refuses_kernels():
    p = ve.Plan(np.array([[4, 8, 1, 8, 0]]), 1, 32, device=-1)
    rc = ve.lib().ve_dbuffer_copy_in(p.handle, 0, C.c_void_p(16), C.c_void_p(16), None)
    assert rc == ve.VE_ERR_INVALID_ARG
    hp = ve.AdamHParams(1e-3, 0.9, 0.999, 1e-8, 0.01)
    rc = ve.lib().ve_shard_adam8bit_step(p.handle, 0, C.c_void_p(16), 1, C.byref(hp), 1, None)
    assert rc == ve.VE_ERR_INVALID_ARG


def test_step_argument_checks():
    p = ve.Plan(np.array([[4, 8, 1, 8, 0]]), 2, 16, device=-1)
    hp = ve.AdamHParams(1e-3, 0.9, 0.999, 1e-8, 0.01)
    L = ve.lib()
    assert L.ve_shard_adam8bit_step(p.handle, 2, C.c_void_p(16), 1, C.byref(hp), 1, None) == ve.VE_ERR_INVALID_ARG
    assert L.ve_shard_adam8bit_step(p.handle, 0, None, 1, C.byref(hp), 1, None) == ve.VE_ERR_INVALID_ARG
    assert L.ve_shard_adam8bit_step(p.handle, 0, C.c_void_p(16), 0, C.byref(hp), 1, None) == ve.VE_ERR_INVALID_ARG
    assert L.ve_shard_adam8bit_step(p.handle, 0, C.c_void_p(16), 1, C.byref(hp), 0, None) == ve.VE_ERR_INVALID_ARG
    bad = ve.AdamHParams(1e-3, 1.0, 0.999, 1e-8, 0.01)
    assert L.ve_shard_adam8bit_step(p.handle, 0, C.c_void_p(16), 1, C.byref(bad), 1, None) == ve.VE_ERR_INVALID_ARG
    assert L.ve_dbuffer_slice(p.handle, 0, 5, C.byref(C.c_int64()), C.byref(C.c_int64()),
                              C.byref(C.c_int64())) == ve.VE_ERR_INVALID_ARG


def test_group_op_argument_checks():
    # host-only plan: every call is refused before anything reaches a device
    p = ve.Plan(np.array([[4, 8, 1, 8, 0]]), 2, 16, device=-1)
    L = ve.lib()
    ops = C.c_void_p(16)   # never dereferenced: every call below is refused first
    assert L.ve_dbuffer_group_op(None, 0, ve.GROUP_ZERO, 1.0, ops, 1, None) == ve.VE_ERR_INVALID_ARG
    assert L.ve_dbuffer_group_op(p.handle, 2, ve.GROUP_ZERO, 1.0, ops, 1, None) == ve.VE_ERR_INVALID_ARG
    assert L.ve_dbuffer_group_op(p.handle, -2, ve.GROUP_ZERO, 1.0, ops, 1, None) == ve.VE_ERR_INVALID_ARG
    assert L.ve_dbuffer_group_op(p.handle, 0, 3, 1.0, ops, 1, None) == ve.VE_ERR_INVALID_ARG
    assert "unknown group op" in ve.lib().ve_last_error().decode()
    assert L.ve_dbuffer_group_op(p.handle, 0, -1, 1.0, ops, 1, None) == ve.VE_ERR_INVALID_ARG
    assert L.ve_dbuffer_group_op(p.handle, 0, ve.GROUP_SCALE, 1.0, ops, -1, None) == ve.VE_ERR_INVALID_ARG
    assert L.ve_dbuffer_group_op(p.handle, 0, ve.GROUP_SCALE, 1.0, ops, 65536, None) == ve.VE_ERR_INVALID_ARG
    assert L.ve_dbuffer_group_op(p.handle, 0, ve.GROUP_SCALE, 1.0, None, 1, None) == ve.VE_ERR_INVALID_ARG
    assert L.ve_dbuffer_group_op(p.handle, -1, ve.GROUP_ACCUMULATE, 1.0, ops, 1, None) == ve.VE_ERR_INVALID_ARG
    assert "host-only" in ve.lib().ve_last_error().decode()


def test_tensor_spanning_many_ranks_and_unsorted_specs():
    # specs in any order; a 1-D tensor crossing several chunks of 128-element units
    specs = np.array([[2048, 1, 128, 1, 256], [100, 1, 1, 1, 0], [37, 2, 1, 2, 112]])
    oracle.validate(specs, 6, 384)
    p = ve.Plan(specs, 6, 384, device=-1)
    for r in range(6):
        nb, nv = oracle.rank_blocks(specs, 384, r)
        assert p.query(r)[:2] == (nv, nb)
        for k in range(3):
            assert p.slice(r, k) == oracle.slice_(specs, 6, 384, r, k)


def test_muon_workspace_and_argument_checks():
    # sizing is pure host arithmetic: X, X^T twice (m*n each), A and B (m*m), norm partials
    ve_ = ve
    m, n = 8192, 28672
    got = ve_.muon_workspace_bytes(m, n)
    assert got >= 2 * 2 * (m * n * 2) + 2 * (m * m * 2)
    assert ve_.muon_workspace_bytes(n, m) == got            # orientation does not matter
    L = ve_.lib()
    b = C.c_int64()
    assert L.ve_muon_workspace_bytes(0, 5, C.byref(b)) == ve_.VE_ERR_INVALID_ARG
    assert L.ve_muon_workspace_bytes(5, 5, None) == ve_.VE_ERR_INVALID_ARG
    assert L.ve_muon_workspace_bytes(1 << 31, 1 << 31, C.byref(b)) == ve_.VE_ERR_UNSUPPORTED
    # every rejection below happens before any device call
    p = C.c_void_p(256)
    need = ve_.muon_workspace_bytes(8, 8)
    ns = L.ve_muon_newton_schulz
    assert ns(None, p, 8, 8, 5, 1e-7, p, need, None) == ve_.VE_ERR_INVALID_ARG
    assert ns(p, p, 0, 8, 5, 1e-7, p, need, None) == ve_.VE_ERR_INVALID_ARG
    assert ns(p, p, 8, 8, 65, 1e-7, p, need, None) == ve_.VE_ERR_INVALID_ARG
    assert ns(p, p, 8, 8, 5, float("nan"), p, need, None) == ve_.VE_ERR_INVALID_ARG
    assert ns(p, p, 8, 8, 5, 1e-7, p, need - 1, None) == ve_.VE_ERR_INVALID_ARG
    assert "workspace" in ve_.lib().ve_last_error().decode()
    assert ns(p, p, 8, 8, 5, 1e-7, C.c_void_p(272), need, None) == ve_.VE_ERR_INVALID_ARG
    assert "aligned" in ve_.lib().ve_last_error().decode()
    gm = L.ve_gemm_bf16_nt
    assert gm(None, 8, p, 8, None, 0, p, 8, None, 0, 8, 8, 8, 1.0, 0.0, 0, None) == ve_.VE_ERR_INVALID_ARG
    assert gm(p, 8, p, 8, None, 0, None, 0, None, 0, 8, 8, 8, 1.0, 0.0, 0, None) == ve_.VE_ERR_INVALID_ARG
    assert gm(p, 4, p, 8, None, 0, p, 8, None, 0, 8, 8, 8, 1.0, 0.0, 0, None) == ve_.VE_ERR_INVALID_ARG
    assert gm(p, 8, p, 8, None, 0, p, 8, None, 0, 8, 4, 8, 1.0, 0.0, 1, None) == ve_.VE_ERR_INVALID_ARG
    assert gm(p, 8, p, 8, p, 4, p, 8, None, 0, 8, 8, 8, 1.0, 0.5, 0, None) == ve_.VE_ERR_INVALID_ARG


def test_stream_copy_rejects_bad_arguments_without_a_device():
    L = ve.lib()
    buf = C.create_string_buffer(64)
    base = C.addressof(buf)
    a16 = (base + 15) // 16 * 16
    P = C.c_void_p
    assert L.ve_stream_copy(P(a16), P(a16 + 32), 0, None) == ve.VE_OK          # empty: nothing to do
    assert L.ve_stream_copy(P(a16), P(a16 + 32), -16, None) == ve.VE_ERR_INVALID_ARG
    assert L.ve_stream_copy(None, P(a16), 16, None) == ve.VE_ERR_INVALID_ARG
    assert L.ve_stream_copy(P(a16 + 1), P(a16 + 32), 16, None) == ve.VE_ERR_INVALID_ARG
    assert b"multiples of 16" in L.ve_last_error()
    assert L.ve_stream_copy(P(a16), P(a16 + 32), 24, None) == ve.VE_ERR_INVALID_ARG
    assert L.ve_stream_copy(P(a16), P(a16 + 16), 32, None) == ve.VE_ERR_INVALID_ARG
    assert b"overlap" in L.ve_last_error()


def test_options_round_trip_and_restore():
    before = {k: ve.get_option(k) for k in ("wg_threads", "wg_gpt", "gemm_split", "gemm_cfg", "gemm_xcd",
                                            "wg_dynamic", "wg_rows")}
    assert before["gemm_split"] in (0, 1) and before["gemm_xcd"] in (0, 1) and before["wg_dynamic"] in (0, 1)
    assert before["wg_rows"] in (0, 1)
    with ve.options(wg_threads=512, gemm_split=0, wg_dynamic=0, wg_rows=0):
        assert ve.get_option("wg_threads") == 512 and ve.get_option("gemm_split") == 0
        assert ve.get_option("wg_dynamic") == 0 and ve.get_option("wg_rows") == 0
    assert {k: ve.get_option(k) for k in before} == before
    L = ve.lib()
    assert L.ve_set_option(b"no_such_option", 1) == ve.VE_ERR_INVALID_ARG
    assert b"unknown option" in L.ve_last_error()
    assert L.ve_get_option(b"wg_gpt", None) == ve.VE_ERR_INVALID_ARG
