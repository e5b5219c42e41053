"""Checkpoint and resume through per-tensor arrays, on the oracle: k steps,
save, load under the same FSDP size or another one, one more step -- equal
bit for bit to running on without the checkpoint.  Under another FSDP size
this is the sync-free property again: a block's update never depends on
which rank holds it."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import CONFIGS, plan_p0
from synth.data import host_grads, host_master

import ckpt_common as ck
from helpers import hp32


def _run(lay, cfg, stores_in, t, hp):
    """One step of every rank from per-tensor state; returns the new per-tensor state."""
    out = {}
    spec, m, S = lay.spec_array(), lay.fsdp, lay.shard
    grads = host_grads(cfg, lay, 0, t)
    for r in range(m):
        st = ck.tensors_to_shard(lay, r, stores_in)
        oracle.shard_step(spec, m, S, r, grads, st, hp, t)
        ck.shard_to_tensors(lay, r, st, out)
    return out


def _initial(lay, cfg):
    store = {}
    for r in range(lay.fsdp):
        st = oracle.new_state(lay.spec_array(), lay.shard, r, host_master(cfg, lay, 0, r))
        ck.shard_to_tensors(lay, r, st, store)
    return store


@pytest.mark.parametrize("name,m2", [("toy_mix", 4), ("toy_mix", 2), ("toy_mix", 3), ("toy_tile", 2), ("toy_r16", 1)])
def test_resume_after_checkpoint_equals_running_on(name, m2, tmp_path):
    cfg = CONFIGS[name]
    hp = hp32()
    lay = plan_p0(cfg.tensors, cfg.fsdp)
    store = _initial(lay, cfg)
    for t in (1, 2):
        store = _run(lay, cfg, store, t, hp)
    ck.save(store, tmp_path / "ckpt.npz")
    running = _run(lay, cfg, store, 3, hp)                 # without the checkpoint
    lay2 = plan_p0(cfg.tensors, m2)
    resumed = _run(lay2, cfg, ck.load(tmp_path / "ckpt.npz"), 3, hp)
    assert ck.same(running, resumed), (name, m2)
    # and the checkpoint itself round-trips bit for bit
    assert ck.same(store, ck.load(tmp_path / "ckpt.npz"))
