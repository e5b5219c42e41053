"""Checkpoint and resume of the GPU step through per-tensor arrays: two steps
under FSDP size 4, the state written out per tensor (np.savez), read back
under FSDP size 4 and under 2 and 1, one more step -- each equal bit for bit
to running on without the checkpoint."""

from __future__ import annotations

import sys

import numpy as np
import pytest

from synth import CONFIGS, plan_p0
from synth.data import host_grads, host_master

import ckpt_common as ck
from gpu_common import DEV, to_dev_u16
from helpers import hp32

pytestmark = pytest.mark.gpu


def _gpu_run(ve, lay, cfg, store, t, hp):
    """One step of every rank on the GPU from per-tensor state."""
    import torch
    plan = ve.Plan(lay.spec_array(), lay.fsdp, lay.shard, device=0)
    gt = ve.grad_pointer_table([to_dev_u16(g) for g in host_grads(cfg, lay, 0, t)])
    out = {}
    for r in range(lay.fsdp):
        host = ck.tensors_to_shard(lay, r, store)
        st = {f: torch.from_numpy(host[f].view(np.int16) if host[f].dtype == np.uint16 else host[f]).to(DEV)
              for f in ck.STATE + ck.SCALES}
        st["grad_table"] = gt
        if st["m_scale"].numel() == 0:
            st["m_scale"] = torch.zeros(1, dtype=torch.float32, device=DEV)
            st["v_scale"] = torch.zeros(1, dtype=torch.float32, device=DEV)
        plan.step(r, ve.state_table(plan, r, [st]), hp, t)
        torch.cuda.synchronize()
        got = {f: st[f].cpu().numpy() for f in ck.STATE + ck.SCALES}
        for f in ("param_shard", "grad_shard"):
            got[f] = got[f].view(np.uint16)
        nb = len(host["m_scale"])
        got["m_scale"], got["v_scale"] = got["m_scale"][:nb], got["v_scale"][:nb]
        ck.shard_to_tensors(lay, r, got, out)
    plan.close()
    return out


@pytest.mark.parametrize("name", ["toy_mix", "toy_tile"])
def test_gpu_resume_after_checkpoint_equals_running_on(name, tmp_path):
    import ragged_shard_optimizer_amd as ve
    import oracle
    cfg = CONFIGS[name]
    hp = hp32()
    lay = plan_p0(cfg.tensors, cfg.fsdp)
    store = {}
    for r in range(lay.fsdp):
        ck.shard_to_tensors(lay, r, oracle.new_state(lay.spec_array(), lay.shard, r, host_master(cfg, lay, 0, r)),
                            store)
    for t in (1, 2):
        print(f"[gpu] checkpoint {name}: step {t} under FSDP {lay.fsdp}", flush=True)
        store = _gpu_run(ve, lay, cfg, store, t, hp)
    ck.save(store, tmp_path / "ckpt.npz")
    running = _gpu_run(ve, lay, cfg, store, 3, hp)
    for m2 in (4, 2, 1):
        print(f"[gpu] checkpoint {name}: resume under FSDP {m2}", flush=True)
        resumed = _gpu_run(ve, plan_p0(cfg.tensors, m2), cfg, ck.load(tmp_path / "ckpt.npz"), 3, hp)
        assert ck.same(running, resumed), (name, m2)
