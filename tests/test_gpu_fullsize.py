"""Full-size workloads in the launch configuration the benchmark times (all
buckets of a workload in one call): sampled blocks against the oracle, the
whole gradient slice and padding through properties that hold at any size."""

from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from synth.workload import device_buckets

from gpu_common import DEV, Tally, bf16_of, MASTER_RTOL, U32
from helpers import hp32, layout_of, rank_block_coords

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _download(st, nb):
    out = {}
    for k in ("grad_shard", "master", "m_q", "v_q", "m_scale", "v_scale", "param_shard"):
        a = st[k].cpu().numpy()
        out[k] = a.view(np.uint16) if k in ("grad_shard", "param_shard") else a
    out["m_scale"] = out["m_scale"][:nb].copy()
    out["v_scale"] = out["v_scale"][:nb].copy()
    return out


def _block_positions(lay, rank, coord):
    k, p, j = coord
    t = lay.tensors[k]
    (_, lo, _, dst) = next(x for x in lay.chunk_intervals(rank) if x[0] == k)
    r0, r1 = p * t.block_rows, min((p + 1) * t.block_rows, t.rows)
    rows = np.arange(r0, r1, dtype=np.int64)[:, None]
    cols = np.arange(j * t.block_cols, (j + 1) * t.block_cols, dtype=np.int64)[None, :]
    return (dst + rows * t.cols + cols - lo).reshape(-1)


# The benchmark's rank with every bucket in one call, then with two buckets:
# the rank that straddles two tensors of different block geometry
# (LLaMA 35: the end of `down` and rows of q; DeepSeek 42: gate/up panels
# then down panels) and the last rank (padding at the bucket's tail).
FULL_RANKS = [("llama", "largest"), ("gptoss", "largest"), ("deepseek", "largest"), ("adversarial", "largest"),
              ("llama", 35), ("llama", "last"), ("gptoss", "last"), ("deepseek", 42), ("deepseek", "last"),
              ("adversarial", "last")]


@pytest.mark.parametrize("name,which", FULL_RANKS)
def test_full_size_sampled(name, which):
    import torch
    import ragged_shard_optimizer_amd as ve
    cfg, lay = layout_of(name)
    rank = lay.largest_rank() if which == "largest" else (lay.fsdp - 1 if which == "last" else which)
    spec, m, S = lay.spec_array(), lay.fsdp, lay.shard
    hp = hp32()
    plan = ve.Plan(spec, m, S, device=0)
    _, nb, _ = plan.query(rank)
    n_buckets = cfg.n_buckets if which == "largest" else min(2, cfg.n_buckets)
    _say(f"[gpu] full-size {name}: rank {rank}, {n_buckets} buckets, S={S}, blocks={nb}")
    buckets = device_buckets(cfg, lay, rank, DEV, n_buckets=n_buckets)
    states = [ve.new_state(plan, rank, ve.grad_pointer_table(g, DEV), master) for g, master in buckets]
    table = ve.state_table(plan, rank, states)
    coords = rank_block_coords(lay, rank)
    assert len(coords) == nb
    rng = np.random.default_rng(0)
    sel = sorted({0, nb - 1} | set(rng.choice(nb, min(nb, 10), replace=False).tolist()))
    sample_b = sorted({0, n_buckets // 2, n_buckets - 1})
    pieces = list(lay.chunk_intervals(rank))
    mask = torch.from_numpy(lay.valid_mask(rank)).to(DEV)
    tally = Tally(f"full-size {name} rank {rank}")
    for t in (1, 2):
        pre = {b: _download(states[b], nb) for b in sample_b}
        _say(f"[gpu] full-size {name}: step {t}, {len(states)} states in one call")
        plan.step(rank, table, hp, t)
        torch.cuda.synchronize()
        for b in sample_b:
            grads_dev, _ = buckets[b]
            # whole gradient slice: every piece bit-exact, padding zero (on the device)
            gs = states[b]["grad_shard"]
            for k, lo, hi, dst in pieces:
                assert torch.equal(gs[dst:dst + hi - lo], grads_dev[k][lo:hi]), (name, b, k)
            assert not gs[~mask].any() and not states[b]["param_shard"][~mask].any()
            # sampled blocks through the oracle
            got = _download(states[b], nb)
            grads, bases = [None] * len(lay.tensors), [0] * len(lay.tensors)
            for k, lo, hi, dst in pieces:
                grads[k] = grads_dev[k][lo:hi].cpu().numpy().view(np.uint16)
                bases[k] = lo
            want = {k: v.copy() for k, v in pre[b].items()}
            oracle.shard_step(spec, m, S, rank, grads, want, hp, t, bases=bases, blocks=sel)
            for blk in sel:
                pos = _block_positions(lay, rank, coords[blk])
                g, w = got["master"][pos].astype(np.float64), want["master"][pos].astype(np.float64)
                rel = np.abs(g - w) / np.maximum(np.abs(w), hp["lr"])
                assert rel.max() <= MASTER_RTOL, (name, b, blk, rel.max())
                assert np.array_equal(got["param_shard"][pos], bf16_of(got["master"][pos]))
                for key in ("m_q", "v_q"):
                    d = np.abs(got[key][pos].astype(np.int16) - want[key][pos].astype(np.int16))
                    assert d.max() <= 1, (name, key, blk)
                    tally.add(key, d)
                # scales within the fp32 evaluation bound of the block's moments
                g = (got["grad_shard"][pos].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
                pb = pre[b]
                m0 = pb["m_q"][pos].astype(np.float64) * float(pb["m_scale"][blk])
                v0 = pb["v_q"][pos].astype(np.float64) * float(pb["v_scale"][blk])
                bm = 4 * U32 * (np.abs(hp["beta1"] * m0) + np.abs((1 - hp["beta1"]) * g)).max() / 127
                bv = 4 * U32 * (np.abs(hp["beta2"] * v0) + np.abs((1 - hp["beta2"]) * g * g)).max() / 127
                for key, bnd in (("m_scale", bm), ("v_scale", bv)):
                    gs_, ws_ = float(got[key][blk]), float(want[key][blk])
                    assert abs(gs_ - ws_) <= bnd + float(np.spacing(np.float32(abs(ws_)))), (key, blk, gs_, ws_)
    tally.check()
    del states, table, buckets
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["llama", "gptoss"])
def test_full_size_persistent_equals_one_shot(name):
    """Every element of every bucket on the benchmark's rank: the persistent,
    ticket-scheduled step (the default for these row blocks) against the
    one-shot launch (wg_dynamic = 0) on copies of the same states, two steps,
    bit-identical.  The sampled test above checks the persistent form against
    the oracle at these sizes; this one reaches every block it schedules."""
    import torch
    import ragged_shard_optimizer_amd as ve
    cfg, lay = layout_of(name)
    rank = lay.largest_rank()
    plan = ve.Plan(lay.spec_array(), lay.fsdp, lay.shard, device=0)
    hp = hp32()
    buckets = device_buckets(cfg, lay, rank, DEV)
    _say(f"[gpu] full-size {name}: rank {rank}, {len(buckets)} buckets, persistent vs one-shot")
    dyn = [ve.new_state(plan, rank, ve.grad_pointer_table(g, DEV), m) for g, m in buckets]
    one = [ve.new_state(plan, rank, ve.grad_pointer_table(g, DEV), m.clone()) for g, m in buckets]
    t_dyn, t_one = ve.state_table(plan, rank, dyn), ve.state_table(plan, rank, one)
    keys = ("grad_shard", "master", "m_q", "v_q", "m_scale", "v_scale", "param_shard")
    for t in (1, 2):
        with ve.options(wg_dynamic=2):
            plan.step(rank, t_dyn, hp, t)
        with ve.options(wg_dynamic=0):
            plan.step(rank, t_one, hp, t)
        torch.cuda.synchronize()
        for b, (x, y) in enumerate(zip(dyn, one)):
            for k in keys:
                assert torch.equal(x[k], y[k]), (name, t, b, k)
    del dyn, one, t_dyn, t_one, buckets
    plan.close()
    torch.cuda.empty_cache()


def test_full_size_row_items_equal_one_shot():
    """A LLaMA rank that holds only 8,192-element rows (93 of the 128 ranks
    hold such rows; rank 36 nothing else): every bucket stepped in items of
    four rows against one workgroup a row (wg_rows = 0), two steps,
    bit-identical."""
    import torch
    import ragged_shard_optimizer_amd as ve
    cfg, lay = layout_of("llama")
    rank = 36
    rows = {lay.tensors[k].block_rows * lay.tensors[k].cols for k, *_ in lay.chunk_intervals(rank)}
    assert rows == {8192}, rows
    plan = ve.Plan(lay.spec_array(), lay.fsdp, lay.shard, device=0)
    hp = hp32()
    buckets = device_buckets(cfg, lay, rank, DEV)
    _say(f"[gpu] full-size llama: rank {rank}, {len(buckets)} buckets, row items vs one-shot")
    itm = [ve.new_state(plan, rank, ve.grad_pointer_table(g, DEV), m) for g, m in buckets]
    one = [ve.new_state(plan, rank, ve.grad_pointer_table(g, DEV), m.clone()) for g, m in buckets]
    t_itm, t_one = ve.state_table(plan, rank, itm), ve.state_table(plan, rank, one)
    keys = ("grad_shard", "master", "m_q", "v_q", "m_scale", "v_scale", "param_shard")
    for t in (1, 2):
        with ve.options(wg_dynamic=2, wg_rows=1):
            plan.step(rank, t_itm, hp, t)
        with ve.options(wg_dynamic=2, wg_rows=0):
            plan.step(rank, t_one, hp, t)
        torch.cuda.synchronize()
        for b, (x, y) in enumerate(zip(itm, one)):
            for k in keys:
                assert torch.equal(x[k], y[k]), (t, b, k)
    del itm, one, t_itm, t_one, buckets
    plan.close()
    torch.cuda.empty_cache()


def test_adversarial_whole_bucket_copy_in():
    """Copy-in of the whole adversarial bucket (10,000 tensors, ~2.9 GB
    moved): every tensor lands at its offset bit for bit, all padding zero."""
    import torch
    import ragged_shard_optimizer_amd as ve
    from synth.workload import whole_bucket_grads
    cfg, lay = layout_of("adversarial")
    plan = ve.Plan(lay.spec_array(), lay.fsdp, lay.shard, device=0)
    grads = whole_bucket_grads(cfg, lay, DEV)
    gt = ve.grad_pointer_table(grads, DEV)
    bucket = torch.full((lay.bucket_elems,), -1, dtype=torch.int16, device=DEV)
    _say(f"[gpu] whole-bucket copy-in: {lay.bucket_elems} elements")
    plan.copy_in(-1, gt, bucket)
    torch.cuda.synchronize()
    covered = torch.zeros(lay.bucket_elems, dtype=torch.bool, device=DEV)
    for k, o in enumerate(lay.offsets):
        n = lay.tensors[k].numel
        assert torch.equal(bucket[o:o + n], grads[k]), k
        covered[o:o + n] = True
    assert not bucket[~covered].any()
    # spot-check against the oracle on a few ranks' chunks
    host = [g.cpu().numpy().view(np.uint16) for g in grads]
    got = bucket.cpu().numpy().view(np.uint16)
    for r in (0, lay.largest_rank(), lay.fsdp - 1):
        want = oracle.copy_in(lay.spec_array(), lay.fsdp, lay.shard, r, host)
        assert np.array_equal(got[r * lay.shard:(r + 1) * lay.shard], want)


def _bf16_noise(n, seed):
    import torch
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randn(n, generator=g, device=DEV).to(torch.bfloat16).view(torch.int16)


@pytest.mark.parametrize("name", ["llama", "gptoss", "deepseek", "adversarial"])
def test_full_size_group_ops(name):
    """Accumulate and scale over every bucket's rank chunk in one launch (the
    shape the benchmark times); sampled buckets compared whole with the
    oracle, bit for bit."""
    import torch
    import ragged_shard_optimizer_amd as ve
    cfg, lay = layout_of(name)
    rank = lay.largest_rank()
    spec, m, S = lay.spec_array(), lay.fsdp, lay.shard
    plan = ve.Plan(spec, m, S, device=0)
    buckets = device_buckets(cfg, lay, rank, DEV)
    gts = [ve.grad_pointer_table(g, DEV) for g, _ in buckets]
    bufs = [_bf16_noise(S, 1000 + b) for b in range(len(buckets))]
    sample_b = sorted({0, len(buckets) // 2, len(buckets) - 1})
    pieces = list(lay.chunk_intervals(rank))
    for op, alpha in ((oracle.GROUP_ACCUMULATE, 0.5), (oracle.GROUP_SCALE, 1.0 / 3.0)):
        pre = {b: bufs[b].cpu().numpy().view(np.uint16).copy() for b in sample_b}
        table = ve.group_table(plan, rank, bufs, gts if op == oracle.GROUP_ACCUMULATE else None)
        _say(f"[gpu] full-size group op {op} {name}: rank {rank}, {len(bufs)} buckets, S={S}")
        plan.group_op(rank, op, alpha, table)
        torch.cuda.synchronize()
        for b in sample_b:
            grads, bases = None, None
            if op == oracle.GROUP_ACCUMULATE:
                grads, bases = [None] * len(lay.tensors), [0] * len(lay.tensors)
                for k, lo, hi, _dst in pieces:
                    grads[k] = buckets[b][0][k][lo:hi].cpu().numpy().view(np.uint16)
                    bases[k] = lo
            want = oracle.group_op(spec, m, S, rank, op, alpha, pre[b], grads=grads, bases=bases)
            got = bufs[b].cpu().numpy().view(np.uint16)
            bad = np.nonzero(got != want)[0]
            assert bad.size == 0, (name, op, b, bad[:5])
    del bufs, gts, buckets
    torch.cuda.empty_cache()


def test_adversarial_whole_bucket_group_scale():
    """Scale of the whole adversarial bucket (10,000 tensors, ~727 M
    elements) against the oracle, bit for bit."""
    import torch
    import ragged_shard_optimizer_amd as ve
    cfg, lay = layout_of("adversarial")
    spec, m, S = lay.spec_array(), lay.fsdp, lay.shard
    plan = ve.Plan(spec, m, S, device=0)
    buf = _bf16_noise(lay.bucket_elems, 77)
    pre = buf.cpu().numpy().view(np.uint16).copy()
    _say(f"[gpu] whole-bucket group scale: {lay.bucket_elems} elements")
    plan.group_op(-1, oracle.GROUP_SCALE, -0.75, ve.group_table(plan, -1, [buf]))
    torch.cuda.synchronize()
    want = oracle.group_op(spec, m, S, -1, oracle.GROUP_SCALE, -0.75, pre)
    assert np.array_equal(buf.cpu().numpy().view(np.uint16), want)
