"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Small workloads are compared element by element over
several teacher-forced steps; edge-case layouts exercise every kernel path
(small groups of 1..64 lanes, workgroup blocks, two-pass huge blocks,
unaligned and misaligned data, empty ranks, padding)."""

from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from synth import CONFIGS, TensorDef, plan_p0
from synth.configs import Config
from synth.layout import Layout

from edge_layouts import EDGE, explicit_layout as _explicit
from gpu_common import (DEV, Guarded, RankProblem, Tally, block_ids, compare, oracle_step, scale_bound,
                        to_dev_u16, CANARY16)
from helpers import hp32, layout_of

pytestmark = pytest.mark.gpu


def _ve():
    import ragged_shard_optimizer_amd as ve
    return ve


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _ranks(lay, limit=6):
    if lay.fsdp <= limit:
        return list(range(lay.fsdp))
    return sorted({0, 1, lay.fsdp // 2, lay.largest_rank(), lay.fsdp - 1})


def _run_parity(cfg, lay, ranks, steps, tally, bucket=0):
    import torch
    ve = _ve()
    hp = hp32()
    plan = ve.Plan(lay.spec_array(), lay.fsdp, lay.shard, device=0)
    for r in ranks:
        prob = RankProblem(ve, cfg, lay, plan, r, bucket)
        valid = lay.valid_mask(r)
        ids = block_ids(lay, r)
        for t in range(1, steps + 1):
            prob.set_grads(t)
            before = prob.download()
            _say(f"[gpu] {cfg.name} rank {r} step {t}: S={lay.shard} blocks={prob.nb}")
            plan.step(r, prob.table, hp, t)
            torch.cuda.synchronize()
            got = prob.download()
            want = oracle_step(prob, before, hp, t)
            bounds = scale_bound(before, want["grad_shard"], ids, prob.nb, hp)
            compare(got, want, valid, hp["lr"], tally, where=f"{cfg.name} r{r} t{t}", bounds=bounds)
        assert prob.guards_intact(), f"guard band overwritten {cfg.name} r{r}"
    plan.close()


SMALL = ["toy_mix", "toy_r1", "toy_r4", "toy_r16", "toy_tile", "llama_mini", "llama_rowblk", "gptoss_mini",
         "deepseek_mini", "adversarial_mini"]


@pytest.mark.parametrize("name", SMALL)
def test_step_parity(name):
    cfg, lay = layout_of(name)
    tally = Tally(name)
    _run_parity(cfg, lay, _ranks(lay), cfg.steps if name.startswith("toy") else 2, tally)
    tally.check()


@pytest.mark.parametrize("name", ["toy_mix", "toy_tile", "llama_mini", "deepseek_mini", "adversarial_mini"])
def test_copy_in_bit_exact(name):
    import torch
    ve = _ve()
    cfg, lay = layout_of(name)
    plan = ve.Plan(lay.spec_array(), lay.fsdp, lay.shard, device=0)
    from synth.data import host_grads
    grads = host_grads(cfg, lay, 0, 1)
    gt = ve.grad_pointer_table([to_dev_u16(g) for g in grads])
    for r in _ranks(lay) + [-1]:
        n = lay.shard * (lay.fsdp if r < 0 else 1)
        out = Guarded(n, torch.int16, CANARY16)
        _say(f"[gpu] copy-in {name} rank {r} n={n}")
        plan.copy_in(r, gt, out.view)
        torch.cuda.synchronize()
        want = oracle.copy_in(lay.spec_array(), lay.fsdp, lay.shard, r, grads)
        assert np.array_equal(out.view.cpu().numpy().view(np.uint16), want), (name, r)
        assert out.guards_intact()
        # zero-copy extraction: every tensor piece read back through its slice
        got = out.view.cpu().numpy().view(np.uint16)
        for k in range(len(lay.tensors)):
            sl = plan.slice(r, k)
            if sl:
                off, lo, hi = sl
                assert np.array_equal(got[off:off + hi - lo], grads[k][lo:hi])
    plan.close()


def test_copy_in_rejects_short_gradient_per_table():
    """The binding checks each gradient table once per rank; a second table
    with a short gradient is still rejected after a good one was used."""
    import torch
    ve = _ve()
    cfg, lay = layout_of("toy_mix")
    plan = ve.Plan(lay.spec_array(), lay.fsdp, lay.shard, device=0)
    from synth.data import host_grads
    grads = [to_dev_u16(g) for g in host_grads(cfg, lay, 0, 1)]
    out = torch.zeros(lay.shard, dtype=torch.int16, device=DEV)
    plan.copy_in(1, ve.grad_pointer_table(grads), out)
    k = plan.pieces(1)[0][0]
    short = list(grads)
    short[k] = grads[k][:1]
    with pytest.raises(ValueError, match="missing or short"):
        plan.copy_in(1, ve.grad_pointer_table(short), out)
    torch.cuda.synchronize()
    plan.close()


# ---------------------------------------------------------------------------
# edge-case layouts, placed by hand (edge_layouts.py)
@pytest.mark.parametrize("case", list(EDGE))
def test_edge_layouts(case):
    cfg, lay = EDGE[case]()
    tally = Tally(cfg.name)
    _run_parity(cfg, lay, list(range(lay.fsdp)), 3, tally)
    tally.check()


# Workgroup blocks take one of three access forms: linear (one contiguous run,
# or tiles whose rows hold a whole number of workgroup sweeps), per-chunk
# offsets (other tiles), general (chunks not all full and aligned).  Each
# tensor below lands in one form; every launch shape here holds its largest
# block, so the forced shape is the one launched.
FORM_TENSORS = [
    TensorDef("tile32", 200, 512, 64, 128),  # 64x128 tiles: 32 chunks per row, divides every T
    TensorDef("tile24", 130, 384, 64, 96),   # 64x96 tiles: 24 chunks per row, divides no T
    TensorDef("rows", 37, 1024, 4, 1024),    # contiguous 4096-element blocks, 1-row last panel
    TensorDef("odd", 50, 102, 25, 102),      # 2550-element row blocks: a partial last chunk
]


@pytest.mark.parametrize("shape", [(256, 8), (512, 4), (1024, 2), (1024, 8), (512, 16), (512, 24), (768, 15),
                                   (1024, 7)])
def test_workgroup_access_forms(shape):
    ve = _ve()
    lay = plan_p0(FORM_TENSORS, 2)
    assert max(t.block_rows * t.block_cols for t in FORM_TENSORS) <= 4 * shape[0] * shape[1]
    cfg = Config("forms", list(FORM_TENSORS), fsdp=2, grad_scale=1e-3, steps=2)
    tally = Tally(cfg.name)
    with ve.options(wg_threads=shape[0], wg_gpt=shape[1]):
        assert (ve.get_option("wg_threads"), ve.get_option("wg_gpt")) == shape
        _run_parity(cfg, lay, [0, 1], 2, tally)
    tally.check()


# The row-block shapes of one workgroup per CU (512 threads with 14 to 24
# groups per thread, 768 threads, 1024 threads with 7 to 10) run persistent:
# each workgroup takes blocks from the rank's
# ticket counter and brings the next contiguous block's gradient and codes
# into LDS during its own phase 2.  Enough blocks that every workgroup runs
# many of them, with staged rows (spans of a multiple of 16 elements),
# contiguous rows that are not staged, tiles and general blocks mixed in one
# launch; three steps in a row also check that each launch leaves the
# counters at zero for the next.
DYN_TENSORS = [
    TensorDef("rows", 1536, 2048, 2, 2048),      # 4,096-element rows: staged
    TensorDef("rows8", 1200, 1000, 5, 1000),     # 5,000-element rows: 5,000 % 16 = 8, not staged
    TensorDef("tile", 512, 512, 64, 128),        # 64x128 tiles
    TensorDef("odd", 50, 102, 25, 102),          # partial last chunk: general form
]


@pytest.mark.parametrize("shape", [(512, 14), (512, 16), (512, 20), (512, 24), (768, 10), (768, 15), (1024, 7),
                                   (1024, 10)])
def test_persistent_row_shapes(shape):
    ve = _ve()
    lay = plan_p0(DYN_TENSORS, 2)
    assert max(t.block_rows * t.block_cols for t in DYN_TENSORS) <= 4 * shape[0] * shape[1]
    cfg = Config("dyn", list(DYN_TENSORS), fsdp=2, grad_scale=1e-3, steps=3)
    tally = Tally(cfg.name)
    with ve.options(wg_threads=shape[0], wg_gpt=shape[1], wg_dynamic=2):
        _run_parity(cfg, lay, [0, 1], 3, tally)
    tally.check()


def test_persistent_equals_one_shot():
    """Three buckets in one call, persistent form against the one-shot
    launch (wg_dynamic=0) on copies of the same states: bit-identical over
    two steps."""
    import torch
    ve = _ve()
    lay = plan_p0(DYN_TENSORS, 2)
    cfg = Config("dyn", list(DYN_TENSORS), fsdp=2, grad_scale=1e-3, steps=2)
    plan = ve.Plan(lay.spec_array(), lay.fsdp, lay.shard, device=0)
    hp = hp32()
    r = 1
    sets = []
    for _ in range(2):
        probs = [RankProblem(ve, cfg, lay, plan, r, bucket=b) for b in range(3)]
        states = []
        for p in probs:
            p.set_grads(1)
            st = {k: b.view for k, b in p.buf.items()}
            st["grad_table"] = p.gt
            states.append(st)
        sets.append((probs, ve.state_table(plan, r, states)))
    _say("[gpu] dyn x3 persistent vs one-shot, 512 x 16")
    with ve.options(wg_threads=512, wg_gpt=16):
        for t in (1, 2):
            with ve.options(wg_dynamic=2):
                plan.step(r, sets[0][1], hp, t)
            with ve.options(wg_dynamic=0):
                plan.step(r, sets[1][1], hp, t)
    torch.cuda.synchronize()
    for p, q in zip(sets[0][0], sets[1][0]):
        a, b = p.download(), q.download()
        for k in a:
            assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k
        assert p.guards_intact() and q.guards_intact()
    plan.close()


# Whole-row blocks of 2,048 and 4,096 groups (rows of 8K and 16K elements)
# run persistent in items of 4 or 2 consecutive blocks streamed as one span,
# each block keeping its own absmax and scales.  Pieces whose block count is
# not a multiple of the item size (a short last item), a one-row last panel
# inside an item (that item goes block by block through the general code),
# and 8,190-element rows (2,048 groups, not whole groups: every item of that
# tensor goes block by block).
ROW_TENSORS = [
    TensorDef("r16k", 61, 16384, 1, 16384),   # 4,096 groups: 2 blocks an item
    TensorDef("r8k", 203, 8192, 1, 8192),     # 2,048 groups: 4 blocks an item
    TensorDef("r2x4k", 301, 4096, 2, 4096),   # 2-row blocks, 1-row last panel
    TensorDef("r8190", 30, 8190, 1, 8190),    # 2,048 groups with a partial last one
]


def _row_layout(steps):
    lay = plan_p0(ROW_TENSORS, 2)
    return Config("rows", list(ROW_TENSORS), fsdp=2, grad_scale=1e-3, steps=steps), lay


def test_row_items_parity():
    ve = _ve()
    cfg, lay = _row_layout(3)
    for r in (0, 1):  # each rank holds ragged pieces of the row tensors
        nbl = {lay.tensors[k].name: (hi - lo) // lay.tensors[k].unit for k, lo, hi, *_ in lay.chunk_intervals(r)}
        assert any(n % 4 for n in nbl.values()), nbl
    tally = Tally(cfg.name)
    with ve.options(wg_dynamic=2, wg_rows=1):
        _run_parity(cfg, lay, [0, 1], 3, tally)
    tally.check()


def _twin_sets(ve, cfg, lay, plan, r, n_buckets):
    sets = []
    for _ in range(2):
        probs = [RankProblem(ve, cfg, lay, plan, r, bucket=b) for b in range(n_buckets)]
        states = []
        for p in probs:
            p.set_grads(1)
            st = {k: b.view for k, b in p.buf.items()}
            st["grad_table"] = p.gt
            states.append(st)
        sets.append((probs, ve.state_table(plan, r, states)))
    return sets


def _assert_twins_equal(sets):
    for p, q in zip(sets[0][0], sets[1][0]):
        a, b = p.download(), q.download()
        for k in a:
            assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k
        assert p.guards_intact() and q.guards_intact()


def test_row_items_equal_one_shot():
    """Three buckets in one call, the multi-block items against one-shot
    launches (wg_rows = 0: one workgroup a block) on copies of the same
    states: bit-identical over two steps, on both ranks."""
    import torch
    ve = _ve()
    cfg, lay = _row_layout(2)
    plan = ve.Plan(lay.spec_array(), lay.fsdp, lay.shard, device=0)
    hp = hp32()
    for r in (0, 1):
        sets = _twin_sets(ve, cfg, lay, plan, r, 3)
        _say(f"[gpu] rows x3 rank {r}: row items vs one-shot")
        for t in (1, 2):
            with ve.options(wg_dynamic=2, wg_rows=1):
                plan.step(r, sets[0][1], hp, t)
            with ve.options(wg_dynamic=2, wg_rows=0):
                plan.step(r, sets[1][1], hp, t)
        torch.cuda.synchronize()
        _assert_twins_equal(sets)
    plan.close()


def test_row_items_misaligned_state_buffers():
    """State arrays shifted by one element: every row item goes block by
    block through the general code, bit-identical to aligned arrays."""
    import torch
    ve = _ve()
    cfg, lay = _row_layout(1)
    plan = ve.Plan(lay.spec_array(), lay.fsdp, lay.shard, device=0)
    hp = hp32()
    r = 0
    prob = RankProblem(ve, cfg, lay, plan, r)
    prob.set_grads(1)
    shifted = {}
    for k, b in prob.buf.items():
        big = torch.zeros(b.view.numel() + 1, dtype=b.view.dtype, device=DEV)
        big[1:].copy_(b.view)
        shifted[k] = big[1:]
    st = dict(shifted)
    st["grad_table"] = prob.gt
    table = ve.state_table(plan, r, [st])
    _say("[gpu] rows rank 0, misaligned state arrays")
    with ve.options(wg_dynamic=2, wg_rows=1):
        plan.step(r, prob.table, hp, 1)
        plan.step(r, table, hp, 1)
    torch.cuda.synchronize()
    for k in prob.buf:
        a = prob.buf[k].view.cpu().numpy()
        b = shifted[k].cpu().numpy()
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), k
    plan.close()


# The two persistent kernels that take work from the rank's counters: the
# row-block form (forced to 512 x 16 on DYN_TENSORS) and the row items.
PERSISTENT_FORMS = {
    "rowblock": (DYN_TENSORS, dict(wg_threads=512, wg_gpt=16, wg_dynamic=2), 1),
    "rowitems": (ROW_TENSORS, dict(wg_dynamic=2, wg_rows=1), 0),
}


def _persistent_form(name, steps):
    tensors, opts, rank = PERSISTENT_FORMS[name]
    lay = plan_p0(tensors, 2)
    return Config(name, list(tensors), fsdp=2, grad_scale=1e-3, steps=steps), lay, opts, rank


@pytest.mark.parametrize("form", list(PERSISTENT_FORMS))
def test_persistent_step_replays_in_a_captured_graph(form):
    """Each persistent launch's last workgroup resets the rank's counters, so
    a captured step replays: three replays, with eager steps of another
    bucket on the same plan and rank in between, each bit-identical to an
    eager step of a twin bucket."""
    import torch
    ve = _ve()
    cfg, lay, opts, r = _persistent_form(form, 2)
    plan = ve.Plan(lay.spec_array(), lay.fsdp, lay.shard, device=0)
    hp = hp32()
    # cap and twin: two copies of bucket 0's state and gradients
    cap, twin, other = (RankProblem(ve, cfg, lay, plan, r, bucket=b) for b in (0, 0, 1))
    cap.set_grads(1)
    twin.set_grads(1)
    other.set_grads(2)
    torch.cuda.synchronize()
    a, b = cap.download(), twin.download()
    assert all(np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)) for k in a)
    with ve.options(**opts):
        _say(f"[gpu] {form} step captured in a graph, rank {r}")
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        with torch.cuda.graph(g, stream=side):
            plan.step(r, cap.table, hp, 3)
        torch.cuda.synchronize()
        for i in range(3):
            _say(f"[gpu] replay {i}")
            g.replay()
            plan.step(r, twin.table, hp, 3)
            plan.step(r, other.table, hp, 4 + i)
            torch.cuda.synchronize()
            a, b = cap.download(), twin.download()
            for k in a:
                assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), (i, k)
    assert cap.guards_intact() and twin.guards_intact() and other.guards_intact()
    del g
    plan.close()


@pytest.mark.parametrize("form", list(PERSISTENT_FORMS))
def test_persistent_steps_of_two_ranks_overlap_on_two_streams(form):
    """Each rank has its own scheduler counters, so step calls for different
    ranks of one plan may run at the same time: ranks 0 and 1 on two
    streams with no ordering between them, three steps, each equal to the
    same steps run one after another on twin buckets."""
    import torch
    ve = _ve()
    cfg, lay, opts, _ = _persistent_form(form, 3)
    plan = ve.Plan(lay.spec_array(), lay.fsdp, lay.shard, device=0)
    hp = hp32()
    run = {r: RankProblem(ve, cfg, lay, plan, r) for r in (0, 1)}
    twin = {r: RankProblem(ve, cfg, lay, plan, r) for r in (0, 1)}
    for p in list(run.values()) + list(twin.values()):
        p.set_grads(1)
    streams = {0: torch.cuda.Stream(), 1: torch.cuda.Stream()}
    torch.cuda.synchronize()
    _say(f"[gpu] {form}, ranks 0 and 1 on two streams")
    with ve.options(**opts):
        for t in (1, 2, 3):
            for r in (0, 1):
                plan.step(r, run[r].table, hp, t, streams[r])
        for t in (1, 2, 3):
            for r in (0, 1):
                plan.step(r, twin[r].table, hp, t)
    torch.cuda.synchronize()
    for r in (0, 1):
        a, b = run[r].download(), twin[r].download()
        for k in a:
            assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), (r, k)
        assert run[r].guards_intact() and twin[r].guards_intact()
    plan.close()


@pytest.mark.parametrize("form", list(PERSISTENT_FORMS))
def test_persistent_steps_of_one_rank_on_two_streams_are_ordered(form):
    """Two buckets of one rank stepped alternately on two streams with no
    ordering by the caller: the library makes each call on a new stream wait
    for the rank's previous one (the counters admit one launch at a time),
    so every bucket equals the same steps run one after another."""
    import torch
    ve = _ve()
    cfg, lay, opts, r = _persistent_form(form, 3)
    plan = ve.Plan(lay.spec_array(), lay.fsdp, lay.shard, device=0)
    hp = hp32()
    run = [RankProblem(ve, cfg, lay, plan, r, bucket=b) for b in (0, 1)]
    twin = [RankProblem(ve, cfg, lay, plan, r, bucket=b) for b in (0, 1)]
    for p in run + twin:
        p.set_grads(1)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    _say(f"[gpu] {form}, rank {r}, two buckets on two streams")
    with ve.options(**opts):
        for t in (1, 2, 3):
            for b in (0, 1):
                plan.step(r, run[b].table, hp, t, streams[b])
        for t in (1, 2, 3):
            for b in (0, 1):
                plan.step(r, twin[b].table, hp, t)
    torch.cuda.synchronize()
    for b in (0, 1):
        x, y = run[b].download(), twin[b].download()
        for k in x:
            assert np.array_equal(x[k].view(np.uint8), y[k].view(np.uint8)), (b, k)
    plan.close()


# A rank holding the end of one tensor and rows of another with smaller
# blocks takes one launch per block shape (llama_mini rank 4: 3,584- and
# 1,024-element rows; llama_rowblk rank 20: 28,672-element rows of `down`,
# then 512-element rows of q, k, v, o).
@pytest.mark.parametrize("name,rank", [("llama_mini", 4), ("llama_rowblk", 20)])
def test_rank_with_two_block_shapes(name, rank):
    cfg, lay = layout_of(name)
    sizes = {lay.tensors[k].block_rows * lay.tensors[k].cols for k, *_ in lay.chunk_intervals(rank)}
    assert len([b for b in sizes if b > 256]) > 1  # two workgroup-path block sizes
    tally = Tally(cfg.name)
    _run_parity(cfg, lay, [rank], 2, tally)
    tally.check()


# One call, two persistent launches on the rank's counters: 28,672-element
# rows (the row-block form, 1024 x 7) and 8,192-element rows (row items),
# as on LLaMA's rank 35; three steps, so each launch must leave the counters
# at zero for the next.
MIXED_PERSISTENT = [
    TensorDef("down", 40, 28672, 1, 28672),
    TensorDef("gate", 301, 8192, 1, 8192),
]


def test_rank_with_row_blocks_and_row_items():
    ve = _ve()
    lay = plan_p0(MIXED_PERSISTENT, 2)
    cfg = Config("mixed", list(MIXED_PERSISTENT), fsdp=2, grad_scale=1e-3, steps=3)
    both = [r for r in (0, 1) if {lay.tensors[k].name for k, *_ in lay.chunk_intervals(r)} == {"down", "gate"}]
    assert both, "a rank holding both tensors"
    tally = Tally(cfg.name)
    with ve.options(wg_dynamic=2, wg_rows=1):
        _run_parity(cfg, lay, both, 3, tally)
    tally.check()


def test_one_element_blocks_codes_exact():
    # 1-element blocks: every nonzero code is +-127 and the scale is |m|/127
    cfg, lay = _explicit("unit", [TensorDef("a", 999, 1, 1, 1), TensorDef("b", 21, 17, 1, 1)], [0, 1008], 2, 768)
    tally = Tally(cfg.name)
    _run_parity(cfg, lay, [0, 1], 3, tally)
    assert tally.mismatch == 0


def test_misaligned_state_buffers_take_scalar_path():
    """State arrays shifted by one element (not 16-byte aligned) must give
    bit-identical results to aligned ones."""
    import torch
    ve = _ve()
    cfg, lay = layout_of("toy_mix")
    plan = ve.Plan(lay.spec_array(), lay.fsdp, lay.shard, device=0)
    hp = hp32()
    r = 1
    prob = RankProblem(ve, cfg, lay, plan, r)
    prob.set_grads(1)
    S, nb = lay.shard, prob.nb
    shifted = {}
    for k, b in prob.buf.items():
        n = b.view.numel()
        big = torch.zeros(n + 1, dtype=b.view.dtype, device=DEV)
        big[1:].copy_(b.view)
        shifted[k] = big[1:]
    st = dict(shifted)
    st["grad_table"] = prob.gt
    table = ve.state_table(plan, r, [st])
    _say("[gpu] misaligned toy_mix rank 1")
    plan.step(r, prob.table, hp, 1)
    plan.step(r, table, hp, 1)
    torch.cuda.synchronize()
    for k in prob.buf:
        a = prob.buf[k].view.cpu().numpy()
        b = shifted[k].cpu().numpy()
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), k
    plan.close()


def test_batched_states_equal_single_calls_and_deterministic():
    import torch
    ve = _ve()
    cfg, lay = layout_of("gptoss_mini")
    plan = ve.Plan(lay.spec_array(), lay.fsdp, lay.shard, device=0)
    hp = hp32()
    r = 0
    probs = [RankProblem(ve, cfg, lay, plan, r, bucket=b) for b in range(3)]
    for p in probs:
        p.set_grads(1)
    twins = [RankProblem(ve, cfg, lay, plan, r, bucket=b) for b in range(3)]
    for p in twins:
        p.set_grads(1)
    states = []
    for p in probs:
        st = {k: b.view for k, b in p.buf.items()}
        st["grad_table"] = p.gt
        states.append(st)
    batched = ve.state_table(plan, r, states)
    _say("[gpu] batched gptoss_mini x3")
    for t in (1, 2):
        plan.step(r, batched, hp, t)
        for p in twins:
            plan.step(r, p.table, hp, t)
    torch.cuda.synchronize()
    for p, q in zip(probs, twins):
        a, b = p.download(), q.download()
        for k in a:
            assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k
    plan.close()


def test_state_table_of_another_rank_or_plan_is_rejected():
    """A state table is sized and checked for one plan and rank; the binding
    refuses it for another before anything is launched (the outputs keep
    their canaries)."""
    import torch
    ve = _ve()
    cfg, lay = layout_of("toy_mix")
    plan = ve.Plan(lay.spec_array(), lay.fsdp, lay.shard, device=0)
    other = ve.Plan(lay.spec_array(), lay.fsdp, lay.shard, device=0)
    prob = RankProblem(ve, cfg, lay, plan, 1)
    prob.set_grads(1)
    before = prob.download()
    hp = hp32()
    with pytest.raises(ValueError, match="another plan or rank"):
        plan.step(2, prob.table, hp, 1)
    with pytest.raises(ValueError, match="another plan or rank"):
        other.step(1, prob.table, hp, 1)
    torch.cuda.synchronize()
    after = prob.download()
    for k in before:
        assert np.array_equal(before[k].view(np.uint8), after[k].view(np.uint8)), k
    plan.step(1, prob.table, hp, 1)  # the matching plan and rank still run
    torch.cuda.synchronize()
    other.close()
    plan.close()
