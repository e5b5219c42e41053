"""GPU parity of the DBuffer group operations (zero, scale, accumulate)
through the C ABI against the CPU oracle, bit for bit: every rank chunk and
the whole bucket of the small workloads and the hand-placed edge layouts,
several buckets per launch, misaligned buffers (2-byte path), special values
(overflow, subnormals, signed zeros) and an accumulate / average sequence.
Full-size buckets in the benchmark's launch shape are compared whole."""

from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from synth.data import f32_to_bf16_bits, host_grads

from edge_layouts import EDGE, explicit_layout
from gpu_common import DEV, Guarded, to_dev_u16
from helpers import layout_of
from synth import TensorDef

pytestmark = pytest.mark.gpu

ZERO, SCALE, ACC = oracle.GROUP_ZERO, oracle.GROUP_SCALE, oracle.GROUP_ACCUMULATE
OPS = [(ZERO, 0.0), (SCALE, 0.37), (SCALE, -1.0 / 3.0), (ACC, 1.0), (ACC, -0.61)]
SMALL = ["toy_mix", "toy_r1", "toy_tile", "llama_mini", "gptoss_mini", "deepseek_mini", "adversarial_mini"]


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


def _start(n, seed):
    """Finite bf16 start contents, nonzero padding included."""
    x = np.random.default_rng(seed).standard_normal(n).astype(np.float32)
    return f32_to_bf16_bits(x)


def _u16(t):
    return t.cpu().numpy().view(np.uint16)


def _run(cfg, lay, ranks, nb=2):
    """Every op on `nb` buckets per launch, each with its own gradients."""
    import torch
    ve = _ve()
    spec, m, S = lay.spec_array(), lay.fsdp, lay.shard
    plan = ve.Plan(spec, m, S, device=0)
    grads = [host_grads(cfg, lay, b, 1) for b in range(nb)]
    gts = [ve.grad_pointer_table([to_dev_u16(g) for g in gb]) for gb in grads]
    for r in ranks:
        n = S * (m if r < 0 else 1)
        for op, alpha in OPS:
            starts = [_start(n, 100 * b + 7 * (r + 1)) for b in range(nb)]
            bufs = [Guarded(n, torch.int16) for _ in range(nb)]
            for b in range(nb):
                bufs[b].view.copy_(to_dev_u16(starts[b]))
            table = ve.group_table(plan, r, [g.view for g in bufs], gts if op == ACC else None)
            _say(f"[gpu] group op {op} alpha {alpha} {cfg.name} rank {r} n={n} buckets={nb}")
            plan.group_op(r, op, alpha, table)
            torch.cuda.synchronize()
            for b in range(nb):
                want = oracle.group_op(spec, m, S, r, op, alpha, starts[b].copy(),
                                       grads=grads[b] if op == ACC else None)
                got = _u16(bufs[b].view)
                bad = np.nonzero(got != want)[0]
                assert bad.size == 0, (cfg.name, r, op, alpha, b, bad[:5], got[bad[:5]], want[bad[:5]])
                assert bufs[b].guards_intact(), (cfg.name, r, op, b)
    plan.close()


@pytest.mark.parametrize("name", SMALL)
def test_group_ops_parity(name):
    cfg, lay = layout_of(name)
    _run(cfg, lay, _ranks(lay) + [-1])


@pytest.mark.parametrize("case", list(EDGE))
def test_group_ops_edge_layouts(case):
    cfg, lay = EDGE[case]()
    _run(cfg, lay, list(range(lay.fsdp)) + [-1], nb=1)


def test_group_ops_misaligned_buffers():
    """Bucket and gradients shifted by one element (2-byte path) give the
    oracle's results bit for bit."""
    import torch
    ve = _ve()
    cfg, lay = layout_of("toy_mix")
    spec, m, S = lay.spec_array(), lay.fsdp, lay.shard
    plan = ve.Plan(spec, m, S, device=0)
    grads = host_grads(cfg, lay, 0, 1)
    gdev = []
    for g in grads:
        big = torch.zeros(g.size + 1, dtype=torch.int16, device=DEV)
        big[1:].copy_(to_dev_u16(g))
        gdev.append(big[1:])
    gt = ve.grad_pointer_table(gdev)
    for r in [0, 1, -1]:
        n = S * (m if r < 0 else 1)
        for op, alpha in OPS:
            start = _start(n, 3 + r)
            big = torch.zeros(n + 1, dtype=torch.int16, device=DEV)
            big[1:].copy_(to_dev_u16(start))
            buf = big[1:]
            _say(f"[gpu] misaligned group op {op} rank {r}")
            plan.group_op(r, op, alpha, ve.group_table(plan, r, [buf], [gt] if op == ACC else None))
            torch.cuda.synchronize()
            want = oracle.group_op(spec, m, S, r, op, alpha, start.copy(), grads=grads if op == ACC else None)
            assert np.array_equal(_u16(buf), want), (r, op)
            assert int(big[0].item()) == 0
    plan.close()


def test_group_ops_special_values():
    """Overflow to infinity, subnormal results, signed zeros, exact ties."""
    import torch
    ve = _ve()
    vals = np.array([3.0e38, -3.0e38, 1.0, -1.0, 2.0 ** -133, -(2.0 ** -133), 2.0 ** -126, 0.0, -0.0,
                     1.0078125, 65504.0, 1e-38, -1e-39, 0.1, -7.5, 2.0 ** -130], np.float32)
    n = 4096 + len(vals) + 5          # a full tile plus a ragged tail
    x = np.resize(vals, n)
    xb = f32_to_bf16_bits(x)
    gb = f32_to_bf16_bits(np.resize(vals[::-1].copy(), n))
    cfg, lay = explicit_layout("special", [TensorDef("s", n, 1, 1, 1)], [0], 1, -(-n // 16) * 16)
    spec, m, S = lay.spec_array(), lay.fsdp, lay.shard
    plan = ve.Plan(spec, m, S, device=0)
    gt = ve.grad_pointer_table([to_dev_u16(gb)])
    start = np.zeros(S, np.uint16)
    start[:n] = xb
    for op, alpha in [(SCALE, 2.0), (SCALE, 0.5), (SCALE, -0.0), (SCALE, 1e-30), (ACC, 1.0), (ACC, -1.0),
                      (ACC, 2.0 ** -7), (ACC, 1.0 + 2.0 ** -23)]:
        buf = to_dev_u16(start)
        plan.group_op(0, op, alpha, ve.group_table(plan, 0, [buf], [gt] if op == ACC else None))
        torch.cuda.synchronize()
        want = oracle.group_op(spec, m, S, 0, op, alpha, start.copy(), grads=[gb] if op == ACC else None)
        got = _u16(buf)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (op, alpha, bad[:5], got[bad[:5]], want[bad[:5]])
    plan.close()


def test_group_accumulate_then_average_sequence():
    """Zero, accumulate three micro-batches, average: the chain matches the
    oracle's chain bit for bit."""
    import torch
    ve = _ve()
    cfg, lay = layout_of("gptoss_mini")
    spec, m, S = lay.spec_array(), lay.fsdp, lay.shard
    plan = ve.Plan(spec, m, S, device=0)
    r = lay.largest_rank()
    buf = Guarded(S, torch.int16, -1)
    host = np.full(S, 0xFFFF, np.uint16)
    micro = [host_grads(cfg, lay, 0, s) for s in range(3)]
    plan.group_op(r, ZERO, 0.0, ve.group_table(plan, r, [buf.view]))
    oracle.group_op(spec, m, S, r, ZERO, 0.0, host)
    for g in micro:
        gt = ve.grad_pointer_table([to_dev_u16(x) for x in g])
        plan.group_op(r, ACC, 1.0, ve.group_table(plan, r, [buf.view], [gt]))
        oracle.group_op(spec, m, S, r, ACC, 1.0, host, grads=g)
        torch.cuda.synchronize()
    plan.group_op(r, SCALE, 1.0 / 3.0, ve.group_table(plan, r, [buf.view]))
    oracle.group_op(spec, m, S, r, SCALE, 1.0 / 3.0, host)
    torch.cuda.synchronize()
    assert np.array_equal(_u16(buf.view), host)
    assert buf.guards_intact()
    plan.close()


def test_group_empty_batch_is_a_no_op():
    ve = _ve()
    cfg, lay = layout_of("toy_mix")
    plan = ve.Plan(lay.spec_array(), lay.fsdp, lay.shard, device=0)
    assert ve.lib().ve_dbuffer_group_op(plan.handle, 0, ZERO, 0.0, None, 0, None) == ve.VE_OK
    plan.close()


@pytest.mark.parametrize("nbytes", [16, 4096, 16 * 1000 + 16, (1 << 24) + 48])
def test_stream_copy_bit_exact(nbytes):
    """The streaming reference copies every byte (grid-stride tail included)
    and nothing past the end."""
    import torch
    import ragged_shard_optimizer_amd as ve
    g = torch.Generator(device="cuda:0")
    g.manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda:0", generator=g)
    dst = torch.full((nbytes + 4096,), 0xA5, dtype=torch.uint8, device="cuda:0")
    print(f"[gpu] stream copy {nbytes} bytes", flush=True)
    ve.stream_copy(dst[:nbytes], src)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert bool((dst[nbytes:] == 0xA5).all())
