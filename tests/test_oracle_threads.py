"""The oracle's multi-threaded form (blocks split over host threads, used to
time it on all host cores) gives the serial result bit for bit."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth.data import host_master, host_piece_grads

from helpers import hp32, layout_of


@pytest.mark.parametrize("name,threads", [("toy_mix", 3), ("llama_mini", 4), ("deepseek_mini", 5),
                                          ("adversarial_mini", 8)])
def test_threaded_step_equals_serial(name, threads):
    cfg, lay = layout_of(name)
    spec, m, S = lay.spec_array(), lay.fsdp, lay.shard
    hp = hp32()
    for rank in sorted({0, lay.largest_rank(), m - 1}):
        grads, bases = host_piece_grads(cfg, lay, 0, rank, step=1)
        master = host_master(cfg, lay, 0, rank)
        a = oracle.new_state(spec, S, rank, master)
        b = oracle.new_state(spec, S, rank, master)
        for st in (a, b):   # canaries: the padding must come back zero either way
            st["grad_shard"][:] = 0xFFFF
            st["param_shard"][:] = 0xFFFF
        for t in (1, 2):
            oracle.shard_step(spec, m, S, rank, grads, a, hp, t, bases=bases)
            oracle.shard_step_threads(spec, m, S, rank, grads, b, hp, t, bases=bases, threads=threads)
            for k in a:
                assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), (name, rank, t, k)


def test_block_selection_in_any_order():
    # a selection is a set: order and repeats do not matter
    cfg, lay = layout_of("toy_tile")
    spec, m, S = lay.spec_array(), lay.fsdp, lay.shard
    hp = hp32()
    grads, bases = host_piece_grads(cfg, lay, 0, 1, step=1)
    master = host_master(cfg, lay, 0, 1)
    nb, _ = oracle.rank_blocks(spec, S, 1)
    sel = np.arange(0, nb, 3)
    a = oracle.shard_step(spec, m, S, 1, grads, oracle.new_state(spec, S, 1, master), hp, 1, bases=bases, blocks=sel)
    b = oracle.shard_step(spec, m, S, 1, grads, oracle.new_state(spec, S, 1, master), hp, 1, bases=bases,
                          blocks=np.concatenate([sel[::-1], sel[:2]]))
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k
