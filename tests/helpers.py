"""Shared test plumbing: build seeded host inputs for a workload and map the
rank-local block order to (tensor, panel, tile) coordinates."""

from __future__ import annotations

import numpy as np

from synth import CONFIGS, HPARAMS, plan_p0
from synth.data import host_grads, host_master, tensors_on_rank


def layout_of(cfg_or_name):
    cfg = CONFIGS[cfg_or_name] if isinstance(cfg_or_name, str) else cfg_or_name
    return cfg, plan_p0(cfg.tensors, cfg.fsdp)


def rank_block_coords(layout, rank):
    """[(k, panel, tile)] in the rank's block order: pieces by ascending bucket
    offset, row panels top to bottom, tiles left to right."""
    out = []
    for k, lo, hi, _dst in sorted(layout.chunk_intervals(rank), key=lambda x: x[3]):
        t = layout.tensors[k]
        unit = t.unit
        for p in range(lo // unit, -(-hi // unit)):
            for j in range(t.cols // t.block_cols):
                out.append((k, p, j))
    return out


def hp32():
    return {k: float(np.float32(v)) for k, v in HPARAMS.items()}


def ulp_diff_f32(a, b):
    """Distance in units in the last place between two fp32 arrays."""
    ai = np.ascontiguousarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.ascontiguousarray(b, np.float32).view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)


__all__ = ["layout_of", "rank_block_coords", "hp32", "ulp_diff_f32", "host_grads", "host_master",
           "tensors_on_rank"]
