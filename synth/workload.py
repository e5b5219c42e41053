"""Full-size seeded inputs on the GPU for one rank of a workload.

For each of the ``n_buckets`` identical buckets: the per-parameter bf16
gradients of the tensors that have a piece on the rank (others are None --
the shard step never reads them) and the rank's fp32 master shard.  Values
come from seeded torch generators on the device, a few draws per bucket.
"""

from __future__ import annotations

from .configs import Config
from .data import device_grads, device_master
from .layout import Layout


def rank_tensors(lay: Layout, rank: int):
    return sorted({k for k, *_ in lay.chunk_intervals(rank)})


def device_buckets(cfg: Config, lay: Layout, rank: int, device, n_buckets: int | None = None, step: int = 0):
    """List over buckets of ``(grads, master)``; ``grads[k]`` is a flat int16
    view of tensor k's bf16 gradient or None."""
    import torch
    n_buckets = cfg.n_buckets if n_buckets is None else n_buckets
    on_rank = set(rank_tensors(lay, rank))
    mask = torch.from_numpy(lay.valid_mask(rank)).to(device)
    out = []
    for b in range(n_buckets):
        drawn = device_grads(cfg, lay, b, sorted(on_rank), device, step)
        grads = [drawn.get(k) for k in range(len(lay.tensors))]
        master = device_master(cfg, lay, b, rank, device, mask=mask)
        out.append((grads, master))
    return out


def whole_bucket_grads(cfg: Config, lay: Layout, device, bucket: int = 0, step: int = 0):
    """Every tensor's bf16 gradient of one bucket (flat int16 views)."""
    drawn = device_grads(cfg, lay, bucket, range(len(lay.tensors)), device, step)
    return [drawn[k] for k in range(len(lay.tensors))]
