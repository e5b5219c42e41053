"""Seeded random values: gradients (bf16 bit patterns) and fp32 master weights.

Host arrays come from numpy ``Generator`` streams keyed by
``(seed, bucket, tensor, kind)``; device tensors come from a seeded torch
generator on the GPU (used for the full-size workloads, where host generation
would dominate).  Nothing here computes any part of the optimizer step.
"""

from __future__ import annotations

import numpy as np

from .configs import Config
from .layout import Layout

_KIND_GRAD = 1
_KIND_PARAM = 2


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, via torch's CPU conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def _rng(cfg: Config, bucket: int, k: int, kind: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg.seed, bucket, k, kind]))


def _draw(rng: np.random.Generator, n: int, dist: str) -> np.ndarray:
    if dist == "normal":
        return rng.standard_normal(n)
    if dist == "student_t3":
        z = rng.standard_normal((4, n))
        chi2 = (z[1] ** 2 + z[2] ** 2 + z[3] ** 2) / 3.0
        return z[0] / np.sqrt(chi2)
    raise ValueError(dist)


def host_grads(cfg: Config, layout: Layout, bucket: int, step: int = 0, only=None):
    """Per-tensor bf16 gradients (uint16 bit arrays, length numel) for the
    tensors in ``layout`` order; entries not in ``only`` are None."""
    out = []
    for k, t in enumerate(layout.tensors):
        if only is not None and k not in only:
            out.append(None)
            continue
        rng = _rng(cfg, bucket * 1009 + step, layout.order[k], _KIND_GRAD)
        g = (_draw(rng, t.numel, cfg.grad_dist) * cfg.grad_scale).astype(np.float32)
        out.append(f32_to_bf16_bits(g))
    return out


def host_master(cfg: Config, layout: Layout, bucket: int, rank: int) -> np.ndarray:
    """fp32 master-weight shard of ``rank`` (length S): N(0, param_std) at
    every tensor element, 0 in padding."""
    S = layout.shard
    rng = _rng(cfg, bucket, rank, _KIND_PARAM)
    x = (rng.standard_normal(S) * cfg.param_std).astype(np.float32)
    x[~layout.valid_mask(rank)] = 0.0
    return x


def tensors_on_rank(layout: Layout, rank: int):
    return sorted({k for k, *_ in layout.chunk_intervals(rank)})


# ----------------------------------------------------------------------------
# device-side generation for full-size workloads
def _torch_gen(device, seed_words):
    import torch
    s = int(np.random.SeedSequence(list(seed_words)).generate_state(1, dtype=np.uint64)[0] >> 1)
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


# Tensors drawn together in one flat buffer: at most this many elements per
# draw (bounds the temporaries), each tensor starting on a 256-byte boundary
# (the GPU step takes its vector path only for 16-byte-aligned gradients).
_FLAT_CHUNK = 1 << 28
_FLAT_ALIGN = 128


def device_grads(cfg: Config, layout: Layout, bucket: int, ks, device, step: int = 0):
    """bf16 gradients (flat int16 device views) of tensors ``ks`` of one
    bucket, drawn a few hundred million elements per launch instead of one
    launch per tensor (a bucket of 10,000 tensors is a handful of launches).
    Returns {k: view}; the views of one draw share one allocation."""
    import torch
    ks = list(ks)
    out = {}
    limit = _FLAT_CHUNK // (4 if cfg.grad_dist != "normal" else 1)
    i = 0
    while i < len(ks):
        group, total = [], 0
        while i < len(ks):
            n = layout.tensors[ks[i]].numel
            pad = -n % _FLAT_ALIGN
            if group and total + n > limit:
                break
            group.append((ks[i], total, n))
            total += n + pad
            i += 1
        g = _torch_gen(device, [cfg.seed, bucket * 1009 + step, layout.order[group[0][0]], _KIND_GRAD, 11])
        if cfg.grad_dist == "normal":
            x = torch.randn(total, generator=g, device=device, dtype=torch.float32)
        else:
            z = torch.randn(4, total, generator=g, device=device, dtype=torch.float32)
            x = z[0] / torch.sqrt((z[1] ** 2 + z[2] ** 2 + z[3] ** 2) / 3.0)
            del z
        x.mul_(cfg.grad_scale)
        flat = x.to(torch.bfloat16).view(torch.int16)
        del x
        for k, o, n in group:
            out[k] = flat[o:o + n]
    return out


def host_piece_grads(cfg: Config, layout: Layout, bucket: int, rank: int, step: int = 0):
    """bf16 gradients of the pieces rank ``rank`` holds (the only gradient
    elements its step reads), for the oracle: (grads, bases) with grads[k]
    the uint16 bits of tensor elements [bases[k], bases[k] + len) or None.
    Each piece has its own seeded stream, so a rank's inputs are drawn
    without generating the whole tensors."""
    grads, bases = [None] * len(layout.tensors), [0] * len(layout.tensors)
    for k, lo, hi, _dst in layout.chunk_intervals(rank):
        rng = np.random.default_rng(np.random.SeedSequence([cfg.seed, bucket * 1009 + step, layout.order[k],
                                                            _KIND_GRAD, rank]))
        g = (_draw(rng, hi - lo, cfg.grad_dist) * cfg.grad_scale).astype(np.float32)
        grads[k] = f32_to_bf16_bits(g)
        bases[k] = lo
    return grads, bases


def device_master(cfg: Config, layout: Layout, bucket: int, rank: int, device, mask=None):
    import torch
    g = _torch_gen(device, [cfg.seed, bucket, rank, _KIND_PARAM, 7])
    x = torch.randn(layout.shard, generator=g, device=device, dtype=torch.float32)
    x.mul_(cfg.param_std)
    if mask is None:
        mask = torch.from_numpy(layout.valid_mask(rank)).to(device)
    x.masked_fill_(~mask, 0.0)
    return x
