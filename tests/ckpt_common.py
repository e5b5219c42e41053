"""Checkpoint helpers: an optimizer state moves between a rank's shard
(shard coordinates, the rank-local block order) and per-tensor arrays
(tensor coordinates, the tensor's own block order).  Per-tensor arrays are
what a distributed checkpoint stores; they do not depend on the FSDP size,
so a checkpoint written under one layout can be loaded under another."""

from __future__ import annotations

import os

import numpy as np

STATE = ("master", "m_q", "v_q", "param_shard", "grad_shard")
SCALES = ("m_scale", "v_scale")
_DT = {"master": np.float32, "m_q": np.int8, "v_q": np.int8, "param_shard": np.uint16, "grad_shard": np.uint16,
       "m_scale": np.float32, "v_scale": np.float32}


def _pieces(lay, rank):
    """(tensor, elem_lo, elem_hi, shard_dst, first local block, blocks) in rank-local block order."""
    out, blk = [], 0
    for k, lo, hi, dst in sorted(lay.chunk_intervals(rank), key=lambda x: x[3]):
        t = lay.tensors[k]
        tiles = t.cols // t.block_cols
        nb = (-(-hi // t.unit) - lo // t.unit) * tiles
        out.append((k, lo, hi, dst, blk, nb))
        blk += nb
    return out


def shard_to_tensors(lay, rank, state, store):
    """Scatter one rank's state arrays into ``store`` (tensor name -> arrays)."""
    for k, lo, hi, dst, b0, nb in _pieces(lay, rank):
        t = lay.tensors[k]
        tiles = t.cols // t.block_cols
        rec = store.setdefault(t.name, {**{f: np.zeros(t.numel, _DT[f]) for f in STATE},
                                        **{f: np.zeros(-(-t.rows // t.block_rows) * tiles, _DT[f]) for f in SCALES}})
        for f in STATE:
            rec[f][lo:hi] = state[f][dst:dst + hi - lo]
        first = lo // t.unit * tiles
        for f in SCALES:
            rec[f][first:first + nb] = state[f][b0:b0 + nb]


def tensors_to_shard(lay, rank, store):
    """One rank's state arrays gathered from ``store`` (padding zero)."""
    S = lay.shard
    pcs = _pieces(lay, rank)
    nb_total = sum(p[5] for p in pcs)
    state = {**{f: np.zeros(S, _DT[f]) for f in STATE}, **{f: np.zeros(max(nb_total, 1), _DT[f]) for f in SCALES}}
    for k, lo, hi, dst, b0, nb in pcs:
        t = lay.tensors[k]
        tiles = t.cols // t.block_cols
        rec = store[t.name]
        for f in STATE:
            state[f][dst:dst + hi - lo] = rec[f][lo:hi]
        first = lo // t.unit * tiles
        for f in SCALES:
            state[f][b0:b0 + nb] = rec[f][first:first + nb]
    for f in SCALES:
        state[f] = state[f][:nb_total].copy() if nb_total else state[f][:0].copy()
    return state


def save(store, path):
    """One .npz per checkpoint (plain arrays, no pickling)."""
    flat = {f"{name}/{f}": a for name, rec in store.items() for f, a in rec.items()}
    np.savez(path, **flat)


def load(path):
    store = {}
    with np.load(path, allow_pickle=False) as z:
        for key in z.files:
            name, f = key.rsplit("/", 1)
            store.setdefault(name, {})[f] = z[key]
    return store


def same(a, b):
    """Per-tensor stores equal bit for bit."""
    if a.keys() != b.keys():
        return False
    return all(np.array_equal(a[n][f].view(np.uint8), b[n][f].view(np.uint8)) for n in a for f in a[n])
