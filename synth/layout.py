"""A simple bucket planner (P0) that produces the layouts the shard step consumes.

The pages describe the structure-aware planner as: order the tensors by block
size, largest first, then place each one so that shard boundaries fall on
block boundaries, with padding only *between* tensors and every tensor kept
contiguous (veScale-FSDP talk notes, "Proposed method / 2. Structure-aware
planning algorithm"; Dutch summary, "2B. Structure-aware planning").  The
dynamic-programming placement itself is not specified on the pages; P0 below
is the plain greedy reading:

* stable sort by shard unit (``block_rows * cols``), descending;
* the bucket is ``m`` equal chunks of ``S`` elements (in-place all-gather and
  reduce-scatter need equal chunks; talk notes, "3. DBuffer");
* ``S`` is the smallest multiple of 16 that holds the bucket and is a multiple
  of the unit of every tensor longer than ``S`` (such a tensor may span two or
  more chunk boundaries, which are then ``S`` apart);
* each tensor goes at the smallest 16-aligned offset at or after the cursor
  such that every chunk boundary strictly inside it is a multiple of its unit
  away from its first element; ``S`` grows by one alignment step until the
  bucket fits.

The result is data: a list of ``(rows, cols, block_rows, block_cols,
offset)`` records plus ``S`` and ``m``.  The shard step and the oracle each
validate it independently.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Sequence

import numpy as np

from .configs import TensorDef

ALIGN = 16


@dataclasses.dataclass
class Layout:
    tensors: List[TensorDef]   # in bucket order (ascending offset)
    offsets: List[int]
    fsdp: int                  # m
    shard: int                 # S
    order: List[int]           # order[k] = index of tensors[k] in the input list

    @property
    def bucket_elems(self) -> int:
        return self.fsdp * self.shard

    @property
    def valid_elems(self) -> int:
        return sum(t.numel for t in self.tensors)

    @property
    def padding(self) -> int:
        return self.bucket_elems - self.valid_elems

    def spec_array(self) -> np.ndarray:
        """``int64[n, 5]``: rows, cols, block_rows, block_cols, offset."""
        return np.array([[t.rows, t.cols, t.block_rows, t.block_cols, o]
                         for t, o in zip(self.tensors, self.offsets)], dtype=np.int64).reshape(-1, 5)

    # -- plain interval helpers for building inputs (no optimizer arithmetic) --
    def chunk_intervals(self, rank: int):
        """Yield ``(k, lo, hi, dst)``: tensor k's elements ``[lo, hi)`` land at
        ``[dst, dst + hi - lo)`` of ``rank``'s chunk (rank -1: whole bucket)."""
        if rank < 0:
            c0, c1 = 0, self.bucket_elems
        else:
            c0, c1 = rank * self.shard, (rank + 1) * self.shard
        for k, (t, o) in enumerate(zip(self.tensors, self.offsets)):
            a, b = max(o, c0), min(o + t.numel, c1)
            if a < b:
                yield k, a - o, b - o, a - c0

    def valid_mask(self, rank: int) -> np.ndarray:
        n = self.bucket_elems if rank < 0 else self.shard
        mask = np.zeros(n, dtype=bool)
        for _, lo, hi, dst in self.chunk_intervals(rank):
            mask[dst:dst + hi - lo] = True
        return mask

    def rank_valid(self, rank: int) -> int:
        return sum(hi - lo for _, lo, hi, _ in self.chunk_intervals(rank))

    def largest_rank(self) -> int:
        """The rank holding the most valid elements (lowest index on ties)."""
        best, best_r = -1, 0
        for r in range(self.fsdp):
            v = self.rank_valid(r)
            if v > best:
                best, best_r = v, r
        return best_r


def _lcm(a: int, b: int) -> int:
    return a // math.gcd(a, b) * b


def _place(tensors: Sequence[TensorDef], m: int, S: int):
    cursor = 0
    offs = []
    for t in tensors:
        n, u = t.numel, t.unit
        off = -(-cursor // ALIGN) * ALIGN
        b1 = (off // S + 1) * S              # first chunk boundary after off
        if off + n > b1 and (b1 - off) % u != 0:
            step = _lcm(u, ALIGN)
            # b1 is a multiple of 16 (S is), so off must be congruent to b1 mod lcm(u, 16)
            off = b1 - ((b1 - cursor) // step) * step
            if off < cursor:
                off += step
        offs.append(off)
        cursor = off + n
    return offs, cursor <= m * S


def plan_p0(tensors: Sequence[TensorDef], m: int) -> Layout:
    order = sorted(range(len(tensors)), key=lambda i: -tensors[i].unit)  # stable
    srt = [tensors[i] for i in order]
    total = sum(t.numel for t in srt)
    S = -(-total // m)
    S = -(-S // ALIGN) * ALIGN
    while True:
        step = ALIGN
        for t in srt:
            if t.numel > S:
                step = _lcm(step, t.unit)
        S2 = -(-S // step) * step
        if S2 == S:
            offs, ok = _place(srt, m, S)
            if ok:
                return Layout(list(srt), offs, m, S, order)
            S += step
        else:
            S = S2
