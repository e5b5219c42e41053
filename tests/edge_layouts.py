"""Hand-placed bucket layouts that exercise every kernel path: small groups
of 1..64 lanes, workgroup blocks, two-pass huge blocks, unaligned offsets,
ranks holding only padding, tensors straddling several ranks."""

from __future__ import annotations

import oracle
from synth import TensorDef
from synth.configs import Config
from synth.layout import Layout


def explicit_layout(name, tensors, offsets, m, S, grad_scale=1e-3, steps=2):
    lay = Layout(list(tensors), list(offsets), m, S, list(range(len(tensors))))
    oracle.validate(lay.spec_array(), m, S)
    return Config(name, list(tensors), fsdp=m, grad_scale=grad_scale, steps=steps), lay


def _group_sizes_case():
    # one tensor per small-path group size (1..64 lanes) and two workgroup sizes
    ts, offs, cur = [], [], 0
    for i, (rows, cols, br, bc) in enumerate([
            (33, 1, 1, 1), (40, 1, 16, 1), (9, 24, 1, 24), (7, 64, 1, 64), (5, 96, 2, 96),
            (6, 128, 2, 128), (8, 64, 8, 64), (4, 256, 4, 256), (3, 1024, 1, 1024),
            (2, 2048, 2, 2048), (40, 48, 8, 12), (64, 80, 16, 16), (17, 7, 3, 7), (36, 1, 4, 1),
            (24, 1, 8, 1), (10, 3, 1, 3)]):
        ts.append(TensorDef(f"g{i}", rows, cols, br, bc))
        offs.append(cur)
        cur += rows * cols + (16 if i % 2 else 0)
    S = -(-cur // 16) * 16
    return explicit_layout("group_sizes", ts, offs, 1, S)


def _unaligned_case():
    # odd offsets: pieces start at shard positions that are not 16-aligned,
    # chunk boundaries inside tensors stay on units
    ts = [TensorDef("u0", 37, 1, 1, 1), TensorDef("u1", 20, 48, 4, 48), TensorDef("u2", 300, 1, 16, 1),
          TensorDef("u3", 12, 40, 3, 8), TensorDef("u4", 10, 1000, 1, 1000)]
    offs = [3, 41, 1001, 1301, 2000]
    return explicit_layout("unaligned", ts, offs, 4, 3000)


def _huge_case():
    # a block of 96 x 2304 = 221,184 elements: beyond the register-resident path
    ts = [TensorDef("h0", 200, 2304, 96, 2304), TensorDef("h1", 64, 64, 8, 8)]
    return explicit_layout("huge", ts, [0, 200 * 2304 + 16], 1, 200 * 2304 + 16 + 4096)


def _empty_rank_case():
    # ranks 1 and 2 hold only padding; rank 0 a partial bucket
    ts = [TensorDef("e0", 10, 16, 4, 16), TensorDef("e1", 3, 1, 1, 1)]
    return explicit_layout("empty_rank", ts, [0, 160], 3, 256)


def _straddle_case():
    # one tensor over five ranks with a short last panel; another starting mid-chunk
    ts = [TensorDef("s0", 50, 32, 4, 16), TensorDef("s1", 9, 128, 1, 128)]
    return explicit_layout("straddle", ts, [0, 1664], 5, 768)


EDGE = {"group_sizes": _group_sizes_case, "unaligned": _unaligned_case, "huge": _huge_case,
        "empty_rank": _empty_rank_case, "straddle": _straddle_case}
