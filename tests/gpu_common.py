"""GPU-test plumbing: put seeded host inputs on the device around guard bands,
run the library, pull results back, and compare with the oracle under the
parity gates."""

from __future__ import annotations

import os

import numpy as np

import oracle
from synth.data import host_grads, host_master

DEV = "cuda:0"
GUARD = 4096          # elements of guard band on each side (keeps 16-byte alignment)
GUARD_BYTE = 0xA5
CANARY16 = -1         # 0xFFFF in an int16 buffer: padding must come back as 0

# parity gates: fp32 master relative error (lr floor) 1e-5; codes may differ
# by one step in at most 0.01% of elements; scales within the fp32 evaluation
# bound of the moments they are taken from (scale_bound below).
MASTER_RTOL = 1e-5
CODE_MAX_FRAC = 1e-4
U32 = 2.0 ** -24  # fp32 unit roundoff


class Guarded:
    """A device buffer with guard bands of GUARD_BYTE on both sides."""

    def __init__(self, n, dtype, fill=None):
        import torch
        self.n = n
        itemsize = torch.empty((), dtype=dtype).element_size()
        self.raw = torch.full(((2 * GUARD + max(n, 1)) * itemsize,), GUARD_BYTE, dtype=torch.uint8, device=DEV)
        self.view = self.raw[GUARD * itemsize:(GUARD + max(n, 1)) * itemsize].view(dtype)[:max(n, 1)]
        if fill is not None:
            self.view.fill_(fill)

    def guards_intact(self) -> bool:
        itemsize = self.view.element_size()
        g = GUARD * itemsize
        return bool((self.raw[:g] == GUARD_BYTE).all()) and bool((self.raw[-g:] == GUARD_BYTE).all())


def to_dev_u16(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


class RankProblem:
    """One bucket on one rank: seeded inputs on the GPU, state in guarded
    buffers, and the matching host arrays for the oracle."""

    def __init__(self, ve, cfg, lay, plan, rank, bucket=0):
        import torch
        self.ve, self.cfg, self.lay, self.plan, self.rank, self.bucket = ve, cfg, lay, plan, rank, bucket
        S = lay.shard
        _, nb, _ = plan.query(rank)
        self.nb = nb
        self.buf = dict(grad_shard=Guarded(S, torch.int16, CANARY16), master=Guarded(S, torch.float32),
                        m_q=Guarded(S, torch.int8, 0), v_q=Guarded(S, torch.int8, 0),
                        m_scale=Guarded(nb, torch.float32, 0.0), v_scale=Guarded(nb, torch.float32, 0.0),
                        param_shard=Guarded(S, torch.int16, CANARY16))
        self.buf["master"].view.copy_(torch.from_numpy(host_master(cfg, lay, bucket, rank)))
        self.grads_host = None
        self.grad_dev = None
        self.table = None

    def set_grads(self, step):
        self.grads_host = host_grads(self.cfg, self.lay, self.bucket, step)
        self.grad_dev = [to_dev_u16(g) for g in self.grads_host]
        self.gt = self.ve.grad_pointer_table(self.grad_dev)
        st = {k: b.view for k, b in self.buf.items()}
        st["grad_table"] = self.gt
        self.table = self.ve.state_table(self.plan, self.rank, [st])

    def download(self) -> dict:
        out = {}
        for k, b in self.buf.items():
            a = b.view.cpu().numpy()
            out[k] = a.view(np.uint16) if k in ("grad_shard", "param_shard") else a
        out["m_scale"] = out["m_scale"][:self.nb].copy()
        out["v_scale"] = out["v_scale"][:self.nb].copy()
        return out

    def guards_intact(self) -> bool:
        return all(b.guards_intact() for b in self.buf.values())


def bf16_of(master: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(master).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


class Tally:
    """Code mismatches of one workload, counted per moment array (m_q and v_q
    apart): each array may differ by one step in at most CODE_MAX_FRAC of its
    elements.  check() gates each array and reports the measured fractions
    (stdout, and a line appended to $VE_PARITY_LOG when that is set)."""

    KEYS = ("m_q", "v_q")

    def __init__(self, name=""):
        self.name = name
        self.elems = {k: 0 for k in self.KEYS}
        self.diff = {k: 0 for k in self.KEYS}

    def add(self, key, d):
        """``d``: |gpu - oracle| of one comparison's codes."""
        self.elems[key] += int(d.size)
        self.diff[key] += int((d != 0).sum())

    @property
    def mismatch(self):
        return sum(self.diff.values())

    def fractions(self):
        return {k: self.diff[k] / max(self.elems[k], 1) for k in self.KEYS}

    def report(self):
        fr = self.fractions()
        line = (f"[parity] {self.name}: m_q {self.diff['m_q']}/{self.elems['m_q']} = {fr['m_q']:.3e}, "
                f"v_q {self.diff['v_q']}/{self.elems['v_q']} = {fr['v_q']:.3e} codes off by one "
                f"(gate {CODE_MAX_FRAC:.0e} each)")
        print(line, flush=True)
        path = os.environ.get("VE_PARITY_LOG")
        if path:
            with open(path, "a") as fh:
                fh.write(line + "\n")
        return line

    def check(self):
        self.report()
        for k in self.KEYS:
            assert self.diff[k] <= CODE_MAX_FRAC * max(self.elems[k], 1), (self.name, k, self.diff[k], self.elems[k])


def block_ids(lay, rank) -> np.ndarray:
    """Rank-local block index of every shard position (-1 in padding), in the
    documented block order."""
    ids = np.full(lay.shard, -1, dtype=np.int64)
    base = 0
    for k, lo, hi, dst in sorted(lay.chunk_intervals(rank), key=lambda x: x[3]):
        t = lay.tensors[k]
        e = np.arange(lo, hi, dtype=np.int64)
        row, col = e // t.cols, e % t.cols
        tiles = t.cols // t.block_cols
        p0 = lo // t.unit
        ids[dst:dst + hi - lo] = base + (row // t.block_rows - p0) * tiles + col // t.block_cols
        base += (-(-hi // t.unit) - p0) * tiles
    return ids


def scale_bound(before: dict, grad_bits: np.ndarray, ids: np.ndarray, nb: int, hp: dict):
    """Per-block admissible |scale_gpu - scale_oracle| for m and v.

    The kernel's fp32 moment m1 = fl(beta1*fl(q*s) + fl((1-beta1)*g)) differs
    from the exactly rounded one by at most 3u*(|beta1*m0| + |(1-beta1)*g|)
    (three roundings against one); the block absmax inherits the largest such
    bound, and each side's scale adds half an ulp.  Same for v."""
    valid = ids >= 0
    g = (grad_bits[valid].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    blk = ids[valid]
    m0 = before["m_q"][valid].astype(np.float64) * before["m_scale"][blk].astype(np.float64)
    v0 = before["v_q"][valid].astype(np.float64) * before["v_scale"][blk].astype(np.float64)
    b1, b2 = hp["beta1"], hp["beta2"]
    em = np.abs(b1 * m0) + np.abs((1 - b1) * g)
    ev = np.abs(b2 * v0) + np.abs((1 - b2) * g * g)
    Mm, Mv = np.zeros(nb), np.zeros(nb)
    np.maximum.at(Mm, blk, em)
    np.maximum.at(Mv, blk, ev)
    return 4 * U32 * Mm / 127.0, 4 * U32 * Mv / 127.0


def compare(got: dict, want: dict, valid: np.ndarray, lr: float, tally: Tally, where="", bounds=None):
    """Parity gates between a GPU result and the oracle's, on one shard."""
    # pack/unpack: bit exact, padding zero
    assert np.array_equal(got["grad_shard"], want["grad_shard"]), f"grad_shard {where}"
    assert not got["param_shard"][~valid].any(), f"param padding {where}"
    # fp32 master
    g, w = got["master"][valid].astype(np.float64), want["master"][valid].astype(np.float64)
    rel = np.abs(g - w) / np.maximum(np.abs(w), lr)
    assert rel.size == 0 or rel.max() <= MASTER_RTOL, f"master rel {rel.max():.3g} {where}"
    assert np.array_equal(got["master"][~valid].view(np.uint32), want["master"][~valid].view(np.uint32)), \
        f"master padding touched {where}"
    # bf16 param is the round-to-nearest-even image of the GPU's own master
    assert np.array_equal(got["param_shard"][valid], bf16_of(got["master"][valid])), f"param != bf16(master) {where}"
    # codes: off by at most one, in a tiny fraction of elements
    for key in ("m_q", "v_q"):
        d = np.abs(got[key][valid].astype(np.int16) - want[key][valid].astype(np.int16))
        assert d.size == 0 or d.max() <= 1, f"{key} differs by {d.max()} {where}"
        tally.add(key, d)
        assert np.array_equal(got[key][~valid], want[key][~valid]), f"{key} padding touched {where}"
    assert got["v_q"].min() >= 0
    # scales: within the fp32 evaluation bound of the moments, plus one ulp
    for key, bnd in zip(("m_scale", "v_scale"), bounds):
        g, w = got[key].astype(np.float64), want[key].astype(np.float64)
        ulp = np.spacing(np.abs(want[key])).astype(np.float64)
        excess = np.abs(g - w) - (bnd + ulp)
        assert excess.size == 0 or excess.max() <= 0, \
            f"{key} off by {np.abs(g - w)[excess.argmax()]:.3g} (bound {(bnd + ulp)[excess.argmax()]:.3g}) {where}"


def oracle_step(prob: RankProblem, before: dict, hp: dict, t: int) -> dict:
    """The oracle's result for one step from ``before`` (copied)."""
    st = {k: v.copy() for k, v in before.items()}
    oracle.shard_step(prob.lay.spec_array(), prob.lay.fsdp, prob.lay.shard, prob.rank, prob.grads_host, st, hp, t)
    return st
