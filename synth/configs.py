"""Bucket definitions for the five workloads and their scaled-down twins.

Every tensor is described as a row-major matrix ``rows x cols`` (a 1-D tensor
is ``numel x 1``) plus its RaggedShard block: ``block_rows`` rows is the shard
unit (the granularity at which a tensor may be cut between ranks) and the
quantisation block is the ``block_rows x block_cols`` tile inside that row
panel.  ``block_cols == cols`` means whole-row blocks.

Shapes follow the model families the pages evaluate (LLaMA-3-70B,
GPT-OSS-120B, DeepSeek-V3; veScale-FSDP talk notes, "Experiments / setup"),
the per-parameter quantisation granularity follows the 8-bit Adam case study
(talk notes, "Case study: 8-bit Adam and distributed Muon": per-parameter
block shape such as 32x32 tiles or 32-row granularity).  Values are synthetic.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List

import numpy as np

# Adam hyper-parameters used for every workload.
HPARAMS = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


@dataclasses.dataclass(frozen=True)
class TensorDef:
    name: str
    rows: int
    cols: int
    block_rows: int
    block_cols: int

    @property
    def numel(self) -> int:
        return self.rows * self.cols

    @property
    def unit(self) -> int:
        """Shard granularity in elements: one row panel of ``block_rows`` rows."""
        return self.block_rows * self.cols


@dataclasses.dataclass
class Config:
    name: str
    tensors: List[TensorDef]      # one bucket, in model (pre-planner) order
    fsdp: int                     # m, number of ranks sharing the bucket
    n_buckets: int = 1            # identical buckets (one per layer)
    grad_dist: str = "normal"     # "normal" or "student_t3"
    grad_scale: float = 1e-3
    param_std: float = 0.02
    steps: int = 3
    seed: int = 0
    description: str = ""

    @property
    def bucket_numel(self) -> int:
        return sum(t.numel for t in self.tensors)


def _rows(name, rows, cols, br, bc=None):
    return TensorDef(name, rows, cols, br, cols if bc is None else bc)


def _vec(name, n, b):
    # a 1-D tensor: n rows of one column; a block of b rows holds b elements
    return TensorDef(name, n, 1, b, 1)


# ----------------------------------------------------------------------------
# Toy bucket: 8 tensors, simulated FSDP size 4.
_TOY_SHAPES = [(64, 48), (128, 64), (48,), (256, 32), (32, 32), (96,), (40, 80), (200,)]


def toy_variants():
    """The toy bucket under several block policies.

    ``mix``: tensor i gets {1,4,16}[i mod 3]-row blocks; ``r1``/``r4``/``r16``:
    uniform row blocks; ``tile``: 16x16 tiles on the 2-D tensors and 16-row
    blocks on the 1-D ones.
    """
    out = {}
    def build(policy):
        ts = []
        for i, s in enumerate(_TOY_SHAPES):
            if policy == "tile":
                if len(s) == 2:
                    ts.append(TensorDef(f"t{i}", s[0], s[1], 16, 16))
                else:
                    ts.append(_vec(f"t{i}", s[0], 16))
                continue
            b = {"mix": [1, 4, 16][i % 3], "r1": 1, "r4": 4, "r16": 16}[policy]
            if len(s) == 2:
                ts.append(_rows(f"t{i}", s[0], s[1], b))
            else:
                ts.append(_vec(f"t{i}", s[0], b))
        return ts
    for p in ["mix", "r1", "r4", "r16", "tile"]:
        out[p] = Config(name=f"toy_{p}", tensors=build(p), fsdp=4, grad_scale=1e-2,
                        steps=3, description=f"toy bucket, {p} blocks, FSDP 4")
    return out


# ----------------------------------------------------------------------------
def llama_bucket(hidden=8192, inter=28672, kv=1024):
    """One LLaMA-3-70B-shaped decoder layer, whole-row blocks (norms: 1 element)."""
    return [
        _rows("q", hidden, hidden, 1), _rows("k", kv, hidden, 1), _rows("v", kv, hidden, 1),
        _rows("o", hidden, hidden, 1), _rows("gate", inter, hidden, 1),
        _rows("up", inter, hidden, 1), _rows("down", hidden, inter, 1),
        _vec("attn_norm", hidden, 1), _vec("mlp_norm", hidden, 1),
    ]


def gptoss_bucket(width=2880, experts=128, expert_rows=(5760, 2880), attn_rows=2880,
                  router_rows=128, block_rows=16):
    """One GPT-OSS-120B-shaped MoE layer, 16-row blocks.

    Attention is represented by four ``attn_rows x width`` projections, a
    ``router_rows x width`` router and two norms of ``width`` (a stand-in: the
    pages give only the width; experts are ~99% of the bucket).
    """
    br = block_rows
    ts = [_rows(n, attn_rows, width, br) for n in ("q", "k", "v", "o")]
    ts.append(_rows("router", router_rows, width, br))
    for e in range(experts):
        ts.append(_rows(f"e{e}.gate_up", expert_rows[0], width, br))
        ts.append(_rows(f"e{e}.down", expert_rows[1], width, br))
    ts.append(_vec("attn_norm", width, br))
    ts.append(_vec("mlp_norm", width, br))
    return ts


def deepseek_bucket(experts=256, hidden=7168, inter=2048, tile=128):
    """One DeepSeek-V3-shaped MoE layer with 128x128 2-D quantisation tiles.

    The shard unit is a row panel of ``tile`` rows; the quantisation block is
    a ``tile x tile`` tile inside it.
    """
    ts = []
    for e in range(experts):
        ts.append(TensorDef(f"e{e}.gate", inter, hidden, tile, tile))
        ts.append(TensorDef(f"e{e}.up", inter, hidden, tile, tile))
        ts.append(TensorDef(f"e{e}.down", hidden, inter, tile, tile))
    return ts


def adversarial_bucket(n=10000, max_numel=1_000_000, seed=0):
    """``n`` 1-D tensors, element counts log-uniform on [1, max_numel], row
    blocks drawn uniformly from {1, 16, 128}."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0xA5A5]))
    u = rng.random(n)
    sizes = np.maximum(1, np.rint(np.exp(u * math.log(max_numel)))).astype(np.int64)
    blocks = rng.choice(np.array([1, 16, 128]), size=n)
    return [_vec(f"a{i}", int(s), int(b)) for i, (s, b) in enumerate(zip(sizes, blocks))]


CONFIGS = {
    # full-size workloads
    "llama": Config("llama", llama_bucket(), fsdp=128, n_buckets=80,
                    description="LLaMA-3-70B-shaped dense buckets: 80 layers, 1-row blocks, FSDP 128"),
    "gptoss": Config("gptoss", gptoss_bucket(), fsdp=256, n_buckets=36,
                     description="GPT-OSS-120B-shaped MoE buckets: 36 layers, 128 experts, 16-row blocks, FSDP 256"),
    "deepseek": Config("deepseek", deepseek_bucket(), fsdp=64, n_buckets=1, grad_dist="student_t3",
                       description="DeepSeek-V3-shaped MoE layer: 256 experts, 128x128 tiles, FSDP 64"),
    "adversarial": Config("adversarial", adversarial_bucket(), fsdp=1024, n_buckets=1,
                          description="10,000 1-D tensors, log-uniform sizes on [1,1e6], {1,16,128}-row blocks, FSDP 1024"),
    # scaled-down twins that keep the block geometry (parity at oracle-friendly sizes)
    "llama_mini": Config("llama_mini", llama_bucket(hidden=1024, inter=3584, kv=128), fsdp=16,
                         n_buckets=2, description="LLaMA-shaped layer scaled by 1/8, FSDP 16"),
    "llama_rowblk": Config("llama_rowblk", llama_bucket(hidden=512, inter=28672, kv=64), fsdp=64,
                           n_buckets=1, description="narrow LLaMA-shaped layer whose down rows are 28,672 wide"),
    "gptoss_mini": Config("gptoss_mini", gptoss_bucket(experts=8, expert_rows=(720, 360), attn_rows=360),
                          fsdp=8, n_buckets=2, description="GPT-OSS-shaped layer, 8 experts, rows / 8, FSDP 8"),
    "deepseek_mini": Config("deepseek_mini", deepseek_bucket(experts=4, hidden=1792, inter=512), fsdp=8,
                            grad_dist="student_t3", description="DeepSeek-shaped layer, 4 experts, 128x128 tiles, FSDP 8"),
    "adversarial_mini": Config("adversarial_mini", adversarial_bucket(n=400, max_numel=100_000, seed=1),
                               fsdp=64, description="400 ragged 1-D tensors, FSDP 64"),
}
CONFIGS.update({c.name: c for c in toy_variants().values()})


def get_config(name: str) -> Config:
    return CONFIGS[name]
