"""The Newton-Schulz entry point that allocates nothing (its workspace is the
library's static device scratch) against the entry point with a caller
workspace: bit for bit, on two calls in a row, the second on a smaller
matrix (the scratch keeps the first call's contents)."""

from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _bf16_matrix(shape, seed):
    import torch
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randn(*shape, generator=g, device=DEV).to(torch.bfloat16).view(torch.int16)


def test_no_alloc_equals_workspace_entry_point_on_two_calls():
    import torch
    import ragged_shard_optimizer_amd as ve
    # first a routed-expert matrix (split products, the largest shape the
    # scratch holds), then a smaller, tall one
    for shape, steps, seed in (((2048, 7168), 5, 31), ((300, 128), 3, 32)):
        print(f"[gpu] no-alloc newton-schulz {shape} steps={steps}", flush=True)
        G = _bf16_matrix(shape, seed)
        got = torch.full(shape, -1, dtype=torch.int16, device=DEV)
        want = torch.full(shape, -1, dtype=torch.int16, device=DEV)
        ve.muon_newton_schulz_noalloc(G, got, steps=steps)
        ws = torch.empty(ve.muon_workspace_bytes(*shape), dtype=torch.uint8, device=DEV)
        ve.muon_newton_schulz(G, want, steps=steps, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(got, want), shape
        assert bool(torch.isfinite(got.view(torch.bfloat16).float()).all()), shape


def test_no_alloc_rejects_a_matrix_beyond_its_scratch():
    import torch
    import ragged_shard_optimizer_amd as ve
    shape = (4096, 8192)
    G = torch.zeros(shape, dtype=torch.int16, device=DEV)
    out = torch.zeros_like(G)
    with pytest.raises(ve.VeError, match="static scratch holds"):
        ve.muon_newton_schulz_noalloc(G, out)
    torch.cuda.synchronize()
    assert not bool(out.any())
