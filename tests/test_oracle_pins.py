"""Pins for the CPU oracle: each checks it against something other than
itself -- hand-derived values, closed forms, a library optimizer, invariants,
and the unsharded brute force.  No GPU involved."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import bruteforce
from synth import CONFIGS, HPARAMS, TensorDef, plan_p0
from synth.configs import Config
from synth.data import bf16_bits_to_f32, f32_to_bf16_bits, host_grads, host_master
from synth.layout import Layout

from helpers import hp32, layout_of, rank_block_coords, ulp_diff_f32

SMALL = ["toy_mix", "toy_r1", "toy_r4", "toy_r16", "toy_tile", "deepseek_mini", "adversarial_mini",
         "gptoss_mini", "llama_mini"]


# ---------------------------------------------------------------------------
# quantiser: hand-derived codes (round half to even, clamp, zero block)
def test_quantize_hand_values_ties_to_even():
    # amax 127 -> scale 1, reciprocal 1: codes are rint(x) with ties to even
    x = np.array([127, 62.5, 63.5, -0.5, 1.5, -127, 0.49999997, 2.5, -2.5], np.float32)
    q, s = oracle.quantize(x)
    assert s == np.float32(1.0)
    assert q.tolist() == [127, 62, 64, 0, 2, -127, 0, 2, -2]


def test_quantize_hand_values_scaled():
    # amax 2: scale fp32(2/127), reciprocal exactly 63.5
    q, s = oracle.quantize(np.array([2.0, 1.0, -0.5, 0.0], np.float32))
    assert s == np.float32(2.0 / 127.0)
    assert q.tolist() == [127, 64, -32, 0]   # 63.5 -> 64, -31.75 -> -32


def test_quantize_zero_block():
    q, s = oracle.quantize(np.zeros(37, np.float32))
    assert s == 0.0 and not q.any()


@pytest.mark.parametrize("n", [1, 2, 17, 1000])
def test_quantize_invariants(n):
    rng = np.random.default_rng(n)
    for trial in range(20):
        x = (rng.standard_normal(n) * 10.0 ** rng.integers(-12, 2)).astype(np.float32)
        if trial % 3 == 0:
            x = np.abs(x)                     # second-moment-like, non-negative
        q, s = oracle.quantize(x)
        am = np.abs(x).max()
        assert s == np.float32(np.float64(am) / 127.0)
        assert q.min() >= -127 and q.max() <= 127
        assert np.abs(q).max() == 127         # the absmax element maps to +-127
        if trial % 3 == 0:
            assert q.min() >= 0
        # dequantisation error bound: half a step (+ fp32 rounding slack)
        err = np.abs(q.astype(np.float64) * np.float64(s) - x.astype(np.float64))
        assert err.max() <= np.float64(s) * (0.5 + 1e-5)
        assert np.array_equal(np.sign(q[np.abs(x) > s]), np.sign(x[np.abs(x) > s]))


# ---------------------------------------------------------------------------
# layout validation
def _spec(rows):
    return np.array(rows, dtype=np.int64)


def test_validate_accepts_all_planned_layouts():
    for name in list(CONFIGS):
        cfg, lay = layout_of(name)
        oracle.validate(lay.spec_array(), lay.fsdp, lay.shard)


@pytest.mark.parametrize("spec,m,S,what", [
    ([[4, 8, 2, 8, 0], [4, 8, 2, 8, 30]], 2, 32, "overlap"),
    ([[4, 8, 2, 8, 0]], 2, 24, "unit boundary"),          # rank cut at row 3 of 2-row panels
    ([[4, 8, 2, 8, 0], [2, 8, 1, 8, 8]], 1, 40, "overlap"),
    ([[4, 8, 1, 8, 40]], 2, 32, "leaves the bucket"),
    ([[4, 8, 1, 3, 0]], 1, 32, "does not divide"),
    ([[0, 8, 1, 8, 0]], 1, 32, "non-positive"),
    ([[4, 8, 0, 8, 0]], 1, 32, "non-positive"),
    ([[4, 8, 1, 8, -1]], 1, 32, "leaves the bucket"),
])
def test_validate_rejects(spec, m, S, what):
    with pytest.raises(oracle.OracleError, match=what):
        oracle.validate(_spec(spec), m, S)


def test_validate_accepts_partial_panel_and_multi_rank_tensor():
    # 10 rows in 4-row panels (last panel 2 rows), spanning 3 ranks of S=16
    oracle.validate(_spec([[10, 4, 4, 4, 0]]), 3, 16)
    assert oracle.rank_blocks(_spec([[10, 4, 4, 4, 0]]), 16, 2) == (1, 8)
    # piece ending at numel mid-panel is fine; a cut mid-panel is not
    with pytest.raises(oracle.OracleError):
        oracle.validate(_spec([[10, 4, 4, 4, 8]]), 3, 16)


# ---------------------------------------------------------------------------
# pack / unpack: copy-in then zero-copy slice is the identity; padding is zero
@pytest.mark.parametrize("name", SMALL)
def test_copy_in_slice_identity(name):
    cfg, lay = layout_of(name)
    spec = lay.spec_array()
    grads = host_grads(cfg, lay, bucket=0)
    whole = oracle.copy_in(spec, lay.fsdp, lay.shard, -1, grads)
    seen = np.zeros(lay.bucket_elems, np.int32)
    for r in range(lay.fsdp):
        chunk = oracle.copy_in(spec, lay.fsdp, lay.shard, r, grads)
        assert np.array_equal(chunk, whole[r * lay.shard:(r + 1) * lay.shard])
        mask = np.zeros(lay.shard, bool)
        for k in range(len(lay.tensors)):
            sl = oracle.slice_(spec, lay.fsdp, lay.shard, r, k)
            if sl is None:
                continue
            off, lo, hi = sl
            assert np.array_equal(chunk[off:off + hi - lo], grads[k][lo:hi])
            assert not mask[off:off + hi - lo].any()
            mask[off:off + hi - lo] = True
            seen[r * lay.shard + off: r * lay.shard + off + hi - lo] += 1
        assert not chunk[~mask].any()                  # padding is zero
    for k, t in enumerate(lay.tensors):                # every element exactly once
        off, lo, hi = oracle.slice_(spec, lay.fsdp, lay.shard, -1, k)
        assert (lo, hi) == (0, t.numel)
        assert np.all(seen[off:off + t.numel] == 1)
        assert np.array_equal(whole[off:off + t.numel], grads[k])
    assert seen.sum() == lay.valid_elems


# ---------------------------------------------------------------------------
# sharded oracle over all ranks == unsharded brute force, bit for bit
def _ragged_small():
    rng = np.random.default_rng(7)
    ts = []
    for i in range(24):
        n = int(max(1, round(math.exp(rng.random() * math.log(3000)))))
        ts.append(TensorDef(f"a{i}", n, 1, int(rng.choice([1, 16, 128])), 1))
    ts.append(TensorDef("tile2d", 40, 48, 8, 16))
    return Config("ragged_small", ts, fsdp=7, grad_scale=1e-3)


@pytest.mark.parametrize("name", ["toy_mix", "toy_r1", "toy_r4", "toy_r16", "toy_tile",
                                  "deepseek_mini", "ragged_small"])
def test_sharded_equals_unsharded_bruteforce(name):
    cfg = _ragged_small() if name == "ragged_small" else CONFIGS[name]
    lay = plan_p0(cfg.tensors, cfg.fsdp)
    spec, m, S = lay.spec_array(), lay.fsdp, lay.shard
    hp = hp32()
    # unsharded tensors: master from the rank shards' initial values
    states = [oracle.new_state(spec, S, r, host_master(cfg, lay, 0, r)) for r in range(m)]
    full = {}
    for k, t in enumerate(lay.tensors):
        w = np.zeros(t.numel, np.float32)
        for r in range(m):
            sl = oracle.slice_(spec, m, S, r, k)
            if sl:
                off, lo, hi = sl
                w[lo:hi] = states[r]["master"][off:off + hi - lo]
        P = -(-t.rows // t.block_rows)
        J = t.cols // t.block_cols
        full[k] = dict(master=w.reshape(t.rows, t.cols), m_q=np.zeros((t.rows, t.cols), np.int8),
                       v_q=np.zeros((t.rows, t.cols), np.int8), m_scale=np.zeros((P, J), np.float32),
                       v_scale=np.zeros((P, J), np.float32))
    coords = [rank_block_coords(lay, r) for r in range(m)]
    for step in range(1, cfg.steps + 1):
        grads = host_grads(cfg, lay, bucket=0, step=step)
        for r in range(m):
            oracle.shard_step(spec, m, S, r, grads, states[r], hp, step)
        for k, t in enumerate(lay.tensors):
            f = full[k]
            out = bruteforce.step_tensor(grads[k].reshape(t.rows, t.cols), f["master"], f["m_q"], f["v_q"],
                                         f["m_scale"], f["v_scale"], t.block_rows, t.block_cols, hp, step)
            f["master"], f["m_q"], f["v_q"], f["m_scale"], f["v_scale"], f["param"] = out
        for r in range(m):
            st = states[r]
            for k in range(len(lay.tensors)):
                sl = oracle.slice_(spec, m, S, r, k)
                if not sl:
                    continue
                off, lo, hi = sl
                f, n = full[k], hi - lo
                assert np.array_equal(st["master"][off:off + n].view(np.uint32),
                                      f["master"].reshape(-1)[lo:hi].view(np.uint32)), (step, r, k)
                assert np.array_equal(st["m_q"][off:off + n], f["m_q"].reshape(-1)[lo:hi])
                assert np.array_equal(st["v_q"][off:off + n], f["v_q"].reshape(-1)[lo:hi])
                assert np.array_equal(st["param_shard"][off:off + n], f["param"].reshape(-1)[lo:hi])
                assert np.array_equal(st["grad_shard"][off:off + n], grads[k][lo:hi])
            for b, (k, p, j) in enumerate(coords[r]):
                assert st["m_scale"][b] == full[k]["m_scale"][p, j], (step, r, b)
                assert st["v_scale"][b] == full[k]["v_scale"][p, j], (step, r, b)
            pad = ~lay.valid_mask(r)
            assert not st["param_shard"][pad].any() and not st["grad_shard"][pad].any()


# ---------------------------------------------------------------------------
# library pin: from a zero state, step 1 of 8-bit AdamW is exactly fp32-stored
# AdamW (the update uses the fresh moments), so it must agree with
# torch.optim.AdamW run in float64.
def _torch_adamw(p0: np.ndarray, grads_seq, hp):
    p = torch.tensor(p0.astype(np.float64), requires_grad=True)
    opt = torch.optim.AdamW([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"], foreach=False)
    outs = []
    for g in grads_seq:
        p.grad = torch.tensor(g.astype(np.float64))
        opt.step()
        outs.append(p.detach().numpy().copy())
    return outs


@pytest.mark.parametrize("name", ["toy_mix", "toy_tile", "deepseek_mini", "adversarial_mini"])
def test_step1_matches_torch_adamw(name):
    cfg, lay = layout_of(name)
    spec, m, S = lay.spec_array(), lay.fsdp, lay.shard
    hp = hp32()
    grads = host_grads(cfg, lay, bucket=0, step=1)
    for r in range(min(m, 4)):
        p0 = host_master(cfg, lay, 0, r)
        st = oracle.new_state(spec, S, r, p0)
        oracle.shard_step(spec, m, S, r, grads, st, hp, 1)
        g_shard = bf16_bits_to_f32(oracle.copy_in(spec, m, S, r, grads))
        (ref,) = _torch_adamw(p0, [g_shard], hp)
        valid = lay.valid_mask(r)
        assert ulp_diff_f32(st["master"][valid], ref[valid].astype(np.float32)).max() <= 1


# 1x1 blocks hold each moment as +-127 times a per-element scale, i.e. to fp32
# precision; several steps must then track float64 AdamW to ~1e-7.
def test_one_element_blocks_track_torch_adamw_over_steps():
    ts = [TensorDef("a", 200, 1, 1, 1), TensorDef("b", 37, 1, 1, 1), TensorDef("c", 16, 24, 1, 1)]
    cfg = Config("unit_blocks", ts, fsdp=3, grad_scale=1e-3)
    lay = plan_p0(ts, 3)
    spec, m, S = lay.spec_array(), lay.fsdp, lay.shard
    hp = hp32()
    for r in range(m):
        p0 = host_master(cfg, lay, 0, r)
        st = oracle.new_state(spec, S, r, p0)
        gseq = []
        for step in range(1, 6):
            grads = host_grads(cfg, lay, bucket=0, step=step)
            oracle.shard_step(spec, m, S, r, grads, st, hp, step)
            gseq.append(bf16_bits_to_f32(oracle.copy_in(spec, m, S, r, grads)))
        ref = _torch_adamw(p0, gseq, hp)[-1]
        valid = lay.valid_mask(r)
        rel = np.abs(st["master"][valid] - ref[valid]) / np.maximum(np.abs(ref[valid]), hp["lr"])
        assert rel.max() < 1e-6
        assert set(np.abs(st["m_q"][valid]).tolist()) <= {0, 127}


# ---------------------------------------------------------------------------
# closed forms
def test_constant_gradient_per_block_closed_form():
    # one block per 4-row panel; inside a block every gradient is the same c,
    # so m_hat = c and v_hat = c^2 exactly, and each step moves the weight by
    # lr * c / (|c| + eps) on top of the decoupled decay.
    t = TensorDef("w", 32, 64, 4, 64)
    lay = plan_p0([t], 1)
    spec, S = lay.spec_array(), lay.shard
    hp = hp32()
    cs = np.array([1e-3 * (k - 3.5) * (1 + k) for k in range(8)], np.float32)
    cb = f32_to_bf16_bits(cs)
    c = bf16_bits_to_f32(cb).astype(np.float64)
    g = np.repeat(cb, 4 * 64)
    p0 = (np.random.default_rng(3).standard_normal(S) * 0.02).astype(np.float32)
    st = oracle.new_state(spec, S, 0, p0)
    decay = 1.0 - hp["lr"] * hp["weight_decay"]
    for step in range(1, 8):
        oracle.shard_step(spec, 1, S, 0, [g], st, hp, step)
        geo = sum(decay ** k for k in range(step))
        ref = p0.astype(np.float64) * decay ** step - hp["lr"] * np.repeat(c / (np.abs(c) + hp["eps"]), 256) * geo
        rel = np.abs(st["master"] - ref) / np.maximum(np.abs(ref), hp["lr"])
        assert rel.max() < 1e-6, step
        assert np.all(np.abs(st["m_q"]) == 127) and np.all(st["v_q"] == 127)


def test_zero_gradient_closed_form():
    cfg, lay = layout_of("toy_mix")
    spec, m, S = lay.spec_array(), lay.fsdp, lay.shard
    hp = hp32()
    zero = [np.zeros(t.numel, np.uint16) for t in lay.tensors]
    decay = 1.0 - hp["lr"] * hp["weight_decay"]
    for r in range(m):
        p0 = host_master(cfg, lay, 0, r)
        st = oracle.new_state(spec, S, r, p0)
        for step in range(1, 6):
            oracle.shard_step(spec, m, S, r, zero, st, hp, step)
            ref = p0.astype(np.float64) * decay ** step
            assert np.all(np.abs(st["master"] - ref) <= 1e-6 * np.abs(ref) + 1e-30)
        assert not st["m_q"].any() and not st["v_q"].any()
        assert not st["m_scale"].any() and not st["v_scale"].any()


def test_block_selection_matches_full_step():
    cfg, lay = layout_of("toy_tile")
    spec, m, S = lay.spec_array(), lay.fsdp, lay.shard
    hp = hp32()
    grads = host_grads(cfg, lay, 0, 1)
    r = 1
    a = oracle.new_state(spec, S, r, host_master(cfg, lay, 0, r))
    b = {k: v.copy() for k, v in a.items()}
    oracle.shard_step(spec, m, S, r, grads, a, hp, 1)
    nb = len(a["m_scale"])
    sel = list(range(0, nb, 3))
    oracle.shard_step(spec, m, S, r, grads, b, hp, 1, blocks=sel)
    coords = rank_block_coords(lay, r)
    assert nb == len(coords)
    assert np.array_equal(a["m_scale"][sel], b["m_scale"][sel])
    assert not b["m_scale"][[i for i in range(nb) if i % 3]].any()
