"""Pins for the oracle's DBuffer group operations (zero, scale, accumulate).

The element arithmetic is checked against exact rational arithmetic written
out here (``fractions.Fraction``): the exact result is rounded once to fp32
and once to bf16, both to nearest-even, which is the reading the oracle
follows (one IEEE fp32 operation on widened bf16 operands, then a bf16
store).  Two hand-built cases fix the reading itself: one where rounding the
exact value straight to bf16 would differ, and one where an unfused
multiply-then-add would differ.  The layout side (padding, rank chunks) is
checked against copy-in and against slicing of the whole-bucket result.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import oracle
from synth.data import bf16_bits_to_f32, f32_to_bf16_bits, host_grads

from helpers import layout_of

ZERO, SCALE, ACC = oracle.GROUP_ZERO, oracle.GROUP_SCALE, oracle.GROUP_ACCUMULATE


# ---------------------------------------------------------------------------
# exact rounding of a rational to a binary format
def _round_binary(q: Fraction, p: int, min_quantum_exp: int, max_finite: Fraction):
    """Nearest value with ``p`` significant bits and quantum >= 2^min_quantum_exp,
    ties to even; returns +-inf (as a float) past the overflow threshold."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()   # 2^e <= a < 2^(e+2)
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    qexp = max(e - (p - 1), min_quantum_exp)
    quantum = Fraction(2) ** qexp
    r = round(a / quantum) * quantum      # round() on a Fraction: ties to even
    if r > max_finite:
        return sign * float("inf")
    return sign * r


def _fp32(q):
    return _round_binary(q, 24, -149, Fraction(2 ** 24 - 1, 2 ** 23) * 2 ** 127)


def _bf16(q):
    return _round_binary(q, 8, -133, Fraction(2 ** 8 - 1, 2 ** 7) * 2 ** 127)


def _bits_of(q, negative_zero=False) -> int:
    """bf16 bit pattern of an exactly representable value (Fraction or +-inf);
    an exact zero takes the sign IEEE 754 gives it."""
    if q == 0:
        return 0x8000 if negative_zero else 0
    f = np.float32(float(q))
    return int(f.view(np.uint32)) >> 16


def _value_sign(bits: int):
    f = float(bf16_bits_to_f32(np.array([bits], np.uint16))[0])
    return Fraction(f), (bits & 0x8000) != 0


def _round_twice(exact: Fraction):
    y = _fp32(exact)
    return _bf16(y) if not isinstance(y, float) else y


def _exact_scale(alpha: np.float32, x_bits: int) -> int:
    x, xneg = _value_sign(x_bits)
    a = Fraction(float(alpha))
    r = _round_twice(a * x)
    # a zero result (exact or underflowed) carries the sign of the product
    return _bits_of(r, negative_zero=(alpha < 0) != xneg)


def _exact_acc(alpha: np.float32, x_bits: int, g_bits: int) -> int:
    x, xneg = _value_sign(x_bits)
    g, gneg = _value_sign(g_bits)
    a = Fraction(float(alpha))
    exact = x + a * g
    r = _round_twice(exact)
    if exact != 0:
        return _bits_of(r, negative_zero=exact < 0)     # underflow keeps the sign
    pneg = (alpha < 0) != gneg                            # sign of the product term
    both_neg = xneg and pneg and x == 0 and a * g == 0
    return _bits_of(r, negative_zero=both_neg)            # exact cancellation: +0


def _one_tensor(n):
    """A one-tensor bucket of n elements on one rank (S = n)."""
    return [(n, 1, 1, 1, 0)], 1, n


def _canon_zero(b):
    b = np.asarray(b, np.uint16).copy()
    b[b == 0x8000] = 0
    return b


def _random_bf16(rng, n):
    """bf16 values spread over many binades, both signs, a few exact zeros."""
    x = rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n).astype(np.float64))
    x[rng.random(n) < 0.02] = 0.0
    return f32_to_bf16_bits(x.astype(np.float32))


# ---------------------------------------------------------------------------
# element arithmetic against exact rationals
@pytest.mark.parametrize("alpha", [1.0 / 3.0, 0.125, -0.7, 1.0 + 2.0 ** -23, 3.0e-5, -1.0])
def test_group_scale_matches_exact_rounding(alpha):
    rng = np.random.default_rng(11)
    x = _random_bf16(rng, 400)
    a32 = np.float32(alpha)
    spec, m, S = _one_tensor(len(x))
    got = oracle.group_op(spec, m, S, 0, SCALE, float(a32), x.copy())
    want = np.array([_exact_scale(a32, int(v)) for v in x], np.uint16)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("alpha", [1.0, 0.5, 1.0 / 3.0, -0.7, 1.0 + 2.0 ** -23, 1.0e-3])
def test_group_accumulate_matches_exact_rounding(alpha):
    rng = np.random.default_rng(12)
    x = _random_bf16(rng, 400)
    g = _random_bf16(rng, 400)
    a32 = np.float32(alpha)
    spec, m, S = _one_tensor(len(x))
    got = oracle.group_op(spec, m, S, 0, ACC, float(a32), x.copy(), grads=[g])
    want = np.array([_exact_acc(a32, int(a), int(b)) for a, b in zip(x, g)], np.uint16)
    assert np.array_equal(got, want)


def test_group_accumulate_rounds_through_fp32_first():
    # x = 1, alpha*g = 2^-8 + 2^-30: the exact sum lies just above the bf16
    # midpoint 1 + 2^-8, but its fp32 image is the midpoint itself (2^-30 is
    # under half an fp32 ulp at 1), which then rounds to the even bf16 value 1.
    alpha = np.float32(1.0 + 2.0 ** -22)
    g = f32_to_bf16_bits(np.array([2.0 ** -8], np.float32))
    x = f32_to_bf16_bits(np.array([1.0], np.float32))
    got = oracle.group_op(*_one_tensor(1), 0, ACC, float(alpha), x.copy(), grads=[g])
    assert got[0] == 0x3F80                 # single rounding to bf16 would give 0x3F81
    assert _exact_acc(alpha, int(x[0]), int(g[0])) == 0x3F80


def test_group_accumulate_is_fused():
    # x = 1, g = 1 + 2^-7, alpha = 1 + 2^-23: alpha*g = 1 + 2^-7 + 2^-23 + 2^-30.
    # Fused: fp32(2 + 2^-7 + 2^-23 + 2^-30) = 2 + 2^-7 + 2^-22 -> bf16 2 + 2^-6.
    # Unfused, the product first rounds to 1 + 2^-7 + 2^-23, the sum is an fp32
    # tie that goes to 2 + 2^-7, and that bf16 tie goes to 2.
    alpha = np.float32(1.0 + 2.0 ** -23)
    g = np.array([0x3F81], np.uint16)
    x = np.array([0x3F80], np.uint16)
    got = oracle.group_op(*_one_tensor(1), 0, ACC, float(alpha), x.copy(), grads=[g])
    assert got[0] == 0x4001
    unfused = np.float32(np.float32(1.0) + np.float32(alpha * np.float32(1.0078125)))
    assert f32_to_bf16_bits(np.array([unfused], np.float32))[0] == 0x4000


def test_group_special_values():
    spec, m, S = _one_tensor(6)
    big = f32_to_bf16_bits(np.array([3.0e38, -3.0e38, 1.0, 2.0 ** -133, -(2.0 ** -133), 0.0], np.float32))
    got = oracle.group_op(spec, m, S, 0, SCALE, 2.0, big.copy())
    # overflow to +-inf, exact doubling, the smallest subnormal doubles exactly
    want = f32_to_bf16_bits(np.array([np.inf, -np.inf, 2.0, 2.0 ** -132, -(2.0 ** -132), 0.0], np.float32))
    assert np.array_equal(got, want)
    got = oracle.group_op(spec, m, S, 0, SCALE, 0.5, big.copy())
    # halving the smallest bf16 subnormal is a tie between 0 and it: even is 0
    assert got[3] == 0x0000 and got[4] == 0x8000 and got[2] == 0x3F00


# ---------------------------------------------------------------------------
# closed forms and invariants over real layouts
@pytest.mark.parametrize("name", ["toy_mix", "toy_r4", "toy_tile", "adversarial_mini", "deepseek_mini"])
def test_group_ops_layout(name):
    cfg, lay = layout_of(name)
    m, S = lay.fsdp, lay.shard
    spec = lay.spec_array()
    rng = np.random.default_rng(5)
    grads = host_grads(cfg, lay, 0)
    for rank in [-1] + list(range(m)):
        n = m * S if rank < 0 else S
        junk = rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16)
        junk[(junk & 0x7F80) == 0x7F80] = 0x3F80          # no inf/NaN in the start state
        valid = (np.concatenate([lay.valid_mask(r) for r in range(m)]) if rank < 0
                 else lay.valid_mask(rank))
        # zero: everything, padding included
        z = oracle.group_op(spec, m, S, rank, ZERO, 0.0, junk.copy())
        assert not z.any()
        # scale by 1: tensor elements unchanged, padding cleared
        s1 = oracle.group_op(spec, m, S, rank, SCALE, 1.0, junk.copy())
        assert np.array_equal(s1[valid], junk[valid]) and not s1[~valid].any()
        # scale by 2^-3: exact for normal values (scaled values stay normal here)
        xs = f32_to_bf16_bits((rng.standard_normal(n) * 4.0).astype(np.float32))
        s8 = oracle.group_op(spec, m, S, rank, SCALE, 0.125, xs.copy())
        want = f32_to_bf16_bits(bf16_bits_to_f32(xs) * np.float32(0.125))
        assert np.array_equal(s8[valid], want[valid])
        # accumulate into zeros with alpha 1 is the group copy-in (up to the
        # sign of zero: +0 + -0 = +0)
        a1 = oracle.group_op(spec, m, S, rank, ACC, 1.0, np.zeros(n, np.uint16), grads=grads)
        assert np.array_equal(_canon_zero(a1), _canon_zero(oracle.copy_in(spec, m, S, rank, grads)))
        # accumulate -1 * g into a copy of g cancels to +0 everywhere
        c = oracle.copy_in(spec, m, S, rank, grads)
        cancel = oracle.group_op(spec, m, S, rank, ACC, -1.0, c.copy(), grads=grads)
        assert not cancel.any()


@pytest.mark.parametrize("name", ["toy_mix", "toy_r16", "adversarial_mini"])
@pytest.mark.parametrize("op,alpha", [(SCALE, 0.3), (ACC, -0.55)])
def test_group_whole_bucket_is_the_rank_chunks(name, op, alpha):
    cfg, lay = layout_of(name)
    m, S = lay.fsdp, lay.shard
    spec = lay.spec_array()
    grads = host_grads(cfg, lay, 1)
    base = f32_to_bf16_bits(np.random.default_rng(3).standard_normal(m * S).astype(np.float32))
    whole = oracle.group_op(spec, m, S, -1, op, alpha, base.copy(), grads=grads)
    for r in range(m):
        part = oracle.group_op(spec, m, S, r, op, alpha, base[r * S:(r + 1) * S].copy(), grads=grads)
        assert np.array_equal(part, whole[r * S:(r + 1) * S]), r


def test_group_accumulate_with_grad_bases():
    # a rank may hold only its own rows of a gradient: grads[k] starts at
    # element bases[k]; the result must not depend on where the storage starts
    cfg, lay = layout_of("toy_r4")
    m, S = lay.fsdp, lay.shard
    spec = lay.spec_array()
    grads = host_grads(cfg, lay, 2)
    x = f32_to_bf16_bits(np.random.default_rng(4).standard_normal(S).astype(np.float32))
    for r in range(m):
        full = oracle.group_op(spec, m, S, r, ACC, 0.75, x.copy(), grads=grads)
        lo = {k: a for k, a, _b, _d in lay.chunk_intervals(r)}
        part = [None if k not in lo else g[lo[k]:] for k, g in enumerate(grads)]
        bases = [lo.get(k, 0) for k in range(len(grads))]
        got = oracle.group_op(spec, m, S, r, ACC, 0.75, x.copy(), grads=part, bases=bases)
        assert np.array_equal(got, full)


def test_group_op_rejects_bad_arguments():
    spec, m, S = _one_tensor(4)
    b = np.zeros(4, np.uint16)
    with pytest.raises(oracle.OracleError):
        oracle.group_op(spec, m, S, 0, 3, 1.0, b)
    with pytest.raises(oracle.OracleError):
        oracle.group_op(spec, m, S, 1, SCALE, 1.0, b)
