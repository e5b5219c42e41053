"""Pins for the Newton-Schulz oracle (oracle/muon.py), against what the
mathematics fixes: the SVD form of the iteration (numpy's SVD), equivariance
under orthogonal transforms, the scalar recursion on diagonal inputs (with the
bf16 roundings), the published polynomial, and the flop count."""

from __future__ import annotations

import numpy as np
import pytest

from oracle import muon


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _orthogonal(n, seed):
    q, r = np.linalg.qr(_rand((n, n), seed))
    return q * np.sign(np.diag(r))


@pytest.mark.parametrize("shape", [(24, 40), (40, 24), (32, 32), (1, 17), (17, 1)])
def test_exact_iteration_is_the_quintic_on_singular_values(shape):
    # in exact arithmetic X_k = U p^k(S / (|G|_F + eps)) V^T for G = U S V^T
    G = _rand(shape, 1)
    U, S, Vt = np.linalg.svd(G, full_matrices=False)
    s0 = S / (np.sqrt((G * G).sum()) + muon.NS_EPS)
    want = (U * muon.scalar_quintic(s0)) @ Vt
    got = muon.newton_schulz(G, rounding=False)
    assert got.shape == G.shape
    assert np.abs(got - want).max() <= 1e-12 * max(1.0, np.abs(want).max())


def test_scalar_quintic_published_coefficients():
    # p(s) = 3.4445 s - 4.7750 s^3 + 2.0315 s^5: p(1) = 0.701, p'(0) = 3.4445
    p = lambda s: muon.scalar_quintic(s, steps=1)
    assert p(1.0) == pytest.approx(0.701, abs=1e-12)
    assert p(1e-6) / 1e-6 == pytest.approx(3.4445, rel=1e-9)
    assert p(-0.5) == pytest.approx(-p(0.5))              # odd polynomial


def test_orthogonal_equivariance():
    G = _rand((12, 20), 2)
    Q, R = _orthogonal(12, 3), _orthogonal(20, 4)
    lhs = muon.newton_schulz(Q @ G @ R.T, rounding=False)
    rhs = Q @ muon.newton_schulz(G, rounding=False) @ R.T
    assert np.abs(lhs - rhs).max() <= 1e-12


def test_diagonal_input_follows_the_scalar_recursion_with_roundings():
    # all matrices stay diagonal, so each stored value is the scalar recursion
    # with the same bf16 rounding points (fp64 -> fp32 -> bf16)
    d = np.array([3.0, 1.0, 0.5, 0.25, 2.0 ** -6, 7.0])
    G = np.diag(d)
    got = np.diag(muon.newton_schulz(G))
    a, b, c = muon.NS_COEFFS

    def rnd(v):
        return float(muon._bf16_round(np.array([v]))[0])

    norm = float(np.sqrt((d * d).sum()))
    for i, v in enumerate(d):
        x = rnd(v / (norm + muon.NS_EPS))
        for _ in range(muon.NS_STEPS):
            A = rnd(x * x)
            B = rnd(b * A + c * A * A)
            x = rnd(a * x + B * x)
        assert got[i] == x, (i, got[i], x)
    off = muon.newton_schulz(G) - np.diag(got)
    assert not off.any()


def test_bf16_round_ties_to_even_and_double_rounding_path():
    r = muon._bf16_round
    # 1 + 2^-8 is a bf16 tie -> 1; 1 + 3*2^-8 -> 1 + 2^-6
    assert r(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert r(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    # fp64 just above the tie rounds to the tie in fp32 first, then to even
    assert r(np.array([1 + 2.0 ** -8 + 2.0 ** -40]))[0] == 1.0
    bits = muon.f64_to_bf16_bits(np.array([1.0, -2.0, 0.0]))
    assert bits.tolist() == [0x3F80, 0xC000, 0x0000]
    assert muon.bf16_bits_to_f64(bits).tolist() == [1.0, -2.0, 0.0]


def test_rounded_iteration_stays_near_the_exact_one():
    # the bf16 iteration follows the exact one to within a few bf16 ulps of the
    # largest entry (a sanity bound, not a parity gate)
    G = _rand((48, 80), 5)
    ex = muon.newton_schulz(G, rounding=False)
    rd = muon.newton_schulz(G)
    assert np.abs(rd - ex).max() <= 0.05 * np.abs(ex).max()


def test_flop_count():
    # 2 x 3 (m=2, n=3), one step: X X^T half = m*m*n = 12, A A half = m^3 = 8,
    # B X = 2*m*m*n = 24 -> 44
    assert muon.flops(2, 3, steps=1) == 44
    assert muon.flops(3, 2, steps=1) == 44
    assert muon.flops(8192, 28672) == 5 * (3 * 8192 ** 2 * 28672 + 8192 ** 3)


# ---------------------------------------------------------------------------
# Pins of the product oracle gemm_nt (C = bf16(alpha P Q^T + beta D)): values
# the arithmetic fixes without reusing numpy's matmul as the reference.

def _int_mat(shape, seed, lo=-4, hi=4):
    return np.random.default_rng(seed).integers(lo, hi + 1, size=shape).astype(np.float64)


def _loops_nt(P, Q):
    """Plain triple loop over Python integers: C[i][j] = sum_k P[i][k] Q[j][k]."""
    M, K = P.shape
    N = Q.shape[0]
    return [[sum(int(P[i, k]) * int(Q[j, k]) for k in range(K)) for j in range(N)] for i in range(M)]


def test_gemm_nt_small_integers_exact():
    # entries in [-4, 4] and K = 16 keep every sum within +-256: exact in
    # fp32 and in bf16, so C must equal the integer product; M, N, K distinct
    # so a transposed operand cannot line up
    P, Q = _int_mat((5, 16), 11), _int_mat((7, 16), 12)
    want = np.array(_loops_nt(P, Q), dtype=np.float64)
    got = muon.gemm_nt(P, Q)
    assert got.shape == (5, 7)
    assert np.array_equal(got, want)


def test_gemm_nt_identity_and_permutation():
    X = muon.bf16_bits_to_f64(muon.f64_to_bf16_bits(_rand((6, 9), 13)))
    assert np.array_equal(muon.gemm_nt(X, np.eye(9)), X)          # X I^T = X
    perm = np.array([3, 0, 8, 1, 7, 2, 6, 4, 5])
    Pm = np.zeros((9, 9))
    Pm[np.arange(9), perm] = 1.0                                    # row j picks column perm[j]
    got = muon.gemm_nt(X, Pm)
    assert np.array_equal(got, X[:, perm])                          # C[i, j] = X[i, perm[j]]
    assert np.array_equal(muon.gemm_nt(np.eye(6), X.T.copy()), X)  # I (X^T)^T = X


def test_gemm_nt_alpha_beta_powers_of_two():
    P, Q = _int_mat((4, 4), 21, -2, 2), _int_mat((3, 4), 22, -2, 2)
    D = _int_mat((4, 3), 23, -4, 4)
    base = np.array(_loops_nt(P, Q), dtype=np.float64)   # integers in [-16, 16]
    for alpha, beta in ((0.125, 4.0), (-2.0, 0.5), (1.0, 0.0), (0.0, -1.0)):
        want = alpha * base + beta * D
        # every result is a multiple of 1/8 below 32 in magnitude: at most 8
        # significant bits, so bf16 holds it exactly and no rounding happens
        assert np.all(want * 8 == np.round(want * 8)) and np.abs(want).max() < 32
        assert np.array_equal(muon.gemm_nt(P, Q, D, alpha=alpha, beta=beta), want), (alpha, beta)
    # without D, beta plays no part
    assert np.array_equal(muon.gemm_nt(P, Q, None, alpha=2.0, beta=3.0), 2.0 * base)


def test_gemm_nt_double_rounding_decides():
    # exact 1 + 2^-8 + 2^-30: fp64 -> fp32 gives the bf16 tie 1 + 2^-8 (the
    # 2^-30 is below half an fp32 ulp), which rounds to even: 1.0.  A single
    # rounding straight to bf16 would give 1 + 2^-7.
    P = np.array([[1.0, 2.0 ** -8, 2.0 ** -30]])
    Q = np.ones((1, 3))
    assert muon.gemm_nt(P, Q)[0, 0] == 1.0
    # 1 + 2^-8 + 2^-20 survives fp32 above the tie and rounds up
    P2 = np.array([[1.0, 2.0 ** -8, 2.0 ** -20]])
    assert muon.gemm_nt(P2, Q)[0, 0] == 1.0 + 2.0 ** -7
    # the same through beta * D: D = 2^-30, beta 1
    C = muon.gemm_nt(np.array([[1.0, 2.0 ** -8]]), np.ones((1, 2)), D=np.array([[2.0 ** -30]]), beta=1.0)
    assert C[0, 0] == 1.0


def test_gemm_nt_alpha_is_taken_in_fp32():
    # alpha = 0.1 reaches the kernel as the fp32 number nearest 0.1
    P = np.array([[1.0]])
    a32 = float(np.float32(0.1))
    want = muon._bf16_round(np.array([a32]))[0]
    assert muon.gemm_nt(P, P, alpha=0.1)[0, 0] == want
