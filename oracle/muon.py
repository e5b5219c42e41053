"""Plain reference of Muon's Newton-Schulz orthogonalisation of one gathered
2-D matrix.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may use this module; it shares nothing with the
GPU library.

The pages run Muon's Newton-Schulz iteration on the root rank after
gathering the full 2-D matrix there (talk notes, "Case study: 8-bit Adam and
distributed Muon": the whole parameter matrix is redistributed to one rank,
iterated, and redistributed back; Dutch summary, "Muon-optimalisator").  They
give no formula.  The reading taken is the published Muon iteration (Jordan
et al., 2024): normalise by the Frobenius norm, work on the wide orientation
(transpose a tall matrix), then apply five times the quintic

    A = X X^T,   B = b A + c A A,   X <- a X + B X,
    (a, b, c) = (3.4445, -4.7750, 2.0315),

which maps every singular value s of X to p(s) = a s + b s^3 + c s^5 and
leaves the singular vectors alone.

Precision (the method's, as Muon runs it): the operands X, A, B are stored as
bf16 between the products; products accumulate in (at least) fp32; each
stored result is the fp32 value rounded to nearest even.  Here every product
is evaluated in fp64 and each stored value is rounded fp64 -> fp32 -> bf16,
the two roundings the GPU applies.  With ``rounding=False`` nothing is
rounded (the exact iteration, used to pin this module against the SVD form).
"""

from __future__ import annotations

import numpy as np

NS_COEFFS = (3.4445, -4.7750, 2.0315)
NS_STEPS = 5
NS_EPS = 1e-7


def _bf16_round(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 (nearest even) -> bf16 (nearest even), back as fp64."""
    f = np.ascontiguousarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << 16
    r[nan] = 0x7FC00000
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    r = _bf16_round(x).astype(np.float32).view(np.uint32)
    return (r >> 16).astype(np.uint16)


def newton_schulz(G, steps: int = NS_STEPS, eps: float = NS_EPS, coeffs=NS_COEFFS, rounding: bool = True,
                  trace: list | None = None) -> np.ndarray:
    """Newton-Schulz orthogonalisation of a rows x cols matrix ``G`` (values,
    any float dtype).  Returns fp64 values (bf16-representable when
    ``rounding``).  ``trace``, if a list, receives (X0, [(A, B, X), ...]) in
    the wide orientation."""
    a, b, c = (float(v) for v in coeffs)
    rnd = _bf16_round if rounding else (lambda v: v)
    G = np.asarray(G, dtype=np.float64)
    if G.ndim != 2:
        raise ValueError("G must be 2-D")
    tall = G.shape[0] > G.shape[1]
    norm = float(np.sqrt(np.sum(G * G)))
    X = rnd(G / (norm + eps))
    if tall:
        X = X.T.copy()
    stages = []
    for _ in range(steps):
        A = rnd(X @ X.T)
        B = rnd(b * A + c * (A @ A))
        X = rnd(a * X + B @ X)
        stages.append((A, B, X))
    if trace is not None:
        trace.append(stages)
    return X.T.copy() if tall else X


def scalar_quintic(s, steps: int = NS_STEPS, coeffs=NS_COEFFS):
    """The map the iteration applies to each singular value: p applied
    ``steps`` times, p(s) = a s + b s^3 + c s^5."""
    a, b, c = coeffs
    s = np.asarray(s, dtype=np.float64)
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def flops(rows: int, cols: int, steps: int = NS_STEPS) -> int:
    """Multiply-add work of the iteration counted the minimal way, as two
    flops per multiply-add: X X^T and A A are symmetric (half their entries
    are needed), B X is a full product.  m = min(rows, cols), n = max:
    per step m*m*n + m*m*m + 2*m*m*n."""
    m, n = min(rows, cols), max(rows, cols)
    return steps * (3 * m * m * n + m * m * m)


def gemm_nt(P, Q, D=None, alpha: float = 1.0, beta: float = 0.0, rounding: bool = True) -> np.ndarray:
    """C = alpha * P Q^T + beta * D, evaluated in fp64 and rounded like a
    stored result (fp64 -> fp32 -> bf16).  ``alpha`` and ``beta`` are taken
    as the fp32 numbers the product kernel receives."""
    a, b = float(np.float32(alpha)), float(np.float32(beta))
    C = a * (np.asarray(P, np.float64) @ np.asarray(Q, np.float64).T)
    if D is not None:
        C = C + b * np.asarray(D, np.float64)
    return _bf16_round(C) if rounding else C
