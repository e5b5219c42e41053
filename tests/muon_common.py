"""Error bounds for comparing the MFMA product kernel and the Newton-Schulz
iteration with the oracle.

A stored result c = bf16(fp32(alpha * sum_k p_k q_k + beta * d)) computed on
the GPU differs from the oracle's bf16(fp32(exact)) by at most the fp32
evaluation error of the GPU before the rounding plus one bf16 ulp: the
accumulation of K products is within gamma_K * sum_k |p_k q_k| (products of
bf16 numbers are exact in fp32; gamma_K = K u / (1 - K u), with u = 2^-23 so
that a truncating accumulator is covered too), and the epilogue's scaling
and addition add two more roundings of relative size u.  When the operands
themselves carry errors dP, dQ, dD (from earlier stages), their first- and
second-order effects are added.  Everything is evaluated in fp64 with
absolute values, so the bound is rigorous and elementwise.
"""

from __future__ import annotations

import numpy as np

U = 2.0 ** -23


def gamma(k: int) -> float:
    return k * U / (1.0 - k * U)


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    """The bf16 spacing at |v| (at least the subnormal spacing 2^-133)."""
    a = np.maximum(np.abs(v), 2.0 ** -133)
    return np.exp2(np.maximum(np.floor(np.log2(a)) - 7, -133))


def product_bound(P, Q, D=None, alpha=1.0, beta=0.0, dP=None, dQ=None, dD=None, C=None):
    """Elementwise bound on |C_gpu - C_oracle| for C = bf16(alpha P Q^T + beta D)."""
    aP, aQ = np.abs(P), np.abs(Q)
    K = P.shape[1]
    a, b = abs(float(np.float32(alpha))), abs(float(np.float32(beta)))
    PQ = aP @ aQ.T
    err = a * gamma(K) * PQ
    if dP is not None:
        err = err + a * (dP @ aQ.T)
    if dQ is not None:
        err = err + a * (aP @ dQ.T)
    if dP is not None and dQ is not None:
        err = err + a * (dP @ dQ.T)
    mag = a * PQ
    if D is not None:
        mag = mag + b * np.abs(D)
        if dD is not None:
            err = err + b * dD
    err = err + 2 * U * mag
    ref = np.abs(C) if C is not None else mag
    return err + ulp_bf16(ref + err)


def ns_one_step_bound(X0, A, B, X1, dX0):
    """Bound on |X1_gpu - X1_oracle| after one Newton-Schulz step, given the
    oracle's stages and the bound dX0 on the normalised input (wide
    orientation)."""
    from oracle import muon
    a, b, c = muon.NS_COEFFS
    dA = product_bound(X0, X0, dP=dX0, dQ=dX0, C=A)
    dB = product_bound(A, A, D=A, alpha=c, beta=b, dP=dA, dQ=dA, dD=dA, C=B)
    dX1 = product_bound(B, X0.T, D=X0, alpha=1.0, beta=a, dP=dB, dQ=dX0.T, dD=dX0, C=X1)
    return dX1
