"""GPU parity of Muon's Newton-Schulz path: the MFMA product kernel
(``ve_gemm_bf16_nt``) and the whole iteration (``ve_muon_newton_schulz``)
against the oracle (oracle/muon.py) on seeded inputs.

Gates (tests/muon_common.py): a product, and one Newton-Schulz step, must lie
within a rigorous elementwise bound of the oracle (fp32 accumulation error
plus one bf16 ulp, propagated through the stages).  Over five steps that
bound is too loose to use (it compounds the absolute values), so the five-
step result is compared in relative Frobenius norm with a first-order
allowance: the GPU and the oracle round at the same points and differ where
the accumulation order flips a rounding, about one bf16 ulp on a small share
of the entries per stage; the iteration amplifies such a perturbation at most
by max |p'(s)| over the singular values (about 3.8 on [0, 1.2]) per step.
Five steps of three stages with a 2^-8 relative perturbation each, amplified
that way, stay below 2^-8 * 3 * (1 + 3.8 + ...) applied to the share of
flipped entries; the gate is 3 % of |X|_F.  Full-size products are checked
on sampled output elements, each computed exactly on the host.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

from oracle import muon
from muon_common import U, product_bound, ns_one_step_bound, ulp_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _ve():
    import ragged_shard_optimizer_amd as ve
    return ve


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bf16_host(shape, seed, scale=1.0):
    x = np.random.default_rng(seed).standard_normal(shape) * scale
    return muon.f64_to_bf16_bits(x)


def _dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)


def _host(t):
    return muon.bf16_bits_to_f64(t.cpu().numpy().view(np.uint16))


def _empty(shape, fill=-1):
    import torch
    return torch.full(shape, fill, dtype=torch.int16, device=DEV)


# ---------------------------------------------------------------------------
# the product kernel
PRODUCT_CASES = [
    # M, N, K, alpha, beta, with D
    (128, 128, 64, 1.0, 0.0, False),
    (256, 384, 512, 1.0, 0.0, False),
    (200, 300, 136, 0.7, -1.3, True),       # ragged tiles, K tail within a step
    (37, 53, 29, 1.5, 0.25, True),          # K % 8 != 0: the 2-byte operand path
    (1, 1, 1, 1.0, 0.0, False),
    (130, 7, 1000, -2.0, 3.4445, True),
    (64, 2880, 2880, 1.0, 3.4445, True),    # GPT-OSS expert width
]


@pytest.mark.parametrize("M,N,K,alpha,beta,has_d", PRODUCT_CASES)
def test_product_parity(M, N, K, alpha, beta, has_d):
    import torch
    ve = _ve()
    Pb, Qb = _bf16_host((M, K), 1 + M), _bf16_host((N, K), 2 + N)
    Db = _bf16_host((M, N), 3) if has_d else None
    P, Q = muon.bf16_bits_to_f64(Pb), muon.bf16_bits_to_f64(Qb)
    D = muon.bf16_bits_to_f64(Db) if has_d else None
    C, CT = _empty((M, N)), _empty((N, M))
    _say(f"[gpu] product M={M} N={N} K={K}")
    ve.gemm_bf16_nt(_dev(Pb), _dev(Qb), C=C, CT=CT, D=_dev(Db) if has_d else None, alpha=alpha, beta=beta)
    torch.cuda.synchronize()
    want = muon.gemm_nt(P, Q, D, alpha, beta)
    got = _host(C)
    bound = product_bound(P, Q, D, alpha, beta, C=want)
    bad = np.abs(got - want) > bound
    assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[:3])
    # the transposed output is the same values, bit for bit
    assert np.array_equal(C.cpu().numpy().T, CT.cpu().numpy())


@pytest.mark.parametrize("n,K", [(128, 256), (384, 200), (300, 64), (45, 77)])
def test_product_symmetric_tiles(n, K):
    """X X^T with only the upper tiles computed: exactly symmetric, and
    within the bound of the oracle everywhere."""
    import torch
    ve = _ve()
    Xb = _bf16_host((n, K), 7)
    X = muon.bf16_bits_to_f64(Xb)
    Xd = _dev(Xb)
    C = _empty((n, n))
    ve.gemm_bf16_nt(Xd, Xd, C=C, symmetric=True)
    torch.cuda.synchronize()
    got = _host(C)
    assert np.array_equal(got, got.T)
    want = muon.gemm_nt(X, X)
    assert (np.abs(got - want) <= product_bound(X, X, C=want)).all()
    # with an addend, as in B = c A A + b A
    Ab = muon.f64_to_bf16_bits(want)
    A = muon.bf16_bits_to_f64(Ab)
    Ad = _dev(Ab)
    B = _empty((n, n))
    ve.gemm_bf16_nt(Ad, Ad, C=B, D=Ad, alpha=2.0315, beta=-4.7750, symmetric=True)
    torch.cuda.synchronize()
    gotB = _host(B)
    assert np.array_equal(gotB, gotB.T)
    wantB = muon.gemm_nt(A, A, A, 2.0315, -4.7750)
    assert (np.abs(gotB - wantB) <= product_bound(A, A, A, 2.0315, -4.7750, C=wantB)).all()


def test_product_rejects_bad_arguments():
    import ctypes as C
    ve = _ve()
    L = ve.lib()
    p = C.c_void_p(256)   # never dereferenced: each call is refused first
    assert L.ve_gemm_bf16_nt(None, 8, p, 8, None, 0, p, 8, None, 0, 8, 8, 8, 1.0, 0.0, 0, None) == ve.VE_ERR_INVALID_ARG
    assert L.ve_gemm_bf16_nt(p, 8, p, 8, None, 0, None, 0, None, 0, 8, 8, 8, 1.0, 0.0, 0, None) == ve.VE_ERR_INVALID_ARG
    assert L.ve_gemm_bf16_nt(p, 4, p, 8, None, 0, p, 8, None, 0, 8, 8, 8, 1.0, 0.0, 0, None) == ve.VE_ERR_INVALID_ARG
    assert L.ve_gemm_bf16_nt(p, 8, p, 8, None, 0, p, 8, None, 0, 8, 4, 8, 1.0, 0.0, 1, None) == ve.VE_ERR_INVALID_ARG
    assert L.ve_gemm_bf16_nt(p, 8, p, 8, None, 0, p, 8, None, 0, 0, 8, 8, 1.0, 0.0, 0, None) == ve.VE_ERR_INVALID_ARG


# ---------------------------------------------------------------------------
# the iteration
def _run_ns(Gb, steps):
    import torch
    ve = _ve()
    G = _dev(Gb)
    out = _empty(Gb.shape)
    ve.muon_newton_schulz(G, out, steps=steps)
    torch.cuda.synchronize()
    return _host(out)


@pytest.mark.parametrize("shape", [(64, 160), (160, 64), (96, 96), (37, 100), (1, 50), (50, 1)])
def test_normalisation(shape):
    Gb = _bf16_host(shape, 11, scale=3.0)
    G = muon.bf16_bits_to_f64(Gb)
    _say(f"[gpu] newton-schulz steps=0 {shape}")
    got = _run_ns(Gb, 0)
    want = muon.newton_schulz(G, steps=0)
    assert np.all(np.abs(got - want) <= U * np.abs(want) + ulp_bf16(want))


@pytest.mark.parametrize("shape", [(64, 160), (160, 64), (128, 128), (37, 100), (100, 37), (200, 520)])
def test_one_step_within_propagated_bound(shape):
    Gb = _bf16_host(shape, 12)
    G = muon.bf16_bits_to_f64(Gb)
    _say(f"[gpu] newton-schulz steps=1 {shape}")
    got = _run_ns(Gb, 1)
    trace = []
    want = muon.newton_schulz(G, steps=1, trace=trace)
    X0 = muon.newton_schulz(G, steps=0)
    if shape[0] > shape[1]:
        X0 = X0.T
    (A, B, X1), = trace[0]
    dX0 = U * np.abs(X0) + ulp_bf16(X0)
    bound = ns_one_step_bound(X0, A, B, X1, dX0)
    if shape[0] > shape[1]:
        bound = bound.T
    bad = np.abs(got - want) > bound
    assert not bad.any(), (int(bad.sum()), float(np.abs(got - want).max()))


NS5_ULPS = 8.0
NS5_FROB = 1.5e-2
NS5_SV = 0.012


@pytest.mark.parametrize("shape", [(256, 512), (512, 256), (300, 300), (128, 1000)])
def test_five_steps(shape):
    Gb = _bf16_host(shape, 13)
    G = muon.bf16_bits_to_f64(Gb)
    _say(f"[gpu] newton-schulz steps=5 {shape}")
    got = _run_ns(Gb, 5)
    want = muon.newton_schulz(G, steps=5)
    # The elementwise bound of one step compounds absolute values and is
    # useless after two steps.  Both sides round at the same points; they
    # differ only where the fp32 accumulation order flips a rounding, and
    # the iteration amplifies such a flip by at most max|p'(s)| ~ 3.8 per
    # step on [0, 1.2].  Gate: the largest difference within NS5_ULPS bf16
    # ulps of the largest entry, and the relative Frobenius difference within
    # NS5_FROB.  Measured on MI355X over the four shapes below: 2-5 ulps and
    # 2.7e-3-7.4e-3, singular values 0.005-0.007 from the exact iteration's
    # (the oracle's own bf16 result: 0.008); the gates are about 1.6-2x those.
    top = float(np.abs(want).max())
    ulps = float(np.abs(got - want).max() / ulp_bf16(np.array([top]))[0])
    rel = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    # the structure of the result: the singular values follow the quintic map
    exact = muon.newton_schulz(G, steps=5, rounding=False)
    s_got = np.linalg.svd(got, compute_uv=False)
    s_ex = np.linalg.svd(exact, compute_uv=False)
    sv = float(np.abs(s_got - s_ex).max())
    _say(f"[gpu] newton-schulz steps=5 {shape}: max diff {ulps:.2f} bf16 ulps of max|X|, rel Frobenius {rel:.2e}, "
         f"singular values within {sv:.4f} of the exact iteration")
    assert ulps <= NS5_ULPS, ulps
    assert rel <= NS5_FROB, rel
    assert sv <= NS5_SV, sv


# Split products: a product whose last round of 256 x 256 tiles is short
# (at most a quarter of the CUs), or that has fewer tiles than CUs, has that
# round's tiles cut along K, their fp32 slices summed in a second kernel.
#   5760 x 5760: all three products split their tail (symmetric 276 tiles, 20
#     in the tail; B X 529, 17 in the tail; 11 slices of 90 K steps, the last
#     one empty);
#   1024 x 8192: X X^T (10 tiles, 16 slices) and B X (128 tiles, 2 slices)
#     split whole, A A stays on 128 x 128 tiles;
#   2048 x 7168 (a routed expert) and its transpose: X X^T (36 tiles, 7
#     slices) and A A (4 slices) split whole, B X does not.
SPLIT_SHAPES = [(5760, 5760), (1024, 8192), (2048, 7168), (7168, 2048)]


@pytest.mark.parametrize("shape", SPLIT_SHAPES)
def test_split_one_step_within_propagated_bound(shape):
    Gb = _bf16_host(shape, 15)
    G = muon.bf16_bits_to_f64(Gb)
    _say(f"[gpu] newton-schulz steps=1 {shape} (split products)")
    got = _run_ns(Gb, 1)
    trace = []
    want = muon.newton_schulz(G, steps=1, trace=trace)
    X0 = muon.newton_schulz(G, steps=0)
    if shape[0] > shape[1]:
        X0 = X0.T
    (A, B, X1), = trace[0]
    dX0 = U * np.abs(X0) + ulp_bf16(X0)
    bound = ns_one_step_bound(X0, A, B, X1, dX0)
    if shape[0] > shape[1]:
        bound = bound.T
    bad = np.abs(got - want) > bound
    assert not bad.any(), (int(bad.sum()), float(np.abs(got - want).max()))


@pytest.mark.parametrize("shape", SPLIT_SHAPES[:3])
def test_split_matches_unsplit(shape):
    """The split path only reorders fp32 additions: two steps with and
    without it agree to within a few bf16 roundings."""
    ve = _ve()
    Gb = _bf16_host(shape, 16)
    _say(f"[gpu] newton-schulz steps=2 {shape}, split and unsplit")
    a = _run_ns(Gb, 2)
    with ve.options(gemm_split=0):
        b = _run_ns(Gb, 2)
    assert not np.array_equal(a, b)  # the split did change the summation order somewhere
    assert np.isfinite(a).all() and np.isfinite(b).all()
    assert np.linalg.norm(a - b) <= 1e-3 * np.linalg.norm(b)
    assert np.abs(a - b).max() <= 2.0 ** -6 * np.abs(b).max()


def test_repeat_calls_are_deterministic():
    import torch
    ve = _ve()
    Gb = _bf16_host((192, 640), 14)
    G = _dev(Gb)
    outs = []
    ws = torch.empty(ve.muon_workspace_bytes(192, 640), dtype=torch.uint8, device=DEV)
    for _ in range(3):
        out = _empty((192, 640))
        ve.muon_newton_schulz(G, out, steps=5, workspace=ws)
        outs.append(out)
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])


def test_newton_schulz_rejects_bad_arguments():
    import ctypes as C
    import torch
    ve = _ve()
    L = ve.lib()
    G = _empty((8, 8), 0)
    out = _empty((8, 8), 0)
    need = ve.muon_workspace_bytes(8, 8)
    ws = torch.empty(need + 256, dtype=torch.uint8, device=DEV)
    g, o, w = C.c_void_p(G.data_ptr()), C.c_void_p(out.data_ptr()), C.c_void_p(ws.data_ptr())
    assert L.ve_muon_newton_schulz(None, o, 8, 8, 5, 1e-7, w, need, None) == ve.VE_ERR_INVALID_ARG
    assert L.ve_muon_newton_schulz(g, o, 0, 8, 5, 1e-7, w, need, None) == ve.VE_ERR_INVALID_ARG
    assert L.ve_muon_newton_schulz(g, o, 8, 8, -1, 1e-7, w, need, None) == ve.VE_ERR_INVALID_ARG
    assert L.ve_muon_newton_schulz(g, o, 8, 8, 5, -1.0, w, need, None) == ve.VE_ERR_INVALID_ARG
    assert L.ve_muon_newton_schulz(g, o, 8, 8, 5, 1e-7, w, need - 1, None) == ve.VE_ERR_INVALID_ARG
    assert L.ve_muon_newton_schulz(g, o, 8, 8, 5, 1e-7, C.c_void_p(ws.data_ptr() + 16), need, None) \
        == ve.VE_ERR_INVALID_ARG


# ---------------------------------------------------------------------------
# full size: the three products of one step at a real matrix's shapes,
# sampled output elements computed exactly on the host
FULL = [("llama_mlp", 8192, 28672), ("deepseek_expert", 2048, 7168), ("gptoss_expert", 2880, 5760)]


@pytest.mark.parametrize("name,m,n", FULL)
def test_full_size_products_sampled(name, m, n):
    import torch
    ve = _ve()
    g = torch.Generator(device=DEV)
    g.manual_seed(m * 7 + n)
    # X with rows of norm ~ 1/sqrt(m) (as after normalisation), A and B of the
    # magnitudes a step produces
    X = (torch.randn(m, n, generator=g, device=DEV) / np.sqrt(m * n) * 4).to(torch.bfloat16).view(torch.int16)
    XT = X.view(torch.bfloat16).t().contiguous().view(torch.int16)
    A = _empty((m, m))
    _say(f"[gpu] full-size products {name}: {m} x {n}")
    ve.gemm_bf16_nt(X, X, C=A, symmetric=True)
    B = _empty((m, m))
    ve.gemm_bf16_nt(A, A, C=B, D=A, alpha=2.0315, beta=-4.7750, symmetric=True)
    Y, YT = _empty((m, n)), _empty((n, m))
    ve.gemm_bf16_nt(B, XT, C=Y, CT=YT, D=X, alpha=1.0, beta=3.4445)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    Xh, Ah, Bh = _host(X), _host(A), _host(B)
    Yh = _host(Y)
    assert torch.equal(Y.view(torch.bfloat16).t().contiguous().view(torch.int16), YT)
    for (P, Q, D, alpha, beta, C) in ((Xh, Xh, None, 1.0, 0.0, Ah), (Ah, Ah, Ah, 2.0315, -4.7750, Bh),
                                      (Bh, Xh.T, Xh, 1.0, 3.4445, Yh)):
        rows = rng.integers(0, C.shape[0], 64)
        cols = rng.integers(0, C.shape[1], 64)
        Pr, Qc = P[rows], Q[cols]
        Dr = None if D is None else D[rows, cols][:, None]
        for t in range(len(rows)):
            want = muon.gemm_nt(Pr[t:t + 1], Qc[t:t + 1], None if Dr is None else Dr[t:t + 1], alpha, beta)
            bd = product_bound(Pr[t:t + 1], Qc[t:t + 1], None if Dr is None else Dr[t:t + 1], alpha, beta, C=want)
            assert abs(C[rows[t], cols[t]] - want[0, 0]) <= bd[0, 0], (name, rows[t], cols[t])
    del X, XT, A, B, Y, YT
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M,N,K,sym", [(7000, 7040, 1024, False), (8000, 8000, 1024, True), (6000, 9000, 2880, False)])
def test_large_ragged_products_sampled(M, N, K, sym):
    """Products large enough for the direct-to-LDS kernel, with ragged tile
    edges (rows past M or N read clamped rows whose outputs are dropped) and a
    partial last tile of a symmetric product: sampled elements within the
    bound, C^T equal to C, the symmetric result exactly symmetric."""
    import torch
    ve = _ve()
    g = torch.Generator(device=DEV)
    g.manual_seed(M + N + K)
    P = torch.randn(M, K, generator=g, device=DEV).to(torch.bfloat16).view(torch.int16)
    Q = P if sym else torch.randn(N, K, generator=g, device=DEV).to(torch.bfloat16).view(torch.int16)
    D = torch.randn(M, N, generator=g, device=DEV).to(torch.bfloat16).view(torch.int16)
    if sym:
        D = (D.view(torch.bfloat16) + D.view(torch.bfloat16).t()).contiguous().view(torch.int16)
    C = _empty((M, N))
    CT = None if sym else _empty((N, M))
    _say(f"[gpu] large product M={M} N={N} K={K} symmetric={sym}")
    ve.gemm_bf16_nt(P, Q, C=C, CT=CT, D=D, alpha=0.75, beta=-0.5, symmetric=sym)
    torch.cuda.synchronize()
    if sym:
        assert torch.equal(C, C.view(torch.bfloat16).t().contiguous().view(torch.int16))
    else:
        assert torch.equal(C.view(torch.bfloat16).t().contiguous().view(torch.int16), CT)
    Ph, Qh, Dh, Ch = _host(P), _host(Q), _host(D), _host(C)
    rng = np.random.default_rng(1)
    rows = np.concatenate([rng.integers(0, M, 200), [M - 1, M - 1, 0]])
    cols = np.concatenate([rng.integers(0, N, 200), [N - 1, 0, N - 1]])
    for i, j in zip(rows, cols):
        want = muon.gemm_nt(Ph[i:i + 1], Qh[j:j + 1], Dh[i:i + 1, j:j + 1], 0.75, -0.5)
        bd = product_bound(Ph[i:i + 1], Qh[j:j + 1], Dh[i:i + 1, j:j + 1], 0.75, -0.5, C=want)
        assert abs(Ch[i, j] - want[0, 0]) <= bd[0, 0], (i, j, Ch[i, j], want[0, 0])


# The direct-to-LDS product configurations: 6 (4 waves of 128 x 128, two
# LDS stages), 9 (8 waves of 128 x 64, two stages), 13 (8 waves, P in three
# LDS stages, Q staged through registers) and 14 (128 x 128 tiles of 2
# waves of 128 x 64, two stages).  They feed the MFMAs the same fragments in
# the same order, so their outputs agree bit for bit; ragged edges (rows
# past M or N), a symmetric product and C^T included.
@pytest.mark.parametrize("M,N,K,sym", [(7000, 7040, 1024, False), (2048, 2048, 7168, True), (300, 520, 640, False),
                                       (1000, 300, 2880, False)])
def test_product_configurations_agree(M, N, K, sym):
    import torch
    ve = _ve()
    g = torch.Generator(device=DEV)
    g.manual_seed(M * 3 + N + K)
    P = torch.randn(M, K, generator=g, device=DEV).to(torch.bfloat16).view(torch.int16)
    Q = P if sym else torch.randn(N, K, generator=g, device=DEV).to(torch.bfloat16).view(torch.int16)
    D = torch.randn(M, N, generator=g, device=DEV).to(torch.bfloat16).view(torch.int16)
    if sym:
        D = (D.view(torch.bfloat16) + D.view(torch.bfloat16).t()).contiguous().view(torch.int16)
    outs = {}
    for cfg in (9, 6, 13, 14):
        C = _empty((M, N))
        CT = None if sym else _empty((N, M))
        _say(f"[gpu] product configuration {cfg}: M={M} N={N} K={K} symmetric={sym}")
        with ve.options(gemm_cfg=cfg):
            ve.gemm_bf16_nt(P, Q, C=C, CT=CT, D=D, alpha=0.75, beta=-0.5, symmetric=sym)
        torch.cuda.synchronize()
        outs[cfg] = (C, CT)
    for cfg in (6, 13, 14):
        assert torch.equal(outs[cfg][0], outs[9][0]), cfg
        if not sym:
            assert torch.equal(outs[cfg][1], outs[9][1]), cfg
    # and the default within the bound on sampled elements
    Ph, Qh, Dh, Ch = _host(P), _host(Q), _host(D), _host(outs[13][0])
    rng = np.random.default_rng(2)
    for i, j in zip(np.concatenate([rng.integers(0, M, 60), [M - 1]]), np.concatenate([rng.integers(0, N, 60), [N - 1]])):
        want = muon.gemm_nt(Ph[i:i + 1], Qh[j:j + 1], Dh[i:i + 1, j:j + 1], 0.75, -0.5)
        bd = product_bound(Ph[i:i + 1], Qh[j:j + 1], Dh[i:i + 1, j:j + 1], 0.75, -0.5, C=want)
        assert abs(Ch[i, j] - want[0, 0]) <= bd[0, 0], (i, j)
