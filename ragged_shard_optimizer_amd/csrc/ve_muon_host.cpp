// ve_muon_host.cpp -- C entry points of the Newton-Schulz path: workspace
// sizing, argument checks and the launch sequence (kernels in ve_muon.hip).
//
// Sequence for a rows x cols gradient G (m = min, n = max, "wide" = rows <= cols):
//   1. fp64 partial sums of squares of G, then s = 1 / (|G|_F + eps) in fp32;
//   2. X0 = bf16(G s) in the wide orientation (m x n) and its transpose
//      (n x m), one pass through LDS tiles;
//   3. per step: A = X X^T (symmetric tiles), B = c A A + b A (symmetric
//      tiles, A as the addend), X' = B X + a X (reads X^T as the second
//      operand; writes X' and X'^T, or on the last step only the output in
//      G's orientation).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "ve.h"
#include "ve_muon.h"

using namespace ve;

namespace {

constexpr float kNsA = 3.4445f, kNsB = -4.7750f, kNsC = 2.0315f;

int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }

struct MuonLayout {
    int64_t partial, scale, x[2], xt[2], a, b, split, total;
};

// Workspace carve-up; false if the sizes overflow.
bool muon_layout(int64_t rows, int64_t cols, MuonLayout& L) {
    const int64_t m = std::min(rows, cols), n = std::max(rows, cols);
    if (m < 1 || n > (int64_t(1) << 40) / m) return false;
    const int64_t mn = round256(m * n * 2), mm = round256(m * m * 2);
    int64_t off = 0;
    L.partial = off; off += round256(int64_t(norm_blocks()) * 8);
    L.scale = off; off += 256;
    for (int i = 0; i < 2; ++i) { L.x[i] = off; off += mn; L.xt[i] = off; off += mn; }
    L.a = off; off += mm;
    L.b = off; off += mm;
    // scratch for split products: a split needs a contraction of at least
    // 16 steps of 64 (K = n for X X^T)
    L.split = -1;
    if (n >= 1024) { L.split = off; off += kSplitPartialBytes; }
    L.total = off;
    return true;
}

ve_status status_of(hipError_t e, const char* what) {
    if (e == hipSuccess) return VE_OK;
    return fail(VE_ERR_DEVICE, "%s launch failed: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

ve_status gemm(GemmArgs g, hipStream_t s, const char* what) {
    g.vec_p = aligned(g.P, 16) && g.ldp % 8 == 0;
    g.vec_q = aligned(g.Q, 16) && g.ldq % 8 == 0;
    g.vec_d = g.D && aligned(g.D, 16) && g.ldd % 8 == 0;
    g.vec_c = g.C && aligned(g.C, 16) && g.ldc % 8 == 0;
    g.vec_ct = g.CT && aligned(g.CT, 16) && g.ldct % 8 == 0;
    return status_of(launch_gemm_nt(g, s), what);
}

}  // namespace

extern "C" {

ve_status ve_muon_workspace_bytes(int64_t rows, int64_t cols, int64_t* bytes) {
    if (!bytes) return fail(VE_ERR_INVALID_ARG, "bytes is NULL");
    if (rows < 1 || cols < 1) return fail(VE_ERR_INVALID_ARG, "shape %lld x %lld", (long long)rows, (long long)cols);
    MuonLayout L;
    if (!muon_layout(rows, cols, L)) return fail(VE_ERR_UNSUPPORTED, "matrix too large");
    *bytes = L.total;
    return VE_OK;
}

ve_status ve_gemm_bf16_nt(const uint16_t* P, int64_t ldp, const uint16_t* Q, int64_t ldq, const uint16_t* D,
                          int64_t ldd, uint16_t* C, int64_t ldc, uint16_t* CT, int64_t ldct, int64_t M, int64_t N,
                          int64_t K, float alpha, float beta, int32_t symmetric, void* stream) {
    if (!P || !Q) return fail(VE_ERR_INVALID_ARG, "P or Q is NULL");
    if (!C && !CT) return fail(VE_ERR_INVALID_ARG, "C and CT are both NULL");
    if (M < 1 || N < 1 || K < 1) return fail(VE_ERR_INVALID_ARG, "M, N, K must be >= 1");
    if (ldp < K || ldq < K || (D && ldd < N) || (C && ldc < N) || (CT && ldct < M))
        return fail(VE_ERR_INVALID_ARG, "leading dimension smaller than the row");
    if (symmetric && (M != N || !C)) return fail(VE_ERR_INVALID_ARG, "symmetric needs M == N and C");
    if (gemm_tiles(M, N) > kMaxGridItems / 256 || M > (int64_t(1) << 31) || N > (int64_t(1) << 31))
        return fail(VE_ERR_UNSUPPORTED, "product too large for one launch");
    GemmArgs g{};
    g.P = P; g.ldp = ldp; g.Q = Q; g.ldq = ldq; g.D = D; g.ldd = ldd;
    g.C = C; g.ldc = ldc; g.CT = CT; g.ldct = ldct;
    g.M = M; g.N = N; g.K = K; g.alpha = alpha; g.beta = beta; g.symmetric = symmetric != 0;
    (void)hipGetLastError();
    return gemm(g, (hipStream_t)stream, "product");
}

ve_status ve_muon_newton_schulz(const uint16_t* G, uint16_t* out, int64_t rows, int64_t cols, int32_t steps,
                                float eps, void* workspace, int64_t workspace_bytes, void* stream) {
    if (!G || !out) return fail(VE_ERR_INVALID_ARG, "G or out is NULL");
    if (rows < 1 || cols < 1) return fail(VE_ERR_INVALID_ARG, "shape %lld x %lld", (long long)rows, (long long)cols);
    if (steps < 0 || steps > 64) return fail(VE_ERR_INVALID_ARG, "steps %d outside [0, 64]", steps);
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(VE_ERR_INVALID_ARG, "eps must be finite and >= 0");
    MuonLayout L;
    if (!muon_layout(rows, cols, L)) return fail(VE_ERR_UNSUPPORTED, "matrix too large");
    if (!workspace || workspace_bytes < L.total)
        return fail(VE_ERR_INVALID_ARG, "workspace of %lld bytes needed", (long long)L.total);
    if (!aligned(workspace, 256)) return fail(VE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    const int64_t m = std::min(rows, cols), n = std::max(rows, cols);
    if (gemm_tiles(m, n) > kMaxGridItems / 256 || ((rows + 63) / 64) * ((cols + 63) / 64) > kMaxGridItems / 256)
        return fail(VE_ERR_UNSUPPORTED, "matrix too large for one launch");
    const bool wide = rows <= cols;
    char* w = (char*)workspace;
    double* partial = (double*)(w + L.partial);
    float* scale = (float*)(w + L.scale);
    uint16_t* X[2] = {(uint16_t*)(w + L.x[0]), (uint16_t*)(w + L.x[1])};
    uint16_t* XT[2] = {(uint16_t*)(w + L.xt[0]), (uint16_t*)(w + L.xt[1])};
    uint16_t* A = (uint16_t*)(w + L.a);
    uint16_t* B = (uint16_t*)(w + L.b);
    float* split = L.split >= 0 ? (float*)(w + L.split) : nullptr;
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    ve_status st;
    if ((st = status_of(launch_sumsq(G, rows * cols, partial, s), "norm")) != VE_OK) return st;
    if ((st = status_of(launch_norm_scale(partial, eps, scale, s), "norm scale")) != VE_OK) return st;
    if (steps == 0) return status_of(launch_normalize(G, rows, cols, scale, out, nullptr, s), "normalise");
    // X0 (m x n) and X0^T (n x m): for a wide G the straight copy is X0, for a tall one it is X0^T
    if ((st = status_of(launch_normalize(G, rows, cols, scale, wide ? X[0] : XT[0], wide ? XT[0] : X[0], s),
                        "normalise")) != VE_OK)
        return st;
    int cur = 0;
    for (int32_t k = 0; k < steps; ++k) {
        const bool last = k + 1 == steps;
        GemmArgs g{};
        // A = X X^T
        g.P = X[cur]; g.ldp = n; g.Q = X[cur]; g.ldq = n; g.C = A; g.ldc = m;
        g.M = m; g.N = m; g.K = n; g.alpha = 1.f; g.beta = 0.f; g.symmetric = 1; g.partial = split;
        if ((st = gemm(g, s, "X X^T")) != VE_OK) return st;
        // B = c A A + b A
        g = GemmArgs{};
        g.P = A; g.ldp = m; g.Q = A; g.ldq = m; g.D = A; g.ldd = m; g.C = B; g.ldc = m;
        g.M = m; g.N = m; g.K = m; g.alpha = kNsC; g.beta = kNsB; g.symmetric = 1; g.partial = split;
        if ((st = gemm(g, s, "A A")) != VE_OK) return st;
        // X' = B X + a X, with X = (X^T)^T as the second operand
        g = GemmArgs{};
        g.P = B; g.ldp = m; g.Q = XT[cur]; g.ldq = m; g.D = X[cur]; g.ldd = n;
        g.M = m; g.N = n; g.K = m; g.alpha = 1.f; g.beta = kNsA; g.symmetric = 0; g.partial = split;
        if (last) {
            if (wide) { g.C = out; g.ldc = n; }
            else { g.CT = out; g.ldct = m; }
        } else {
            g.C = X[cur ^ 1]; g.ldc = n; g.CT = XT[cur ^ 1]; g.ldct = m;
        }
        if ((st = gemm(g, s, "B X")) != VE_OK) return st;
        cur ^= 1;
    }
    return VE_OK;
}

}  // extern "C"
