// ve_muon.h -- internal interface between the Newton-Schulz kernels
// (ve_muon.hip) and their host side (ve_muon_host.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ve_internal.h"

namespace ve {

constexpr int kCUs = 256;  // MI355X compute units

// Product C = alpha * P Q^T + beta * D on the MFMA units (ve_muon.hip).  P is
// M x K, Q is N x K, D / C are M x N and CT is N x M, all bf16 row-major
// with the given leading dimensions; D, C or CT may be null (C or CT must
// not both be).  symmetric: P Q^T is symmetric (M == N); only tiles on or
// above the diagonal are computed and mirrored into C.
struct GemmArgs {
    const uint16_t* P; int64_t ldp;
    const uint16_t* Q; int64_t ldq;
    const uint16_t* D; int64_t ldd;
    uint16_t* C; int64_t ldc;
    uint16_t* CT; int64_t ldct;
    int64_t M, N, K;
    float alpha, beta;
    int32_t symmetric;
    int32_t tiles_n;                 // set by the launcher
    bool vec_p, vec_q, vec_d, vec_c, vec_ct;  // rows allow 16-byte accesses
    bool xcd_remap;                  // set by the launcher: XCD-aware tile order
    bool sym_blocked;                // set by the launcher: symmetric tiles in 8 x 8 super-blocks (with the remap)
    // Tail split (set by the launcher): a launch covers logical tiles from
    // tile_base; with ksplit > 1 each tile's K steps are cut into ksplit
    // slices whose fp32 accumulators go to `partial` (the caller's scratch,
    // kSplitPartialBytes; null: never split).
    int32_t tiles_total, tile_base, ksplit;
    float* partial;
};
// Scratch for the split tail of a product: at most one launch's worth of
// 256 x 256 fp32 tiles, one per CU (or of 128 x 128 tiles, two per CU).
constexpr int64_t kSplitPartialBytes = int64_t(256) * 256 * 256 * 4;
hipError_t launch_gemm_nt(GemmArgs g, hipStream_t s);
int64_t gemm_tiles(int64_t M, int64_t N);
// Frobenius norm: fp64 partial sums (norm_blocks() of them), then the fp32 scale.
int norm_blocks();
hipError_t launch_sumsq(const uint16_t* x, int64_t n, double* partial, hipStream_t s);
hipError_t launch_norm_scale(const double* partial, float eps, float* scale, hipStream_t s);
hipError_t launch_normalize(const uint16_t* G, int64_t rows, int64_t cols, const float* scale, uint16_t* straight,
                            uint16_t* transposed, hipStream_t s);

}  // namespace ve
