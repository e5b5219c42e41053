// ve_muon.hip -- Muon's Newton-Schulz orthogonalisation of one gathered 2-D
// matrix on the MFMA units.
//
// Distributed Muon gathers each full 2-D update matrix on one root rank,
// runs the Newton-Schulz iteration there and redistributes the result
// (veScale-FSDP talk notes, "Case study: 8-bit Adam and distributed Muon";
// Dutch summary, "Muon-optimalisator").  This file is the root rank's dense
// work.  The iteration is the published Muon quintic (Jordan et al., 2024):
//
//   X0 = G / (|G|_F + eps), transposed to the wide orientation (m <= n);
//   repeat: A = X X^T;  B = b A + c A A;  X <- a X + B X;
//   (a, b, c) = (3.4445, -4.7750, 2.0315).
//
// Precision: X, A, B are stored as bf16; products accumulate in fp32 on the
// MFMA units; every epilogue is fp32 and rounds once to bf16 (nearest even).
// The Frobenius norm is accumulated in fp64.
//
// All three products are "NT" (C = P Q^T, both operands with contiguous
// contraction index): X X^T directly; A A = A A^T since A is symmetric; and
// B X = B (X^T)^T, which reads X^T -- so the step that produces X also
// writes X^T from its epilogue.  X X^T and A A are symmetric: only tiles on
// or above the diagonal are computed and each is mirrored.
//
// Product kernel (gfx950): 256 threads = 4 waves as 2 x 2, a 128 x 128 output
// tile per workgroup, each wave 64 x 64 = 2 x 2 MFMA 32x32x16 bf16 tiles in
// fp32 accumulators.  The contraction runs in steps of 64 through LDS, double
// buffered: the next step's global loads are issued before the current
// step's MFMAs, one barrier per step.  LDS rows are padded by 16 bytes so
// that the 16-byte fragment reads of 16 consecutive rows hit distinct banks.
//
// MFMA 32x32x16 bf16 operand layout (lane l = 0..63): A fragment = 8
// consecutive k of row l%32 starting at k = 8*(l/32); B fragment = the same
// for column l%32; accumulator register r of lane l holds row
// 8*(r/4) + 4*(l/32) + r%4, column l%32.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>

#include "ve_device.h"
#include "ve_muon.h"

namespace ve {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// A product configuration: workgroup tile BM x BN, contraction step BK,
// each wave a WM x WN tile of (WM/32) x (WN/32) MFMA 32x32 blocks.
template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
    static constexpr int THREADS = 64 * WAVES_M * WAVES_N;
    static constexpr int TM = WM / 32, TN = WN / 32;
    static constexpr int LDK = BK + 8;             // padded LDS row (bf16): 16 rows hit distinct banks
    static constexpr int VPR = BK / 8;             // 16-byte vectors per operand row of one step
    static constexpr int PV = BM * VPR / THREADS;  // staged vectors per thread
    static constexpr int QV = BN * VPR / THREADS;
    static constexpr int LDC = BN + 4;             // fp32 output rows (padded)
    static constexpr int OP_BYTES = 2 * (BM + BN) * LDK * 2;
    static constexpr int C_BYTES = WM * LDC * 4;   // one wave-row pass of the output tile
    static constexpr int SMEM = OP_BYTES > C_BYTES ? OP_BYTES : C_BYTES;
    static_assert(BM % WM == 0 && BN % WN == 0 && WM % 32 == 0 && WN % 32 == 0 && BK % 16 == 0, "shape");
    static_assert(PV * THREADS == BM * VPR && QV * THREADS == BN * VPR, "staging must divide evenly");
    static_assert((WM * BN / 8) % THREADS == 0, "epilogue must divide evenly");
};

// The configurations compiled in; VE_GEMM_CFG (environment) selects one for tuning.
#define VE_GEMM_CFGS(X) \
    X(0, 128, 128, 64, 64, 64) \
    X(2, 256, 256, 64, 128, 64)

constexpr int kNormBlocks = 1024;    // partial sums of the Frobenius norm

__device__ __forceinline__ uint16_t to_bf16(float x) { return (uint16_t)pack_bf16x2(x, 0.f); }
__device__ __forceinline__ float from_bf16(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// 8 consecutive bf16 of row `r` starting at column `k` of a row-major matrix
// with `rows` x `cols` valid elements and leading dimension `ld`; zeros
// outside.  VEC: rows are 16-byte aligned and cols is a multiple of 8, so
// every in-range group of 8 is one 16-byte access.
template <bool VEC>
__device__ __forceinline__ u32x4 load8(const uint16_t* base, int64_t ld, int64_t rows, int64_t cols, int64_t r,
                                       int64_t k) {
    u32x4 v = u32x4{0, 0, 0, 0};
    if (r >= rows || k >= cols) return v;
    const VE_GLOBAL uint16_t* p = (const VE_GLOBAL uint16_t*)(base + r * ld + k);
    if constexpr (VEC) {
        return *(const VE_GLOBAL u32x4*)p;
    } else {
        uint16_t e[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) e[t] = (k + t < cols) ? p[t] : (uint16_t)0;
        v.x = e[0] | ((uint32_t)e[1] << 16);
        v.y = e[2] | ((uint32_t)e[3] << 16);
        v.z = e[4] | ((uint32_t)e[5] << 16);
        v.w = e[6] | ((uint32_t)e[7] << 16);
        return v;
    }
}

// Output tile of this workgroup.  Workgroups are dispatched round-robin over
// the 8 XCDs, each with its own L2; with g.xcd_remap each XCD is given a
// contiguous slice of the tile sequence.  A full product walks groups of 8
// tile rows column by column, so the operand panels a slice touches are few
// and stay in its L2.  A symmetric product launches only the tiles on or
// above the diagonal: with the remap in 8 x 8 super-blocks (so that a slice
// touches few panels), else row by row.
// Tile (ti, tj) of logical tile index t.
__device__ __forceinline__ void tile_at(const GemmArgs& g, int t, int& ti, int& tj) {
    if (g.symmetric && g.sym_blocked) {
        // super-blocks of 8 x 8 tiles on or above the diagonal, row by row;
        // inside one, tiles row by row (the triangle on the diagonal)
        constexpr int SB = 8;
        const int n = g.tiles_n, ns = (n + SB - 1) / SB;
        int rem = t;
        for (int I = 0; I < ns; ++I) {
            const int ri = min(SB, n - SB * I);
            for (int J = I; J < ns; ++J) {
                const int cj = min(SB, n - SB * J);
                const int cnt = I == J ? ri * (ri + 1) / 2 : ri * cj;
                if (rem < cnt) {
                    if (I < J) {
                        ti = SB * I + rem / cj;
                        tj = SB * J + rem % cj;
                        return;
                    }
                    int r = 0;
                    while (rem >= ri - r) {
                        rem -= ri - r;
                        ++r;
                    }
                    ti = SB * I + r;
                    tj = SB * I + r + rem;
                    return;
                }
                rem -= cnt;
            }
        }
        ti = tj = 0;  // not reached: t < tiles_total
        return;
    }
    if (g.symmetric) {
        // row r of the upper triangle holds tiles_n - r tiles
        int r = 0, rem = t;
        while (rem >= g.tiles_n - r) {
            rem -= g.tiles_n - r;
            ++r;
        }
        ti = r;
        tj = r + rem;
        return;
    }
    constexpr int kGroup = 8;
    const int tiles_m = g.tiles_total / g.tiles_n;
    const int per_group = kGroup * g.tiles_n;
    const int first = (t / per_group) * kGroup;
    const int gm = min(tiles_m - first, kGroup);
    const int r = t % per_group;
    ti = first + r % gm;
    tj = r / gm;
}

// This workgroup's tile and K slice.  Launches cover logical tiles
// [tile_base, tile_base + gridDim.x / ksplit); with ksplit > 1, consecutive
// workgroups take the K slices of one tile.  Whole-tile launches whose size
// is a multiple of 8 spread consecutive tiles over the 8 XCDs' L2s in
// blocks (block b -> (b mod 8) * nb/8 + b / 8).
__device__ __forceinline__ int tile_of(const GemmArgs& g, int& ti, int& tj) {
    const int nb = gridDim.x;
    int bid = blockIdx.x, split = 0;
    if (g.ksplit > 1) {
        split = bid % g.ksplit;
        bid /= g.ksplit;
    } else if (g.xcd_remap && nb % 8 == 0) {
        bid = (bid % 8) * (nb / 8) + bid / 8;
    }
    tile_at(g, g.tile_base + bid, ti, tj);
    return split;
}

// 8 bf16 <-> a 16-byte vector
__device__ __forceinline__ u32x4 pack8(const float* v) {
    return u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
}

template <class CF, bool HAS_D, bool HAS_C, bool HAS_CT, bool VEC>
__global__ void __launch_bounds__(CF::THREADS) k_gemm_nt(GemmArgs g) {
    constexpr int BM = CF::BM, BN = CF::BN, BK = CF::BK, WM = CF::WM, WN = CF::WN, TM = CF::TM, TN = CF::TN;
    constexpr int LDK = CF::LDK, LDC = CF::LDC, NT = CF::THREADS, VPR = CF::VPR;
    int ti, tj;
    tile_of(g, ti, tj);
    const int64_t i0 = (int64_t)ti * BM, j0 = (int64_t)tj * BN;
    // operand tiles (2 buffers each), reused for the fp32 output afterwards
    __shared__ __attribute__((aligned(16))) unsigned char smem[CF::SMEM];
    uint16_t* sP = (uint16_t*)smem;                   // [2][BM * LDK]
    uint16_t* sQ = sP + 2 * BM * LDK;                 // [2][BN * LDK]
    float* sC = (float*)smem;                         // [WM][LDC], one wave row at a time
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave / CF::WAVES_N, wc = wave % CF::WAVES_N;

    f32x16 acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    // global -> register staging: vector v = tid + NT*q covers row v/VPR, k-vector v%VPR
    u32x4 rp[CF::PV], rq[CF::QV];
    auto gload = [&](int64_t k0) {
#pragma unroll
        for (int q = 0; q < CF::PV; ++q) {
            const int v = tid + NT * q;
            rp[q] = load8<VEC>(g.P, g.ldp, g.M, g.K, i0 + v / VPR, k0 + (v % VPR) * 8);
        }
#pragma unroll
        for (int q = 0; q < CF::QV; ++q) {
            const int v = tid + NT * q;
            rq[q] = load8<VEC>(g.Q, g.ldq, g.N, g.K, j0 + v / VPR, k0 + (v % VPR) * 8);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int q = 0; q < CF::PV; ++q) {
            const int v = tid + NT * q;
            *(u32x4*)&sP[buf * BM * LDK + (v / VPR) * LDK + (v % VPR) * 8] = rp[q];
        }
#pragma unroll
        for (int q = 0; q < CF::QV; ++q) {
            const int v = tid + NT * q;
            *(u32x4*)&sQ[buf * BN * LDK + (v / VPR) * LDK + (v % VPR) * 8] = rq[q];
        }
    };

    const int64_t nk = (g.K + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    const int frow = lane & 31, fk = (lane >> 5) * 8;
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int cur = (int)(kt & 1);
        if (kt + 1 < nk) gload((kt + 1) * BK);
        const uint16_t* cp = sP + cur * BM * LDK + (wr * WM + frow) * LDK + fk;
        const uint16_t* cq = sQ + cur * BN * LDK + (wc * WN + frow) * LDK + fk;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            bf16x8 fa[TM], fb[TN];
#pragma unroll
            for (int t = 0; t < TM; ++t)
                fa[t] = __builtin_bit_cast(bf16x8, *(const u32x4*)&cp[t * 32 * LDK + kk * 16]);
#pragma unroll
            for (int t = 0; t < TN; ++t)
                fb[t] = __builtin_bit_cast(bf16x8, *(const u32x4*)&cq[t * 32 * LDK + kk * 16]);
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int b = 0; b < TN; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
        }
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }

    // epilogue, one wave row (WM rows of the tile) at a time through LDS:
    //   1. the accumulators into the fp32 staging rows (the operand buffers are
    //      dead; stored straight from the accumulator registers);
    //   2. row-major: v = bf16(alpha * stage + beta * D), C written as 16-byte runs of a
    //      row; the rounded value goes back to the stage for the transpose;
    //   3. transposed: C^T (or the mirrored tile of a symmetric C) written as
    //      16-byte runs of its rows, lanes on consecutive columns of the stage
    //      so the LDS reads are conflict-free.
    const bool mirror = g.symmetric && ti < tj;
    const bool transpose = HAS_CT || mirror;
    uint16_t* T = HAS_CT ? g.CT : g.C;
    const int64_t ldt = HAS_CT ? g.ldct : g.ldc;
    const bool vec_t = HAS_CT ? g.vec_ct : g.vec_c;
    const int64_t ncols = min((int64_t)BN, g.N - j0);
#pragma unroll 1
    for (int pass = 0; pass < CF::WAVES_M; ++pass) {
        const int64_t r0 = i0 + (int64_t)pass * WM;                  // first tile row of this pass
        const int64_t mrows = min((int64_t)WM, g.M - r0);
        if (wr == pass) {
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int b = 0; b < TN; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = a * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                        const int col = wc * WN + b * 32 + (lane & 31);
                        sC[row * LDC + col] = acc[a][b][r];
                    }
        }
        __syncthreads();
        if (mrows > 0) {
#pragma unroll 2
            for (int q = 0; q < (WM * BN / 8) / NT; ++q) {
                const int id = tid + NT * q;
                const int row = id / (BN / 8), c8 = (id % (BN / 8)) * 8;
                if (row >= mrows || c8 >= ncols) continue;
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = g.alpha * sC[row * LDC + c8 + e];
                const int64_t i = r0 + row, j = j0 + c8;
                const bool full = c8 + 8 <= ncols;
                if (HAS_D) {
                    if (full && g.vec_d) {
                        const u32x4 d = *(const VE_GLOBAL u32x4*)(g.D + i * g.ldd + j);
                        const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            v[e] = __builtin_fmaf(g.beta, (e & 1) ? bf_hi(dw[e >> 1]) : bf_lo(dw[e >> 1]), v[e]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (c8 + e < ncols) v[e] = __builtin_fmaf(g.beta, from_bf16(g.D[i * g.ldd + j + e]), v[e]);
                    }
                }
                const u32x4 h = pack8(v);
                const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
                if (HAS_C) {
                    if (full && g.vec_c) {
                        *(VE_GLOBAL u32x4*)(g.C + i * g.ldc + j) = h;
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (c8 + e < ncols) g.C[i * g.ldc + j + e] = (uint16_t)(hw[e >> 1] >> (16 * (e & 1)));
                    }
                }
                if (transpose) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        sC[row * LDC + c8 + e] = (e & 1) ? bf_hi(hw[e >> 1]) : bf_lo(hw[e >> 1]);
                }
            }
            if (transpose) {
                __syncthreads();
#pragma unroll 2
                for (int q = 0; q < (WM * BN / 8) / NT; ++q) {
                    const int id = tid + NT * q;
                    const int col = id % BN, r8 = (id / BN) * 8;
                    if (col >= ncols || r8 >= mrows) continue;
                    float v[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = sC[(r8 + e) * LDC + col];
                    const u32x4 h = pack8(v);               // exact: the values are bf16 already
                    const int64_t j = j0 + col, i = r0 + r8;
                    if (r8 + 8 <= mrows && vec_t) {
                        *(VE_GLOBAL u32x4*)(T + j * ldt + i) = h;
                    } else {
                        const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (r8 + e < mrows) T[j * ldt + i + e] = (uint16_t)(hw[e >> 1] >> (16 * (e & 1)));
                    }
                }
            }
        }
        __syncthreads();
    }
}

// Large-tile product with direct global -> LDS loads (gfx950
// global_load_lds_dwordx4: each lane's 16 bytes land at the wave's LDS base
// + 16 * lane).  256 x 256 output tile; waves of WM x WN (WM/32 x WN/32 MFMA
// 32x32 blocks); contraction steps of BK in a ring of STAGES LDS stages, so
// the loads for step k + STAGES - 1 are in flight while step k computes and
// each step waits only for the oldest outstanding stage.  Operand rows are
// BK * 2 bytes with no padding; the 16-byte chunks of row r are stored
// XOR-swizzled (chunk c at slot c ^ s(r)) so that the fragment reads of
// consecutive rows spread over the banks.  Each DMA instruction of a wave
// fills 1 KiB of whole rows.  Requires K % BK == 0 and 16-byte operand rows;
// rows past M or N read a clamped valid row (their outputs are never stored).
// instruction classes for __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100;

// s_waitcnt operand: wait until at most n vector-memory operations are
// outstanding (expcnt and lgkmcnt left unconstrained).
constexpr int waitcnt_vm(int n) { return 0x0F70 | (n & 15) | (((n >> 4) & 3) << 14); }

#ifndef VE_QWRITE_SUBSTEP
#define VE_QWRITE_SUBSTEP 2  // sub-step of a step whose start writes the next step's Q to LDS
#endif
// QST: Q is staged through registers (global -> VGPR two steps ahead ->
// LDS one step ahead, two LDS stages) while P keeps the direct LDS DMA in
// STAGES stages, so that both operands' loads have two steps to land.
template <int WM_, int WN_, int BK_, int STAGES_, bool QST_ = false, int BM_ = 256, int BN_ = 256>
struct DmaCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, STAGES = STAGES_;
    static constexpr bool QST = QST_;
    static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN, WAVES = WAVES_M * WAVES_N;
#ifndef VE_EARLY_BARRIER
#define VE_EARLY_BARRIER 1
#endif
    // The next step's barrier and first fragment reads are placed inside
    // the last sub-step's MFMAs, so the read latency after each barrier is
    // covered by MFMAs instead of stalling every wave at the step boundary.
    static constexpr bool EARLY_BARRIER = VE_EARLY_BARRIER != 0;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int TM = WM / 32, TN = WN / 32;
    static constexpr int CHUNKS = BK / 8;                      // 16-byte chunks per operand row
    static constexpr int ROWS_PER_DMA = 1024 / (BK * 2);       // rows one wave instruction fills
    static constexpr int DMA_PER_OP = BM / ROWS_PER_DMA / WAVES;  // instructions per operand per thread
    static constexpr int STAGE_ELEMS = (BM + BN) * BK;
    static constexpr int OP_BYTES = QST ? (STAGES * BM + 2 * BN) * BK * 2 : STAGES * STAGE_ELEMS * 2;
    static constexpr int PASS_ROWS = 64;
    static constexpr int LDC = BN + 4;
    static constexpr int SMEM = OP_BYTES > PASS_ROWS * LDC * 4 ? OP_BYTES : PASS_ROWS * LDC * 4;
    static_assert(DMA_PER_OP * ROWS_PER_DMA * WAVES == BM, "DMA rows must divide evenly");
    static_assert(SMEM <= 160 * 1024, "LDS");
    // workgroups a CU holds at once, as its LDS allows (the split policy
    // counts that many slots a CU)
    static constexpr int PER_CU = (160 * 1024) / SMEM;
    // swizzle: rows sharing a bank line get distinct slots
    __device__ static __forceinline__ int swz(int r) {
        if constexpr (CHUNKS == 8) return (r & 7) ^ ((r >> 3) & 1);
        else return (r >> 1) & 3;
    }
};

// (id, wave tile, K step, P stages, Q staged through registers, tile);
// 14: 128 x 128 tiles of 2 waves in 64 KiB of LDS, two workgroups a CU.
#define VE_DMA_CFGS(X)                     \
    X(6, 128, 128, 64, 2, false, 256, 256) \
    X(9, 128, 64, 64, 2, false, 256, 256)  \
    X(13, 128, 64, 64, 3, true, 256, 256)  \
    X(14, 128, 64, 64, 2, false, 128, 128)

template <class CF, bool HAS_D, bool HAS_C, bool HAS_CT>
__device__ __forceinline__ void dma_epilogue(const GemmArgs& g, f32x16 (&acc)[CF::TM][CF::TN], int ti, int tj,
                                             unsigned char* smem);

// Raw accumulators of one (tile, K slice) work item, in fragment order
// [wave][a][b][r][lane] (64 consecutive floats per store), at item
// (tile - tile_base) * ksplit + split of the fp32 partial buffer.
template <class CF>
__device__ __forceinline__ float* partial_at(const GemmArgs& g, int item) {
    return g.partial + (int64_t)item * (CF::BM * CF::BN);
}

template <class CF, bool HAS_D, bool HAS_C, bool HAS_CT>
__global__ void __launch_bounds__(CF::THREADS) k_gemm_nt_dma(GemmArgs g) {
    constexpr int BM = CF::BM, BN = CF::BN, BK = CF::BK, WM = CF::WM, WN = CF::WN, TM = CF::TM, TN = CF::TN;
    constexpr int S = CF::STAGES, SE = CF::STAGE_ELEMS;
    int ti, tj;
    const int split = tile_of(g, ti, tj);
    const int64_t i0 = (int64_t)ti * BM, j0 = (int64_t)tj * BN;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[CF::SMEM];
    uint16_t* ops = (uint16_t*)smem;                  // stage s: P rows [BM * BK], then Q rows [BN * BK]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave / CF::WAVES_N, wc = wave % CF::WAVES_N;

    f32x16 acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    // K steps of this work item: all of them, or slice `split` of ksplit
    const int64_t nk_all = g.K / BK;
    int64_t kbeg = 0, nk = nk_all;
    if (g.ksplit > 1) {
        const int64_t per = (nk_all + g.ksplit - 1) / g.ksplit;
        kbeg = min((int64_t)split * per, nk_all);
        nk = min(per, nk_all - kbeg);
    }

    // DMA: instruction q of wave w fills rows [(WAVES q + w) R, +R) of an
    // operand (R = rows per KiB); lane l writes slot l % CHUNKS of row
    // l / CHUNKS, i.e. logical chunk (l % CHUNKS) ^ s(row)
    const int lrow = lane / CF::CHUNKS, lslot = lane % CF::CHUNKS;
    auto dma_op = [&](const uint16_t* base, int64_t ld, int64_t rows, int64_t r0, uint16_t* dst, int64_t k0) {
#pragma unroll
        for (int q = 0; q < CF::DMA_PER_OP; ++q) {
            const int blk = CF::WAVES * q + wave;
            const int row = blk * CF::ROWS_PER_DMA + lrow;
            const int64_t gr = min(r0 + row, rows - 1);
            const uint16_t* src = base + gr * ld + k0 + 8 * (lslot ^ CF::swz(row));
            __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                             (void __attribute__((address_space(3)))*)(dst + blk * CF::ROWS_PER_DMA * BK),
                                             16, 0, 0);
        }
    };
    if constexpr (!CF::QST) {
    auto dma_step = [&](int64_t kt) {
        uint16_t* st = ops + (int)(kt % S) * SE;
        dma_op(g.P, g.ldp, g.M, i0, st, (kbeg + kt) * BK);
        dma_op(g.Q, g.ldq, g.N, j0, st + BM * BK, (kbeg + kt) * BK);
    };

    // prologue: stages 0 .. S-2 in flight
#pragma unroll
    for (int p = 0; p < S - 1; ++p)
        if (p < nk) dma_step(p);
    const int frow = lane & 31, fhalf = lane >> 5;
    const int fs = CF::swz(lane & 15);                // rows t*32 + frow share frow's swizzle
    // fragments double-buffered over the 16-deep sub-steps: the reads for
    // sub-step kk+1 are issued before the MFMAs of kk, so the LDS latency
    // hides behind TM*TN MFMAs
    bf16x8 fa[2][TM], fb[2][TN];
    auto frag = [&](int buf, int kk, int64_t kt) {
        const uint16_t* st = ops + (int)(kt % S) * SE;
        const uint16_t* cp = st + (wr * WM + frow) * BK;
        const uint16_t* cq = st + BM * BK + (wc * WN + frow) * BK;
        const int slot = ((2 * kk + fhalf) ^ fs) * 8;
#pragma unroll
        for (int t = 0; t < TM; ++t) fa[buf][t] = __builtin_bit_cast(bf16x8, *(const u32x4*)&cp[t * 32 * BK + slot]);
#pragma unroll
        for (int t = 0; t < TN; ++t) fb[buf][t] = __builtin_bit_cast(bf16x8, *(const u32x4*)&cq[t * 32 * BK + slot]);
    };
    // step kt's stage is complete when at most the S-2 younger stages are
    // outstanding; then every wave has its own loads of it complete, and a
    // bare barrier (no memory fence, which would wait for the younger stages
    // too) with compiler-level clobbers, so no LDS access moves across it
    auto stage_ready = [&](int64_t kt) {
        if (kt + S - 2 < nk) {
            constexpr int younger = (S - 2) * 2 * CF::DMA_PER_OP;
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(younger));
        } else {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    auto mfma = [&](int buf, int a, int b) {
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][a], fb[buf][b], acc[a][b], 0, 0, 0);
    };
    if constexpr (CF::EARLY_BARRIER) {
        stage_ready(0);
        frag(0, 0, 0);
    }
    for (int64_t kt = 0; kt < nk; ++kt) {
        if constexpr (!CF::EARLY_BARRIER) {
            stage_ready(kt);
            if (kt + S - 1 < nk) dma_step(kt + S - 1);  // into the stage consumed at step kt - 1
            frag(0, 0, kt);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, TM + TN, 0);
        } else {
            // the barrier that frees this stage (every wave's reads of step
            // kt - 1 complete) was passed inside step kt - 1
            if (kt + S - 1 < nk) dma_step(kt + S - 1);
        }
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            if (kk + 1 < BK / 16) frag((kk + 1) & 1, kk + 1, kt);
            if constexpr (CF::EARLY_BARRIER) {
                if (kk + 1 == BK / 16) {
                    // last sub-step: every read of this step's stage is
                    // complete (waited before these MFMAs).  A few MFMAs,
                    // then the next step's barrier and its first fragment
                    // reads, each followed by one MFMA.  On the last step
                    // the reads fetch an unused stage.
                    constexpr int post = TM + TN, pre = TM * TN - post;
                    static_assert(pre >= 1, "early-barrier shape");
#pragma unroll
                    for (int i = 0; i < pre; ++i) mfma(kk & 1, i / TN, i % TN);
                    __builtin_amdgcn_sched_group_barrier(kSchedMfma, pre, 0);
                    stage_ready(kt + 1);
                    frag(0, 0, kt + 1);
#pragma unroll
                    for (int i = pre; i < TM * TN; ++i) mfma(kk & 1, i / TN, i % TN);
#pragma unroll
                    for (int i = 0; i < post; ++i) {
                        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                    }
                    continue;
                }
            }
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int b = 0; b < TN; ++b) mfma(kk & 1, a, b);
            // schedule: one MFMA, then one read of the next sub-step, ...
            if (kk + 1 < BK / 16) {
#pragma unroll
                for (int i = 0; i < TM + TN; ++i) {
                    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
                }
            }
            constexpr int kRestMid = TM * TN - (TM + TN), kRestLast = TM * TN;
            static_assert(kRestMid >= 0, "sub-step too small for the interleave");
            if (kk + 1 < BK / 16) {
                if constexpr (kRestMid > 0) __builtin_amdgcn_sched_group_barrier(kSchedMfma, kRestMid, 0);
            } else {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, kRestLast, 0);
            }
        }
    }
    } else {
        // P: LDS DMA through a buffer resource based at the tile's first row
        // (the MUBUF form: the compiler tracks it like an ordinary load,
        // where the FLAT form makes it wait for every outstanding access
        // before any use of a loaded register).  Q: each thread loads the
        // 16-byte chunks the DMA would have written (same rows, same
        // swizzled slots) into registers two steps ahead and writes them to
        // LDS at the end of the step before their use.  Every step issues
        // the same loads (past the last step they re-read valid data of the
        // last step), so the wait counts are constants.
        constexpr int SP = S, SQ = 2, PE = BM * BK, QE = BN * BK, DL = CF::DMA_PER_OP;
        static_assert(SP == 3, "P stages");
        constexpr int RR = CF::ROWS_PER_DMA * CF::WAVES;  // rows one DMA round covers
        static_assert(CF::CHUNKS == 8 && CF::WAVES % 2 == 0, "swizzle of a thread's rows independent of the round");
        uint16_t* pst = ops;            // [SP][PE]
        uint16_t* qst = ops + SP * PE;  // [SQ][QE]
        // Operand rows past M or N are past the end of the tile's buffer
        // range: their loads return zeros (those outputs are never stored).
        // Thread rows: lane row lrow of 8-row block (WAVES q + wave), whose
        // swizzle does not depend on q; the offsets are recomputed per load
        // from one per-lane base and a wave-uniform part.
        const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(g.P + i0 * g.ldp), (short)0, (int)(uint32_t)((min(i0 + BM, g.M) - i0) * g.ldp * 2), 0x00020000);
        const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(g.Q + j0 * g.ldq), (short)0, (int)(uint32_t)((min(j0 + BN, g.N) - j0) * g.ldq * 2), 0x00020000);
        const int trow = wave * CF::ROWS_PER_DMA + lrow, tchunk = 8 * (lslot ^ CF::swz(trow));
        const uint32_t pv0 = (uint32_t)((trow * g.ldp + tchunk) * 2), qv0 = (uint32_t)((trow * g.ldq + tchunk) * 2);
        auto kcol = [&](int64_t kt) { return (kbeg + (kt < nk ? kt : nk - 1)) * BK; };
        auto pstage = [&](int64_t kt) {
            uint16_t* st = pst + (int)(kt % SP) * PE;
            const uint32_t k2 = (uint32_t)(kcol(kt) * 2);
#pragma unroll
            for (int q = 0; q < DL; ++q) {
                const int blk = CF::WAVES * q + wave;
                uint32_t v = pv0 + k2 + (uint32_t)(q * RR * g.ldp * 2);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    prs, (void __attribute__((address_space(3)))*)(st + blk * CF::ROWS_PER_DMA * BK), 16, (int)v, 0, 0, 0);
            }
        };
        u32x4 qreg[2][DL];
        auto qload = [&](int buf, int64_t kt) {
            const uint32_t k2 = (uint32_t)(kcol(kt) * 2);
#pragma unroll
            for (int q = 0; q < DL; ++q)
                qreg[buf][q] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(qrs, (int)(qv0 + k2 + (uint32_t)(q * RR * g.ldq * 2)), 0, 0));
        };
        auto qwrite = [&](int buf, int64_t kt) {
            uint16_t* st = qst + (int)(kt % SQ) * QE + trow * BK + lslot * 8;
#pragma unroll
            for (int q = 0; q < DL; ++q) *(u32x4*)(st + q * RR * BK) = qreg[buf][q];
        };
        const int frow = lane & 31, fhalf = lane >> 5;
        const int fs = CF::swz(lane & 15);
        bf16x8 fa[2][TM], fb[2][TN];
        auto frag = [&](int buf, int kk, int64_t kt) {
            const uint16_t* cp = pst + (int)(kt % SP) * PE + (wr * WM + frow) * BK;
            const uint16_t* cq = qst + (int)(kt % SQ) * QE + (wc * WN + frow) * BK;
            const int slot = ((2 * kk + fhalf) ^ fs) * 8;
#pragma unroll
            for (int t = 0; t < TM; ++t) fa[buf][t] = __builtin_bit_cast(bf16x8, *(const u32x4*)&cp[t * 32 * BK + slot]);
#pragma unroll
            for (int t = 0; t < TN; ++t) fb[buf][t] = __builtin_bit_cast(bf16x8, *(const u32x4*)&cq[t * 32 * BK + slot]);
        };
        // Inside step kt (at its third sub-step): Q of step kt + 1 into its
        // LDS stage, free since the barrier that ended step kt - 1 (the
        // loads, issued two steps earlier, are complete when at most this
        // step's 2 DL loads are younger; that also covers the P DMA of step
        // kt + 1).  The end of step kt: every wave's LDS writes complete,
        // then the barrier.
        auto q_to_lds = [&](int buf, int64_t kt) {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * DL));
            qwrite(buf, kt + 1);
        };
        auto step_end = [&]() {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * DL) & ~0x0F00);  // and lgkmcnt(0)
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };
        auto mfma = [&](int buf, int a, int b) {
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][a], fb[buf][b], acc[a][b], 0, 0, 0);
        };
        // step kt computes from Q buffer parity qb = kt % 2 (the registers
        // of Q(kt + 1) are in buffer qb ^ 1, those of Q(kt + 2) go to qb)
        auto step = [&](int64_t kt, int qb) {
            __builtin_amdgcn_sched_barrier(0);
            pstage(kt + 2);    // into the P stage consumed at step kt - 1
            qload(qb, kt + 2);  // Q(kt) left these registers at the end of step kt - 1
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kk = 0; kk < BK / 16; ++kk) {
                if (kk == VE_QWRITE_SUBSTEP) q_to_lds(qb ^ 1, kt);
                if (kk + 1 < BK / 16) frag((kk + 1) & 1, kk + 1, kt);
                if (kk + 1 == BK / 16) {
                    constexpr int post = TM + TN, pre = TM * TN - post;
                    static_assert(pre >= 1, "early-barrier shape");
#pragma unroll
                    for (int i = 0; i < pre; ++i) mfma(kk & 1, i / TN, i % TN);
                    __builtin_amdgcn_sched_group_barrier(kSchedMfma, pre, 0);
                    step_end();
                    frag(0, 0, kt + 1);
#pragma unroll
                    for (int i = pre; i < TM * TN; ++i) mfma(kk & 1, i / TN, i % TN);
#pragma unroll
                    for (int i = 0; i < post; ++i) {
                        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                    }
                    continue;
                }
#pragma unroll
                for (int a = 0; a < TM; ++a)
#pragma unroll
                    for (int b = 0; b < TN; ++b) mfma(kk & 1, a, b);
#pragma unroll
                for (int i = 0; i < TM + TN; ++i) {
                    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
                }
                constexpr int kRest = TM * TN - (TM + TN);
                if constexpr (kRest > 0) __builtin_amdgcn_sched_group_barrier(kSchedMfma, kRest, 0);
            }
        };
        // prologue: Q(0), Q(1) into registers, P(0), P(1) by DMA; Q(0) to
        // LDS; P(0) complete (only P(1) younger)
        qload(0, 0);
        qload(1, 1);
        pstage(0);
        pstage(1);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * DL));
        qwrite(0, 0);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(DL) & ~0x0F00);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        frag(0, 0, 0);
        int64_t kt = 0;
        for (; kt + 1 < nk; kt += 2) {
            step(kt, 0);
            step(kt + 1, 1);
        }
        if (kt < nk) step(kt, 0);
        __builtin_amdgcn_s_waitcnt(0);  // loads past the last step land before LDS is reused
    }
    __syncthreads();
    if (g.ksplit > 1) {
        // K slice of a split tile: the raw accumulators, summed later
        float* out = partial_at<CF>(g, (int)blockIdx.x) + (int64_t)wave * (TM * TN * 16 * 64) + lane;
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
            for (int b = 0; b < TN; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) out[((a * TN + b) * 16 + r) * 64] = acc[a][b][r];
        return;
    }
    dma_epilogue<CF, HAS_D, HAS_C, HAS_CT>(g, acc, ti, tj, smem);
}

// Sums of split tiles' K slices, in slice order, into each tile's first
// slice: workgroup b adds up 1024 consecutive floats of tile b / per_tile.
constexpr int kSumChunk = 1024;
__global__ void __launch_bounds__(256) k_split_sum(float* partial, int tile_floats, int ksplit) {
    const int per_tile = tile_floats / kSumChunk;
    const int tile = blockIdx.x / per_tile, chunk = blockIdx.x % per_tile;
    float* base = partial + (int64_t)tile * ksplit * tile_floats + chunk * kSumChunk + threadIdx.x * 4;
    f32x4 acc = *(const f32x4*)base;
    for (int sp = 1; sp < ksplit; ++sp) {
        const f32x4 v = *(const f32x4*)(base + (int64_t)sp * tile_floats);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    *(f32x4*)base = acc;
}

// A split tile's summed accumulators (its first slice), then the epilogue.
template <class CF, bool HAS_D, bool HAS_C, bool HAS_CT>
__global__ void __launch_bounds__(CF::THREADS) k_gemm_split_reduce(GemmArgs g) {
    constexpr int TM = CF::TM, TN = CF::TN;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[CF::SMEM];
    int ti, tj;
    tile_at(g, g.tile_base + (int)blockIdx.x, ti, tj);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    f32x16 acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
    const float* in = partial_at<CF>(g, (int)blockIdx.x * g.ksplit) + (int64_t)wave * (TM * TN * 16 * 64) + lane;
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = in[((a * TN + b) * 16 + r) * 64];
    dma_epilogue<CF, HAS_D, HAS_C, HAS_CT>(g, acc, ti, tj, smem);
}

// Epilogue of the direct-to-LDS kernels: in passes of 64 tile rows, the
// same three phases as the register-staged kernel.
template <class CF, bool HAS_D, bool HAS_C, bool HAS_CT>
__device__ __forceinline__ void dma_epilogue(const GemmArgs& g, f32x16 (&acc)[CF::TM][CF::TN], int ti, int tj,
                                             unsigned char* smem) {
    constexpr int BM = CF::BM, BN = CF::BN, WM = CF::WM, WN = CF::WN, TN = CF::TN;
    constexpr int NT = CF::THREADS, LDC = CF::LDC;
    const int64_t i0 = (int64_t)ti * BM, j0 = (int64_t)tj * BN;
    float* sC = (float*)smem;                         // [PASS_ROWS][LDC]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave / CF::WAVES_N, wc = wave % CF::WAVES_N;
    const bool mirror = g.symmetric && ti < tj;
    const bool transpose = HAS_CT || mirror;
    uint16_t* T = HAS_CT ? g.CT : g.C;
    const int64_t ldt = HAS_CT ? g.ldct : g.ldc;
    const bool vec_t = HAS_CT ? g.vec_ct : g.vec_c;
    const int64_t ncols = min((int64_t)BN, g.N - j0);
    constexpr int PR = CF::PASS_ROWS;
#pragma unroll
    for (int pass = 0; pass < BM / PR; ++pass) {   // unrolled: accumulator indices stay compile-time
        const int64_t r0 = i0 + (int64_t)pass * PR;
        const int64_t mrows = min((int64_t)PR, g.M - r0);
        if (wr == pass / (WM / PR)) {
            constexpr int per = PR / 32;
            const int a0 = (pass % (WM / PR)) * per;
#pragma unroll
            for (int aa = 0; aa < per; ++aa)
#pragma unroll
                for (int b = 0; b < TN; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = aa * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                        const int col = wc * WN + b * 32 + (lane & 31);
                        sC[row * LDC + col] = acc[a0 + aa][b][r];
                    }
        }
        __syncthreads();
        if (mrows > 0) {
#pragma unroll 2
            for (int q = 0; q < (PR * BN / 8) / NT; ++q) {
                const int id = tid + NT * q;
                const int row = id / (BN / 8), c8 = (id % (BN / 8)) * 8;
                if (row >= mrows || c8 >= ncols) continue;
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = g.alpha * sC[row * LDC + c8 + e];
                const int64_t i = r0 + row, j = j0 + c8;
                const bool full = c8 + 8 <= ncols;
                if (HAS_D) {
                    if (full && g.vec_d) {
                        const u32x4 d = *(const VE_GLOBAL u32x4*)(g.D + i * g.ldd + j);
                        const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            v[e] = __builtin_fmaf(g.beta, (e & 1) ? bf_hi(dw[e >> 1]) : bf_lo(dw[e >> 1]), v[e]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (c8 + e < ncols) v[e] = __builtin_fmaf(g.beta, from_bf16(g.D[i * g.ldd + j + e]), v[e]);
                    }
                }
                const u32x4 h = pack8(v);
                const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
                if (HAS_C) {
                    if (full && g.vec_c) {
                        *(VE_GLOBAL u32x4*)(g.C + i * g.ldc + j) = h;
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (c8 + e < ncols) g.C[i * g.ldc + j + e] = (uint16_t)(hw[e >> 1] >> (16 * (e & 1)));
                    }
                }
                if (transpose) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        sC[row * LDC + c8 + e] = (e & 1) ? bf_hi(hw[e >> 1]) : bf_lo(hw[e >> 1]);
                }
            }
            if (transpose) {
                __syncthreads();
#pragma unroll 2
                for (int q = 0; q < (PR * BN / 8) / NT; ++q) {
                    const int id = tid + NT * q;
                    const int col = id % BN, r8 = (id / BN) * 8;
                    if (col >= ncols || r8 >= mrows) continue;
                    float v[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = sC[(r8 + e) * LDC + col];
                    const u32x4 h = pack8(v);
                    const int64_t j = j0 + col, i = r0 + r8;
                    if (r8 + 8 <= mrows && vec_t) {
                        *(VE_GLOBAL u32x4*)(T + j * ldt + i) = h;
                    } else {
                        const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (r8 + e < mrows) T[j * ldt + i + e] = (uint16_t)(hw[e >> 1] >> (16 * (e & 1)));
                    }
                }
            }
        }
        __syncthreads();
    }
}

// Partial sums of squares of n bf16 values, in fp64, one per workgroup.
// Per-workgroup partial sums of squares in fp64, in a fixed order (the same
// grid every call).  Aligned inputs stream as 16-byte vectors (eight bf16),
// four in flight per thread.
__device__ __forceinline__ double sumsq8(double s, u32x4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const double lo = (double)__uint_as_float(w[i] << 16), hi = (double)__uint_as_float(w[i] & 0xffff0000u);
        s = __builtin_fma(lo, lo, s);
        s = __builtin_fma(hi, hi, s);
    }
    return s;
}

__global__ void __launch_bounds__(256) k_sumsq(const uint16_t* x, int64_t n, double* partial) {
    double s = 0.0;
    const int64_t stride = (int64_t)gridDim.x * 256, t0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    int64_t tail0 = 0;
    if (((uintptr_t)x & 15) == 0) {
        const u32x4* xv = (const u32x4*)x;
        const int64_t nv = n / 8;
        int64_t i = t0;
        for (; i + 3 * stride < nv; i += 4 * stride) {
            const u32x4 a = __builtin_nontemporal_load(xv + i), b = __builtin_nontemporal_load(xv + i + stride);
            const u32x4 c = __builtin_nontemporal_load(xv + i + 2 * stride);
            const u32x4 d = __builtin_nontemporal_load(xv + i + 3 * stride);
            s = sumsq8(sumsq8(sumsq8(sumsq8(s, a), b), c), d);
        }
        for (; i < nv; i += stride) s = sumsq8(s, __builtin_nontemporal_load(xv + i));
        tail0 = nv * 8;
    }
    for (int64_t i = tail0 + t0; i < n; i += stride) {
        const double v = (double)from_bf16(x[i]);
        s = __builtin_fma(v, v, s);
    }
    __shared__ double red[256];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) partial[blockIdx.x] = red[0];
}

// s = fp32(1 / (sqrt(sum of the partials) + eps)), one workgroup.
__global__ void __launch_bounds__(256) k_norm_scale(const double* partial, int nparts, float eps, float* scale) {
    __shared__ double red[256];
    double s = 0.0;
    for (int i = threadIdx.x; i < nparts; i += 256) s += partial[i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) *scale = (float)(1.0 / (__builtin_sqrt(red[0]) + (double)eps));
}

// X0 = bf16(fp32(G * s)), written straight (rows x cols, to `straight`) and/or
// transposed (cols x rows, to `transposed`).  64 x 64 tiles through LDS so
// both writes are coalesced.
__global__ void __launch_bounds__(256) k_normalize(const uint16_t* G, int64_t rows, int64_t cols, const float* scale_p,
                                                   uint16_t* straight, uint16_t* transposed, int tiles_c) {
    __shared__ uint16_t tileT[64][66];
    const float scale = *scale_p;
    const int64_t r0 = (int64_t)(blockIdx.x / tiles_c) * 64, c0 = (int64_t)(blockIdx.x % tiles_c) * 64;
    const int tc = threadIdx.x & 63, tr = threadIdx.x >> 6;
    for (int rr = tr; rr < 64; rr += 4) {
        const int64_t r = r0 + rr, c = c0 + tc;
        uint16_t h = 0;
        if (r < rows && c < cols) {
            h = to_bf16(from_bf16(G[r * cols + c]) * scale);
            if (straight) straight[r * cols + c] = h;
        }
        tileT[tc][rr] = h;
    }
    if (!transposed) return;
    __syncthreads();
    for (int cc = tr; cc < 64; cc += 4) {
        const int64_t c = c0 + cc, r = r0 + tc;
        if (c < cols && r < rows) transposed[c * rows + r] = tileT[cc][tc];
    }
}

// The same with 16-byte accesses, when rows and cols are multiples of 8 and
// every pointer is 16-byte aligned: a thread scales 8 consecutive elements of
// a row (one vector load, one vector store straight), and writes 8
// consecutive elements of a transposed row gathered from the LDS tile.
__global__ void __launch_bounds__(256) k_normalize_v(const uint16_t* G, int64_t rows, int64_t cols,
                                                     const float* scale_p, uint16_t* straight, uint16_t* transposed,
                                                     int tiles_c) {
    __shared__ uint32_t tile[64][33];  // 64 rows of 64 bf16 (pairs), padded against bank conflicts
    const float scale = *scale_p;
    const int64_t r0 = (int64_t)(blockIdx.x / tiles_c) * 64, c0 = (int64_t)(blockIdx.x % tiles_c) * 64;
    const int t = threadIdx.x, cc = (t & 7) * 8;
    for (int rr = t >> 3; rr < 64; rr += 32) {
        const int64_t r = r0 + rr, c = c0 + cc;
        u32x4 h = u32x4{0, 0, 0, 0};
        if (r < rows && c < cols) {
            const u32x4 v = __builtin_nontemporal_load((const u32x4*)(G + r * cols + c));
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            uint32_t o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                o[i] = pack_bf16x2(__uint_as_float(w[i] << 16) * scale, __uint_as_float(w[i] & 0xffff0000u) * scale);
            h = u32x4{o[0], o[1], o[2], o[3]};
            if (straight) *(u32x4*)(straight + r * cols + c) = h;
        }
        tile[rr][cc / 2 + 0] = h.x;
        tile[rr][cc / 2 + 1] = h.y;
        tile[rr][cc / 2 + 2] = h.z;
        tile[rr][cc / 2 + 3] = h.w;
    }
    if (!transposed) return;
    __syncthreads();
    const int orr = (t & 7) * 8;  // tile rows gathered: transposed columns r0 + orr ..
    for (int oc = t >> 3; oc < 64; oc += 32) {
        const int64_t c = c0 + oc, r = r0 + orr;
        if (c >= cols || r >= rows) continue;
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t a = tile[orr + 2 * i][oc >> 1], b = tile[orr + 2 * i + 1][oc >> 1];
            const uint32_t ha = (oc & 1) ? a >> 16 : a & 0xffffu, hb = (oc & 1) ? b >> 16 : b & 0xffffu;
            o[i] = ha | (hb << 16);
        }
        *(u32x4*)(transposed + c * rows + r) = u32x4{o[0], o[1], o[2], o[3]};
    }
}

// workgroups of a launch: every tile, or the upper triangle of a symmetric product
int64_t launch_tiles(const GemmArgs& g, int bm) {
    const int64_t tm = (g.M + bm - 1) / bm;
    return g.symmetric ? (int64_t)g.tiles_n * (g.tiles_n + 1) / 2 : tm * g.tiles_n;
}

template <class CF, bool HAS_D, bool HAS_C, bool HAS_CT>
hipError_t launch_gemm_t(GemmArgs g, hipStream_t s) {
    const int64_t tiles = launch_tiles(g, CF::BM);
    g.tiles_total = (int32_t)tiles;
    g.tile_base = 0;
    g.ksplit = 1;
    if (g.vec_p && g.vec_q && g.K % 8 == 0)
        hipLaunchKernelGGL((k_gemm_nt<CF, HAS_D, HAS_C, HAS_CT, true>), dim3((unsigned)tiles), dim3(CF::THREADS), 0, s, g);
    else
        hipLaunchKernelGGL((k_gemm_nt<CF, HAS_D, HAS_C, HAS_CT, false>), dim3((unsigned)tiles), dim3(CF::THREADS), 0, s,
                           g);
    return hipGetLastError();
}

// Tail split: when the tiles fill some whole rounds of the CUs plus a short
// last round (at most a quarter of the CUs), or fewer tiles than CUs in all,
// the last round's tiles are cut along K into slices that fill one round
// (each slice writes fp32 accumulators), and a reduce launch sums the slices
// in order and runs the epilogue.  Only over long contractions (at least 8
// steps per slice).  Returns the slice count (1: no split) and the number of
// tiles launched whole.  The option gemm_split = 0 turns it off.
inline int tail_split(int64_t tiles, int64_t nk, bool has_partial, int64_t& full, int per_cu = 1) {
    full = tiles;
    if (!has_partial || option(kOptGemmSplit) == 0 || nk < 16) return 1;
    const int64_t slots = (int64_t)kCUs * per_cu;  // workgroups resident at once
    const int64_t whole = tiles / slots * slots, tail = tiles - whole;
    if (tail == 0 || (whole > 0 && tail * 4 > slots)) return 1;
    const int64_t ks = std::min<int64_t>(std::min<int64_t>(slots / tail, nk / 8), 32);
    if (ks < 2) return 1;
    full = whole;
    return (int)ks;
}

template <class CF, bool HAS_D, bool HAS_C, bool HAS_CT>
hipError_t launch_dma_t(GemmArgs g, hipStream_t s) {
    const int64_t tiles = launch_tiles(g, CF::BM);
    g.tiles_total = (int32_t)tiles;
    g.tile_base = 0;
    g.ksplit = 1;
    int64_t full = tiles;
    const int ks = tail_split(tiles, g.K / CF::BK, g.partial != nullptr, full, CF::PER_CU);
    if (ks <= 1) {
        hipLaunchKernelGGL((k_gemm_nt_dma<CF, HAS_D, HAS_C, HAS_CT>), dim3((unsigned)tiles), dim3(CF::THREADS), 0, s,
                           g);
        return hipGetLastError();
    }
    const int64_t tail = tiles - full;
    static_assert(int64_t(CF::BM) * CF::BN * 4 * kCUs * CF::PER_CU <= kSplitPartialBytes, "split scratch");
    if (full > 0)  // whole rounds first (none when the product is split whole)
        hipLaunchKernelGGL((k_gemm_nt_dma<CF, HAS_D, HAS_C, HAS_CT>), dim3((unsigned)full), dim3(CF::THREADS), 0, s,
                           g);
    GemmArgs t = g;
    t.tile_base = (int32_t)full;
    t.ksplit = ks;
    hipLaunchKernelGGL((k_gemm_nt_dma<CF, HAS_D, HAS_C, HAS_CT>), dim3((unsigned)(tail * ks)), dim3(CF::THREADS), 0,
                       s, t);
    constexpr int kTileFloats = CF::BM * CF::BN;
    static_assert(kTileFloats % kSumChunk == 0 && kSumChunk == 256 * 4, "slice sum shape");
    hipLaunchKernelGGL(k_split_sum, dim3((unsigned)(tail * (kTileFloats / kSumChunk))), dim3(256), 0, s, g.partial,
                       kTileFloats, ks);
    hipLaunchKernelGGL((k_gemm_split_reduce<CF, HAS_D, HAS_C, HAS_CT>), dim3((unsigned)tail), dim3(CF::THREADS), 0,
                       s, t);
    return hipGetLastError();
}

template <class CF>
hipError_t launch_gemm_dma(GemmArgs g, hipStream_t s) {
    g.tiles_n = (int)((g.N + CF::BN - 1) / CF::BN);
    const bool d = g.D != nullptr, c = g.C != nullptr, ct = g.CT != nullptr;
    if (d && c && ct) return launch_dma_t<CF, true, true, true>(g, s);
    if (d && c) return launch_dma_t<CF, true, true, false>(g, s);
    if (d && ct) return launch_dma_t<CF, true, false, true>(g, s);
    if (c && ct) return launch_dma_t<CF, false, true, true>(g, s);
    if (c) return launch_dma_t<CF, false, true, false>(g, s);
    if (ct) return launch_dma_t<CF, false, false, true>(g, s);
    return hipErrorInvalidValue;
}

template <class CF>
bool dma_ok(const GemmArgs& g) {
    // QST: a tile's P and Q rows are addressed with 32-bit byte offsets
    return g.vec_p && g.vec_q && g.K % CF::BK == 0 &&
           (!CF::QST || std::max(g.ldp, g.ldq) * 2 * CF::BM < (int64_t(1) << 31));
}

template <class CF>
hipError_t launch_gemm_cfg(GemmArgs g, hipStream_t s) {
    g.tiles_n = (int)((g.N + CF::BN - 1) / CF::BN);
    const bool d = g.D != nullptr, c = g.C != nullptr, ct = g.CT != nullptr;
    if (d && c && ct) return launch_gemm_t<CF, true, true, true>(g, s);
    if (d && c) return launch_gemm_t<CF, true, true, false>(g, s);
    if (d && ct) return launch_gemm_t<CF, true, false, true>(g, s);
    if (c && ct) return launch_gemm_t<CF, false, true, true>(g, s);
    if (c) return launch_gemm_t<CF, false, true, false>(g, s);
    if (ct) return launch_gemm_t<CF, false, false, true>(g, s);
    return hipErrorInvalidValue;
}

// The option gemm_cfg pins one configuration for tuning; otherwise large
// tiles are used when they still give every CU several tiles.
int gemm_cfg_override() { return (int)option(kOptGemmCfg); }

// The direct-to-LDS kernel with 8 waves of 128 x 64 where it applies (K a
// multiple of 64, 16-byte operand rows) and the product has at least two
// rounds of 256 x 256 tiles; else the register-staged 256 x 256 or 128 x 128
// kernel by the same rule.
// 256 x 256 tiles on the direct-to-LDS kernel from two rounds of them on;
// below that, the configuration with the smaller modelled time: rounds of
// work items times their K steps, a 128 x 128 step costing 0.45 of a
// 256 x 256 one (a quarter of the work at 56% of the rate, measured), split
// slices adding their fp32 traffic (about 0.05 of a step each).  Before
// that model, symmetric products with K >= 4096 and at most one round of
// 128 x 128 tiles take configuration 14.
int gemm_cfg_auto(const GemmArgs& g) {
    const int64_t tm = (g.M + 255) / 256, tn = (g.N + 255) / 256;
    const int64_t active = g.symmetric ? tm * (tm + 1) / 2 : tm * tn;
    const bool dma = g.vec_p && g.vec_q && g.K % 64 == 0;
    if (!dma) return active >= 2 * kCUs ? 2 : 0;
    // the staged-Q form where its 32-bit row offsets reach, else the plain one
    const int big = dma_ok<DmaCfg<128, 64, 64, 3, true>>(g) ? 13 : 9;
    if (active >= 2 * kCUs) return big;
    // A symmetric product with a long contraction (K >= 4096, X X^T) whose
    // 128 x 128 tiles fit in one round of the two-per-CU configuration 14
    // (then split along K over those slots).  Measured, Newton-Schulz per
    // call, interleaved on one box: 2048 x 7168 0.86 ms against 0.90,
    // 1024 x 8192 0.445 against 0.49.  Not for A A at those sizes (K = m:
    // slices of ~11 steps do not pay for their sums: 0.90 and 0.48 ms with
    // it), nor beyond one round (5760 x 5760, 1,035 such tiles: 4.47
    // against 4.20 ms).
    using C14 = DmaCfg<128, 64, 64, 2, false, 128, 128>;
    if (g.symmetric && g.K >= 4096) {
        const int64_t s = (g.M + C14::BM - 1) / C14::BM;
        if (s * (s + 1) / 2 <= (int64_t)kCUs * C14::PER_CU && dma_ok<C14>(g)) return 14;
    }
    const int64_t nk = g.K / 64;
    auto rounds = [](int64_t items) { return (double)((items + kCUs - 1) / kCUs); };
    int64_t full = active;
    const int ks = tail_split(active, nk, g.partial != nullptr, full);
    const int64_t sliced = (active - full) * ks;
    double t9 = rounds(full) * (double)nk;
    if (sliced > 0) t9 += rounds(sliced) * (double)((nk + ks - 1) / ks) + 0.05 * (double)sliced;
    const int64_t sm = (g.M + 127) / 128, sn = (g.N + 127) / 128;
    const int64_t tiles0 = g.symmetric ? sm * (sm + 1) / 2 : sm * sn;
    const double t0 = rounds(tiles0) * (double)nk * 0.45;
    return t9 <= t0 ? big : 0;
}

}  // namespace

int64_t gemm_tiles(int64_t M, int64_t N) { return ((M + 127) / 128) * ((N + 127) / 128); }
int norm_blocks() { return kNormBlocks; }

hipError_t launch_gemm_nt(GemmArgs g, hipStream_t s) {
    g.xcd_remap = option(kOptGemmXcd) != 0;
    g.sym_blocked = g.xcd_remap;
    const int cfg = gemm_cfg_override();
    switch (cfg >= 0 ? cfg : gemm_cfg_auto(g)) {
#define VE_GEMM_CASE(ID, BM, BN, BK, WM, WN) \
        case ID: return launch_gemm_cfg<Cfg<BM, BN, BK, WM, WN>>(g, s);
        VE_GEMM_CFGS(VE_GEMM_CASE)
#undef VE_GEMM_CASE
#define VE_DMA_CASE(ID, WM, WN, BK, ST, QS, BM, BN)                                                   \
        case ID:                                                                                        \
            return dma_ok<DmaCfg<WM, WN, BK, ST, QS, BM, BN>>(g)                                        \
                       ? launch_gemm_dma<DmaCfg<WM, WN, BK, ST, QS, BM, BN>>(g, s)                      \
                       : (BM == 256 ? launch_gemm_cfg<Cfg<256, 256, 64, 128, 64>>(g, s)                 \
                                    : launch_gemm_cfg<Cfg<128, 128, 64, 64, 64>>(g, s));
        VE_DMA_CFGS(VE_DMA_CASE)
#undef VE_DMA_CASE
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_sumsq(const uint16_t* x, int64_t n, double* partial, hipStream_t s) {
    hipLaunchKernelGGL(k_sumsq, dim3(kNormBlocks), dim3(256), 0, s, x, n, partial);
    return hipGetLastError();
}

hipError_t launch_norm_scale(const double* partial, float eps, float* scale, hipStream_t s) {
    hipLaunchKernelGGL(k_norm_scale, dim3(1), dim3(256), 0, s, partial, kNormBlocks, eps, scale);
    return hipGetLastError();
}

hipError_t launch_normalize(const uint16_t* G, int64_t rows, int64_t cols, const float* scale, uint16_t* straight,
                            uint16_t* transposed, hipStream_t s) {
    const int tiles_c = (int)((cols + 63) / 64);
    const int64_t tiles = ((rows + 63) / 64) * tiles_c;
    auto a16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
    if (rows % 8 == 0 && cols % 8 == 0 && a16(G) && a16(straight) && a16(transposed))
        hipLaunchKernelGGL(k_normalize_v, dim3((unsigned)tiles), dim3(256), 0, s, G, rows, cols, scale, straight,
                           transposed, tiles_c);
    else
        hipLaunchKernelGGL(k_normalize, dim3((unsigned)tiles), dim3(256), 0, s, G, rows, cols, scale, straight,
                           transposed, tiles_c);
    return hipGetLastError();
}

}  // namespace ve
