// ve_kernels.hip -- gfx950 kernels of the RaggedShard shard step.
//
// Per element the step streams 18 bytes through HBM (bf16 gradient read and
// copy-in write, fp32 master read+write, two int8 codes read+write, bf16
// parameter write) and does ~40 VALU operations, so it is bandwidth-bound;
// nothing here is a dense contraction and no MFMA is used.
//
// The one non-local step is the block absmax: every quantisation block's new
// codes need the maximum of its *fresh* moments (veScale-FSDP talk notes,
// "1. RaggedShard": one scale per block, and a block never straddles ranks,
// so the reduction never leaves the GPU).  To keep the HBM traffic at the
// algorithmic 18 B/element, a block's inputs (bf16 gradient + both int8
// codes = exactly one dword per element) stay in VGPRs across the reduction
// and the moments are recomputed from them afterwards:
//
//   phase 1  load inputs (+ master), compute moments, update master, write
//            master / bf16 param / gradient copy, running absmax;
//   reduce   DPP / ds_swizzle inside a wave, LDS across waves;
//   phase 2  recompute the moments from the registers, quantise with the new
//            scale, write the codes.
//
// Row blocks of 16K to 49K elements run a persistent form of the wg class
// (k_step_dyn): one workgroup per CU takes blocks from a ticket counter and
// stages the next block's gradient and codes in LDS during its own phase 2.
// Whole-row blocks of 8K or 16K elements take the same loop in items of
// four or two consecutive blocks (k_step_rows), each block keeping its own
// absmax and scales.  The host uses both only where a launch has enough
// blocks per CU to repay their fixed cost.
//
// Block-size classes (decided per rank segment at plan load):
//   small  <= 64 chunks of kSmallChunk (4) elements: a group of G (power of
//          two) lanes of one wave owns a block, one chunk per lane, 64/G
//          blocks per wave (16- and 128-element blocks of ragged buckets);
//   unit   one-element blocks, kSmallChunk blocks per lane (norms, ragged
//          buckets' 1-row vectors);
//   wg     one workgroup owns a block; lanes own 4-element groups so that
//          every wave-wide access is one contiguous span (1 KB of fp32
//          master, 512 B of bf16, 256 B of codes), GPT groups per thread
//          held in VGPRs (row blocks of 8K..46K elements, 128x128 tiles);
//   huge   one workgroup, two passes (inputs re-read) for blocks too large to
//          hold on chip.
// Runs (copy-in, padding zero-fill) are plain tiled copies.
//
// Floating point: fp32 with fused multiply-adds, hardware sqrt/reciprocal
// (about 1 ulp) in the weight update, correctly rounded 127/amax per block,
// round-half-even for codes and bf16.  The moment formulas are written once
// (moments()) and the compiler is kept from contracting differently, so the
// recomputed moments equal the ones whose maximum was taken.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ve_device.h"
#include "ve_internal.h"

namespace ve {
namespace {

// ---------------------------------------------------------------------------
// scalar helpers
__device__ __forceinline__ float code_at(uint32_t w, int b) {
    return (float)((int32_t)(w << (24 - 8 * b)) >> 24);  // sign-extended byte b
}

// Keep the compiler from proving a value equal to an earlier one (forces the
// moments to be recomputed from registers instead of kept alive).
__device__ __forceinline__ void opaque(uint32_t& x) { asm volatile("" : "+v"(x)); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xb1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4e;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

__device__ __forceinline__ float swz_xor16(float v) {
    // ds_swizzle bit-mask mode: and 0x1f, or 0, xor 0x10 (within 32 lanes)
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401f));
}

// Maximum over aligned groups of G lanes (G a power of two <= 64, wave-
// uniform); every lane of a group receives the group maximum.  Values are
// non-negative.
__device__ __forceinline__ float group_max(float v, int G) {
    if (G > 1) v = fmaxf(v, dpp<kQuadXor1>(v));
    if (G > 2) v = fmaxf(v, dpp<kQuadXor2>(v));
    if (G > 4) v = fmaxf(v, dpp<kRowHalfMirror>(v));  // lane i <-> 7-i: the other quad
    if (G > 8) v = fmaxf(v, dpp<kRowMirror>(v));      // lane i <-> 15-i: the other half-row
    if (G > 16) v = fmaxf(v, swz_xor16(v));
    if (G > 32) v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

// Wave maximum, returned as a wave-uniform value.
// Workgroup barrier for LDS traffic only: waits for this wave's LDS (and
// scalar) accesses, not for its outstanding global loads and stores.  A
// __syncthreads also drains those, which would expose the write latency of a
// block's phase-1 stores, and any loads already issued for the next block,
// at every reduction.  The memory clobbers keep the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ float wave_max(float v) {
    v = group_max(v, 32);
    const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    return fmaxf(lo, hi);
}

// ---------------------------------------------------------------------------
// global-memory access (vector types and ldv/stv in ve_device.h)

// Every byte is touched once; where a wave-wide access covers whole cache
// lines (lane-contiguous layouts) it carries a non-temporal (streaming) hint.
// Where lanes are strided (16-element chunks), partial lines are merged in
// the L2 across accesses, which the hint would defeat, so those stay plain.
template <int CH>
constexpr bool kStream = VE_NONTEMPORAL && CH == kWgChunk;

// Wave-uniform reads of device memory the reading workgroup alone may later
// change (the gradient pointer table, a block's old scales) go through the
// constant address space, i.e. scalar loads.
#define VE_CONST __attribute__((address_space(4)))
template <class T>
__device__ __forceinline__ T sload(const T* p) {
    return *(const VE_CONST T*)p;
}

struct Ptrs {
    const VE_GLOBAL uint16_t* __restrict__ grad;
    VE_GLOBAL uint16_t* __restrict__ grad_shard;
    VE_GLOBAL float* __restrict__ master;
    VE_GLOBAL int8_t* __restrict__ m_q;
    VE_GLOBAL int8_t* __restrict__ v_q;
    VE_GLOBAL uint16_t* __restrict__ param;
    bool aligned;  // every base pointer 16-byte aligned
};

template <bool UNIFORM = false>
__device__ __forceinline__ Ptrs make_ptrs(const ve_shard_state& st, int tensor) {
    Ptrs p;
    const uint16_t* g = UNIFORM ? sload(st.grad_ptrs + tensor) : st.grad_ptrs[tensor];
    p.aligned = (((uintptr_t)g | (uintptr_t)st.grad_shard | (uintptr_t)st.master | (uintptr_t)st.m_q |
                  (uintptr_t)st.v_q | (uintptr_t)st.param_shard) & 15) == 0;
    p.grad = (const VE_GLOBAL uint16_t*)g;
    p.grad_shard = (VE_GLOBAL uint16_t*)st.grad_shard;
    p.master = (VE_GLOBAL float*)st.master;
    p.m_q = (VE_GLOBAL int8_t*)st.m_q;
    p.v_q = (VE_GLOBAL int8_t*)st.v_q;
    p.param = (VE_GLOBAL uint16_t*)st.param_shard;
    return p;
}

// ---------------------------------------------------------------------------
// block and chunk geometry
struct Geo {
    int64_t e0;      // tensor element of the block's first element
    int64_t stride;  // tensor elements between consecutive runs (rows of a tile)
    int32_t run;     // contiguous elements per run
    int32_t nruns;
    int32_t cpr;     // chunks per run
    int32_t nchunks;
    int64_t blk;     // rank-local block index (scale slot)
};

template <int CH>
__device__ __forceinline__ Geo block_geo(const Seg& sg, int64_t k) {
    Geo g;
    const int64_t q = k / sg.tiles;
    const int64_t j = k - q * sg.tiles;
    const int64_t r0 = (sg.panel0 + q) * sg.block_rows;
    const int64_t rows_in = min(sg.block_rows, sg.rows - r0);
    if (sg.tiles == 1) {  // whole-row blocks: one contiguous run
        g.e0 = r0 * sg.cols;
        g.run = (int32_t)(rows_in * sg.cols);
        g.nruns = 1;
        g.stride = 0;
    } else {              // a tile: rows_in runs of block_cols, row stride cols
        g.e0 = r0 * sg.cols + j * sg.block_cols;
        g.run = (int32_t)sg.block_cols;
        g.nruns = (int32_t)rows_in;
        g.stride = sg.cols;
    }
    g.cpr = (g.run + CH - 1) / CH;
    g.nchunks = g.nruns * g.cpr;
    g.blk = sg.block0 + k;
    return g;
}

struct ChunkPos {
    int64_t e;  // tensor element of the chunk's first element
    int64_t s;  // shard coordinate of the same element
    int32_t n;  // valid elements (1..CH), contiguous
};

template <int CH>
__device__ __forceinline__ ChunkPos chunk_pos(const Geo& g, int64_t shard_base, int ci) {
    int ri = 0, w = ci * CH;
    if (g.nruns != 1) {
        ri = ci / g.cpr;
        w = (ci - ri * g.cpr) * CH;
    }
    ChunkPos c;
    c.e = g.e0 + (int64_t)ri * g.stride + w;
    c.s = shard_base + c.e;
    c.n = min(CH, g.run - w);
    return c;
}

// A chunk takes the vector path when it is full and every access is
// naturally aligned (CH codes, CH/4 16-byte master vectors, CH bf16 values).
template <int CH>
__device__ __forceinline__ bool vec_ok(const Ptrs& p, const ChunkPos& c) {
    constexpr int kGradAlign = CH >= 8 ? 8 : CH;  // elements: 16 B (CH 16) or 8 B (CH 4)
    return p.aligned && c.n == CH && (c.s & (CH - 1)) == 0 && (c.e & (kGradAlign - 1)) == 0;
}

// ---------------------------------------------------------------------------
// per-chunk data movement and arithmetic
template <int CH>
struct In {
    uint32_t g[CH / 2];  // CH bf16 gradients
    uint32_t m[CH / 4];  // CH first-moment codes
    uint32_t v[CH / 4];  // CH second-moment codes
};

// Both access paths produce plain values and the registers are assigned
// once afterwards (stores from two branches into one array would otherwise be
// merged into a store through a selected address, which demotes the array to
// scratch memory).
template <int CH>
__device__ __forceinline__ void load_in(In<CH>& x, const Ptrs& p, const ChunkPos& c, bool vec) {
    uint32_t gw[CH / 2], mw[CH / 4], vw[CH / 4];
    if (vec) {
        if constexpr (CH == 16) {
            const u32x4 g0 = ldv<kStream<CH>>((const VE_GLOBAL u32x4*)(p.grad + c.e));
            const u32x4 g1 = ldv<kStream<CH>>((const VE_GLOBAL u32x4*)(p.grad + c.e + 8));
            const u32x4 m = ldv<kStream<CH>>((const VE_GLOBAL u32x4*)(p.m_q + c.s));
            const u32x4 v = ldv<kStream<CH>>((const VE_GLOBAL u32x4*)(p.v_q + c.s));
            gw[0] = g0.x; gw[1] = g0.y; gw[2] = g0.z; gw[3] = g0.w;
            gw[4] = g1.x; gw[5] = g1.y; gw[6] = g1.z; gw[7] = g1.w;
            mw[0] = m.x; mw[1] = m.y; mw[2] = m.z; mw[3] = m.w;
            vw[0] = v.x; vw[1] = v.y; vw[2] = v.z; vw[3] = v.w;
        } else {
            static_assert(CH == 4, "chunks are 4 or 16 elements");
            const u32x2 g = ldv<kStream<CH>>((const VE_GLOBAL u32x2*)(p.grad + c.e));
            gw[0] = g.x;
            gw[1] = g.y;
            mw[0] = ldv<kStream<CH>>((const VE_GLOBAL uint32_t*)(p.m_q + c.s));
            vw[0] = ldv<kStream<CH>>((const VE_GLOBAL uint32_t*)(p.v_q + c.s));
        }
    } else {
#pragma unroll
        for (int i = 0; i < CH / 2; ++i) {
            const uint32_t lo = (2 * i < c.n) ? p.grad[c.e + 2 * i] : 0u;
            const uint32_t hi = (2 * i + 1 < c.n) ? p.grad[c.e + 2 * i + 1] : 0u;
            gw[i] = lo | (hi << 16);
        }
#pragma unroll
        for (int i = 0; i < CH / 4; ++i) {
            uint32_t a = 0, b = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (4 * i + k < c.n) {
                    a |= (uint32_t)(uint8_t)p.m_q[c.s + 4 * i + k] << (8 * k);
                    b |= (uint32_t)(uint8_t)p.v_q[c.s + 4 * i + k] << (8 * k);
                }
            }
            mw[i] = a;
            vw[i] = b;
        }
    }
#pragma unroll
    for (int i = 0; i < CH / 2; ++i) x.g[i] = gw[i];
#pragma unroll
    for (int i = 0; i < CH / 4; ++i) {
        x.m[i] = mw[i];
        x.v[i] = vw[i];
    }
}

template <int CH>
__device__ __forceinline__ void load_master(float (&mst)[CH], const Ptrs& p, const ChunkPos& c, bool vec) {
    f32x4 f[CH / 4];
    if (vec) {
        const VE_GLOBAL f32x4* mp = (const VE_GLOBAL f32x4*)(p.master + c.s);
#pragma unroll
        for (int i = 0; i < CH / 4; ++i) f[i] = ldv<kStream<CH>>(mp + i);
    } else {
        float t[CH];
#pragma unroll
        for (int k = 0; k < CH; ++k) t[k] = (k < c.n) ? p.master[c.s + k] : 0.f;
#pragma unroll
        for (int i = 0; i < CH / 4; ++i) f[i] = f32x4{t[4 * i], t[4 * i + 1], t[4 * i + 2], t[4 * i + 3]};
    }
#pragma unroll
    for (int i = 0; i < CH / 4; ++i) {
        mst[4 * i] = f[i].x; mst[4 * i + 1] = f[i].y; mst[4 * i + 2] = f[i].z; mst[4 * i + 3] = f[i].w;
    }
}

// Adam moments from the dequantised stored moments (the one definition used
// by both phases).
__device__ __forceinline__ void moments(float g, float cm, float cv, float sm, float sv,
                                        const StepScalars& sc, float& m1, float& v1) {
    m1 = __builtin_fmaf(sc.beta1, cm * sm, sc.omb1 * g);
    v1 = __builtin_fmaf(sc.beta2, cv * sv, sc.omb2 * (g * g));
}

template <int CH>
__device__ __forceinline__ float elem_g(const In<CH>& x, int i) {
    return (i & 1) ? bf_hi(x.g[i >> 1]) : bf_lo(x.g[i >> 1]);
}

// AdamW update of one chunk's master values from its held inputs; folds the
// fresh moments into the running absmax (nothing when act is false: an idle
// lane whose registers duplicate a valid chunk).
// The fresh moments are also left in km / kv (for a caller that keeps them
// in registers through the reduction instead of recomputing them).
template <int CH>
__device__ __forceinline__ void adam_update_k(const In<CH>& x, float (&mst)[CH], float sm, float sv,
                                              const StepScalars& sc, float& am, float& av, float (&km)[CH],
                                              float (&kv)[CH], bool act = true) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        float m1, v1;
        moments(elem_g(x, i), code_at(x.m[i >> 2], i & 3), code_at(x.v[i >> 2], i & 3), sm, sv, sc, m1, v1);
        km[i] = m1;
        kv[i] = v1;
        am = fmaxf(am, act ? fabsf(m1) : 0.f);
        av = fmaxf(av, act ? v1 : 0.f);
        const float d = __builtin_fmaf(__builtin_amdgcn_sqrtf(v1), sc.inv_sqrt_bc2, sc.eps);
        const float u = m1 * __builtin_amdgcn_rcpf(d);
        mst[i] = __builtin_fmaf(-sc.step_size, u, mst[i] * sc.decay);
    }
}

template <int CH>
__device__ __forceinline__ void adam_update(const In<CH>& x, float (&mst)[CH], float sm, float sv,
                                            const StepScalars& sc, float& am, float& av, bool act = true) {
    float km[CH], kv[CH];
    adam_update_k(x, mst, sm, sv, sc, am, av, km, kv, act);
}

// Phase 1 on one chunk: moments, AdamW update, writes of master, bf16 param
// and the gradient copy; folds the chunk into the running absmax.
template <int CH>
__device__ __forceinline__ void store_phase1(const In<CH>& x, const float (&mst)[CH], const Ptrs& p,
                                             const ChunkPos& c, bool vec) {
    uint32_t pb[CH / 2];
#pragma unroll
    for (int i = 0; i < CH / 2; ++i) pb[i] = pack_bf16x2(mst[2 * i], mst[2 * i + 1]);
    if (vec) {
        VE_GLOBAL f32x4* mp = (VE_GLOBAL f32x4*)(p.master + c.s);
#pragma unroll
        for (int i = 0; i < CH / 4; ++i) stv<kStream<CH>>(mp + i, f32x4{mst[4 * i], mst[4 * i + 1], mst[4 * i + 2], mst[4 * i + 3]});
        if constexpr (CH == 16) {
            VE_GLOBAL u32x4* pp = (VE_GLOBAL u32x4*)(p.param + c.s);
            stv<kStream<CH>>(pp, u32x4{pb[0], pb[1], pb[2], pb[3]});
            stv<kStream<CH>>(pp + 1, u32x4{pb[4], pb[5], pb[6], pb[7]});
            VE_GLOBAL u32x4* gp = (VE_GLOBAL u32x4*)(p.grad_shard + c.s);
            stv<kStream<CH>>(gp, u32x4{x.g[0], x.g[1], x.g[2], x.g[3]});
            stv<kStream<CH>>(gp + 1, u32x4{x.g[4], x.g[5], x.g[6], x.g[7]});
        } else {
            stv<kStream<CH>>((VE_GLOBAL u32x2*)(p.param + c.s), u32x2{pb[0], pb[1]});
            stv<kStream<CH>>((VE_GLOBAL u32x2*)(p.grad_shard + c.s), u32x2{x.g[0], x.g[1]});
        }
    } else {
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            if (k < c.n) {
                p.master[c.s + k] = mst[k];
                p.param[c.s + k] = (uint16_t)(pb[k >> 1] >> (16 * (k & 1)));
                p.grad_shard[c.s + k] = (uint16_t)(x.g[k >> 1] >> (16 * (k & 1)));
            }
        }
    }
}

template <int CH>
__device__ __forceinline__ void phase1(const In<CH>& x, float (&mst)[CH], const Ptrs& p, const ChunkPos& c,
                                       bool vec, float sm, float sv, const StepScalars& sc, float& am,
                                       float& av) {
    adam_update(x, mst, sm, sv, sc, am, av);
    store_phase1(x, mst, p, c, vec);
}

__device__ __forceinline__ uint32_t quant_byte(float x, float inv) {
    float q = __builtin_rintf(x * inv);
    q = __builtin_fminf(__builtin_fmaxf(q, -127.f), 127.f);
    return (uint32_t)((int32_t)q) & 0xffu;
}

// Codes of one chunk under the block's new scales, recomputed from the held
// inputs.
template <int CH>
__device__ __forceinline__ void quantise(const In<CH>& x, float sm, float sv, float im, float iv,
                                         const StepScalars& sc, uint32_t (&qm)[CH / 4], uint32_t (&qv)[CH / 4]) {
#pragma unroll
    for (int i = 0; i < CH / 4; ++i) qm[i] = qv[i] = 0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        float m1, v1;
        moments(elem_g(x, i), code_at(x.m[i >> 2], i & 3), code_at(x.v[i >> 2], i & 3), sm, sv, sc, m1, v1);
        qm[i >> 2] |= quant_byte(m1, im) << (8 * (i & 3));
        qv[i >> 2] |= quant_byte(v1, iv) << (8 * (i & 3));
    }
}

// Phase 2 on one chunk: recompute the moments from the held inputs and write
// their codes under the block's new scales.
template <int CH>
__device__ __forceinline__ void store_codes(const uint32_t (&qm)[CH / 4], const uint32_t (&qv)[CH / 4],
                                            const Ptrs& p, const ChunkPos& c, bool vec) {
    if (vec) {
        if constexpr (CH == 16) {
            stv<kStream<CH>>((VE_GLOBAL u32x4*)(p.m_q + c.s), u32x4{qm[0], qm[1], qm[2], qm[3]});
            stv<kStream<CH>>((VE_GLOBAL u32x4*)(p.v_q + c.s), u32x4{qv[0], qv[1], qv[2], qv[3]});
        } else {
            stv<kStream<CH>>((VE_GLOBAL uint32_t*)(p.m_q + c.s), qm[0]);
            stv<kStream<CH>>((VE_GLOBAL uint32_t*)(p.v_q + c.s), qv[0]);
        }
    } else {
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            if (k < c.n) {
                p.m_q[c.s + k] = (int8_t)(qm[k >> 2] >> (8 * (k & 3)));
                p.v_q[c.s + k] = (int8_t)(qv[k >> 2] >> (8 * (k & 3)));
            }
        }
    }
}

template <int CH>
__device__ __forceinline__ void phase2(const In<CH>& x, const Ptrs& p, const ChunkPos& c, bool vec, float sm,
                                       float sv, float im, float iv, const StepScalars& sc) {
    uint32_t qm[CH / 4], qv[CH / 4];
    quantise(x, sm, sv, im, iv, sc, qm, qv);
    store_codes<CH>(qm, qv, p, c, vec);
}

// ---------------------------------------------------------------------------
// Block-relative access for fully vectorised workgroup blocks.  Every
// stream is a raw buffer resource (wave-uniform base at the block's first
// element, range = the block's span) addressed by one 32-bit per-lane
// element offset per 4-element chunk; the same offset serves the tensor-side
// gradient and the shard-side arrays.  A lane without a chunk uses an offset
// beyond every range: the hardware's range check then returns zeros for its
// loads and drops its stores, so a block needs no branch at all (zero inputs
// give zero moments, which never raise the absmax).
struct FastRsrc {
    __amdgpu_buffer_rsrc_t grad;        // bf16, tensor element e0
    __amdgpu_buffer_rsrc_t grad_shard;  // bf16, shard element shard_base + e0 (same for the rest)
    __amdgpu_buffer_rsrc_t master;      // fp32
    __amdgpu_buffer_rsrc_t m_q;         // int8
    __amdgpu_buffer_rsrc_t v_q;         // int8
    __amdgpu_buffer_rsrc_t param;       // bf16
};
// Buffer resource word 3 for raw (unformatted, stride 0) buffers on gfx9-
// family targets; cache-policy bit 1 = non-temporal.
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kBufNT = VE_NONTEMPORAL ? 2 : 0;
// FAST blocks span fewer than 2^27 elements, so every byte offset inside a
// block, and every scalar slot offset (at most twice the span), is below
// 2^30.  A lane without a chunk takes the per-lane byte offset kNoChunkByte:
// past the end of every stream, with or without the scalar part added, and
// without wrapping 32 bits.
constexpr int64_t kFastMaxSpan = int64_t(1) << 27;
constexpr uint32_t kNoChunkByte = 1u << 31;

template <class T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const VE_GLOBAL T* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)base, (short)0, (int)(uint32_t)bytes,
                                             kRawBufferWord3);
}

typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Byte offsets of one chunk in the 1-, 2- and 4-byte streams: a per-lane
// part (v*) and a wave-uniform part (s*, the instruction's scalar offset).
struct ChunkAddr {
    uint32_t v1, v2, v4;
    uint32_t s1, s2, s4;
};

__device__ __forceinline__ void load_in_fast(In<4>& x, const FastRsrc& f, const ChunkAddr& a) {
    const i32x2 g = __builtin_amdgcn_raw_buffer_load_b64(f.grad, (int)a.v2, (int)a.s2, kBufNT);
    x.g[0] = (uint32_t)g.x;
    x.g[1] = (uint32_t)g.y;
    x.m[0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(f.m_q, (int)a.v1, (int)a.s1, kBufNT);
    x.v[0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(f.v_q, (int)a.v1, (int)a.s1, kBufNT);
}

__device__ __forceinline__ void load_master_fast(float (&mst)[4], const FastRsrc& f, const ChunkAddr& a) {
    const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(f.master, (int)a.v4, (int)a.s4, kBufNT);
    mst[0] = __int_as_float(v.x);
    mst[1] = __int_as_float(v.y);
    mst[2] = __int_as_float(v.z);
    mst[3] = __int_as_float(v.w);
}

// The gradient-slice copy is stored here, or in phase 2 when LATE.
__device__ __forceinline__ void store_grad_copy(const In<4>& x, const FastRsrc& f, const ChunkAddr& a) {
    __builtin_amdgcn_raw_buffer_store_b64(i32x2{(int32_t)x.g[0], (int32_t)x.g[1]}, f.grad_shard, (int)a.v2,
                                          (int)a.s2, kBufNT);
}

template <bool LATE>
__device__ __forceinline__ void phase1_fast_k(const In<4>& x, float (&mst)[4], const FastRsrc& f,
                                              const ChunkAddr& a, float sm, float sv, const StepScalars& sc,
                                              float& am, float& av, float (&km)[4], float (&kv)[4]) {
    adam_update_k(x, mst, sm, sv, sc, am, av, km, kv);
    const uint32_t p0 = pack_bf16x2(mst[0], mst[1]), p1 = pack_bf16x2(mst[2], mst[3]);
    const i32x4 mv = {__float_as_int(mst[0]), __float_as_int(mst[1]), __float_as_int(mst[2]), __float_as_int(mst[3])};
    __builtin_amdgcn_raw_buffer_store_b128(mv, f.master, (int)a.v4, (int)a.s4, kBufNT);
    __builtin_amdgcn_raw_buffer_store_b64(i32x2{(int32_t)p0, (int32_t)p1}, f.param, (int)a.v2, (int)a.s2, kBufNT);
    if constexpr (!LATE) store_grad_copy(x, f, a);
}

template <bool LATE>
__device__ __forceinline__ void phase1_fast(const In<4>& x, float (&mst)[4], const FastRsrc& f,
                                            const ChunkAddr& a, float sm, float sv, const StepScalars& sc,
                                            float& am, float& av) {
    float km[4], kv[4];
    phase1_fast_k<LATE>(x, mst, f, a, sm, sv, sc, am, av, km, kv);
}

// Phase 2 from moments kept in registers since phase 1.
template <bool LATE>
__device__ __forceinline__ void phase2_fast_kept(const In<4>& x, const float (&km)[4], const float (&kv)[4],
                                                 const FastRsrc& f, const ChunkAddr& a, float im, float iv) {
    if constexpr (LATE) store_grad_copy(x, f, a);
    uint32_t qm = 0, qv = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        qm |= quant_byte(km[i], im) << (8 * i);
        qv |= quant_byte(kv[i], iv) << (8 * i);
    }
    __builtin_amdgcn_raw_buffer_store_b32((int32_t)qm, f.m_q, (int)a.v1, (int)a.s1, kBufNT);
    __builtin_amdgcn_raw_buffer_store_b32((int32_t)qv, f.v_q, (int)a.v1, (int)a.s1, kBufNT);
}

template <bool LATE>
__device__ __forceinline__ void phase2_fast(const In<4>& x, const FastRsrc& f, const ChunkAddr& a, float sm,
                                            float sv, float im, float iv, const StepScalars& sc) {
    if constexpr (LATE) store_grad_copy(x, f, a);
    uint32_t qm[1], qv[1];
    quantise(x, sm, sv, im, iv, sc, qm, qv);
    __builtin_amdgcn_raw_buffer_store_b32((int32_t)qm[0], f.m_q, (int)a.v1, (int)a.s1, kBufNT);
    __builtin_amdgcn_raw_buffer_store_b32((int32_t)qv[0], f.v_q, (int)a.v1, (int)a.s1, kBufNT);
}

template <int CH>
__device__ __forceinline__ void make_opaque(In<CH>& x) {
#pragma unroll
    for (int i = 0; i < CH / 2; ++i) opaque(x.g[i]);
#pragma unroll
    for (int i = 0; i < CH / 4; ++i) {
        opaque(x.m[i]);
        opaque(x.v[i]);
    }
}

// ---------------------------------------------------------------------------
// work lookup: which segment holds work item w (a block, or a wave of small
// blocks), and the item's offset inside that segment.  w is wave-uniform, so
// every load here is a scalar (or read-first-lane) load.

// Workgroup paths: the slice of segments handled by this launch is in the
// kernel arguments.
__device__ __forceinline__ Seg find_inline(const StepArgs& a, int64_t w, int64_t& local) {
    int i = 0;
#pragma unroll
    for (int j = 1; j < kInlineSegs; ++j)
        if (j < a.n_inline && a.inl_prefix[j] <= w) i = j;
    local = w - a.inl_prefix[i];
    return a.inl_segs[i];
}

// Small-block path: binary search in the segmented descriptor table in
// device memory (classes can hold hundreds of segments).
__device__ __forceinline__ Seg find_global(const StepArgs& a, int64_t w, int64_t& local) {
    int lo = 0, hi = a.work.n - 1;  // largest i with prefix[i] <= w
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.work.prefix[mid] <= w) lo = mid; else hi = mid - 1;
    }
    local = w - a.work.prefix[lo];
    const int32_t* src = reinterpret_cast<const int32_t*>(a.segs + a.work.seg_idx[lo]);
    Seg sg;
    int32_t* dst = reinterpret_cast<int32_t*>(&sg);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(Seg) / 4); ++i) dst[i] = __builtin_amdgcn_readfirstlane(src[i]);
    return sg;
}

// ---------------------------------------------------------------------------
// kernels
// Tiled runs: copy a tensor range into the output, or write zeros.
// mode 0: one output `out`; mode 1: grad_shard and param_shard of states[y].
__device__ __forceinline__ void run_tile(const RunArgs& r, int64_t tile, const uint16_t* const* grad_ptrs,
                                         uint16_t* out, const ve_shard_state* states, int mode, int y) {
    constexpr int V = 8;                        // bf16 per 16-byte vector
    constexpr int PER = kRunTile / (256 * V);   // vectors per thread
    const int ri = r.tile_run[tile];
    const Run rn = r.runs[ri];
    int64_t t0, len;
    run_tile_span(rn.dst, rn.len, tile - r.tile_prefix[ri], t0, len);
    uint16_t* o0 = out;
    uint16_t* o1 = nullptr;
    if (mode == 1) {
        o0 = states[y].grad_shard;
        o1 = states[y].param_shard;
    }
    const uint16_t* src = rn.tensor >= 0 ? grad_ptrs[rn.tensor] + rn.src + t0 : nullptr;
    const bool aligned = (((uintptr_t)(o0 + rn.dst + t0) | (uintptr_t)(o1 ? o1 + rn.dst + t0 : nullptr) |
                           (uintptr_t)src) & 15) == 0;
    const VE_GLOBAL uint16_t* s = (const VE_GLOBAL uint16_t*)src;
    VE_GLOBAL uint16_t* d0 = (VE_GLOBAL uint16_t*)(o0 + rn.dst + t0);
    VE_GLOBAL uint16_t* d1 = o1 ? (VE_GLOBAL uint16_t*)(o1 + rn.dst + t0) : nullptr;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        // vector q*256 + tid: each wave-wide access is 1 KB contiguous
        const int64_t i0 = ((int64_t)q * 256 + threadIdx.x) * V;
        if (i0 >= len) break;
        if (aligned && i0 + V <= len) {
            u32x4 a = u32x4{0, 0, 0, 0};
            if (s) a = ldv<VE_NONTEMPORAL>((const VE_GLOBAL u32x4*)(s + i0));
            stv<VE_NONTEMPORAL>((VE_GLOBAL u32x4*)(d0 + i0), a);
            if (d1) stv<VE_NONTEMPORAL>((VE_GLOBAL u32x4*)(d1 + i0), a);
        } else {
            const int64_t n = min((int64_t)V, len - i0);
            for (int64_t k = 0; k < n; ++k) {
                const uint16_t v = s ? s[i0 + k] : (uint16_t)0;
                d0[i0 + k] = v;
                if (d1) d1[i0 + k] = v;
            }
        }
    }
}

__global__ void __launch_bounds__(256) k_runs(RunArgs r, const uint16_t* const* grad_ptrs, uint16_t* out,
                                              const ve_shard_state* states, int mode) {
    run_tile(r, blockIdx.x, grad_ptrs, out, states, mode, blockIdx.y);
}

// Code of a one-element block whose absmax is a = max(0, |x|) (the element
// itself).  For a > 0 the general path computes rint(x * fl(127 / a)) and
// clamps it: fl(127 / a) is within a relative 2^-24 of 127 / a and the
// product adds one more rounding of the same size, so x * fl(127 / a) lies
// within 127 * 2^-23 of +-127 (or is +-inf where 127 / a overflows); rint
// and the clamp then give exactly +-127, with the sign of x.  For a == 0 (x
// a signed zero, or a NaN that the max dropped) the general formula, with
// the reciprocal 0, is kept as it is.  So the result equals the general
// path's without its correctly rounded division.
__device__ __forceinline__ uint32_t unit_code(float x, float a) {
    return a > 0.f ? (x < 0.f ? 0x81u : 0x7fu) : quant_byte(x, 0.f);
}

// One-element blocks (kUnit): a lane takes one chunk, i.e. kSmallChunk
// consecutive blocks, each with its own pair of scales.  A block's maximum is
// its element's own |m1| (v1), so no lane exchange is needed.  Every value
// goes through the general path's operations in the same order, so the
// results are bit-identical to a group of one lane per block.
__device__ __forceinline__ void step_unit(const StepArgs& a, const Seg& sg, const ve_shard_state& st,
                                          int64_t local, int lane) {
    constexpr int CH = kSmallChunk;
    const int64_t k0 = local * kUnitPerWave + (int64_t)lane * CH;  // the lane's first block
    const int64_t left = sg.nblocks - k0;
    if (left <= 0) return;
    const Ptrs p = make_ptrs(st, sg.tensor);
    ChunkPos c;
    c.e = sg.panel0 + k0;  // one element per row, one row per block
    c.s = sg.shard_base + c.e;
    c.n = (int32_t)min((int64_t)CH, left);
    const bool vec = vec_ok<CH>(p, c);
    VE_GLOBAL float* msc = (VE_GLOBAL float*)st.m_scale + (sg.block0 + k0);
    VE_GLOBAL float* vsc = (VE_GLOBAL float*)st.v_scale + (sg.block0 + k0);
    const bool svec = c.n == CH && ((((uintptr_t)msc) | ((uintptr_t)vsc)) & 15) == 0;
    In<CH> x;
    float mst[CH], sm[CH], sv[CH];
    load_in(x, p, c, vec);
    load_master(mst, p, c, vec);
    if (svec) {
#pragma unroll
        for (int i = 0; i < CH / 4; ++i) {
            const f32x4 m = ((const VE_GLOBAL f32x4*)msc)[i], v = ((const VE_GLOBAL f32x4*)vsc)[i];
            sm[4 * i] = m.x; sm[4 * i + 1] = m.y; sm[4 * i + 2] = m.z; sm[4 * i + 3] = m.w;
            sv[4 * i] = v.x; sv[4 * i + 1] = v.y; sv[4 * i + 2] = v.z; sv[4 * i + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            sm[i] = i < c.n ? msc[i] : 0.f;
            sv[i] = i < c.n ? vsc[i] : 0.f;
        }
    }
    uint32_t qm[CH / 4], qv[CH / 4];
    float nm[CH], nv[CH];
#pragma unroll
    for (int i = 0; i < CH / 4; ++i) qm[i] = qv[i] = 0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        float m1, v1;
        moments(elem_g(x, i), code_at(x.m[i >> 2], i & 3), code_at(x.v[i >> 2], i & 3), sm[i], sv[i], a.sc, m1, v1);
        const float am = fmaxf(0.f, fabsf(m1)), av = fmaxf(0.f, v1);
        const float d = __builtin_fmaf(__builtin_amdgcn_sqrtf(v1), a.sc.inv_sqrt_bc2, a.sc.eps);
        const float u = m1 * __builtin_amdgcn_rcpf(d);
        mst[i] = __builtin_fmaf(-a.sc.step_size, u, mst[i] * a.sc.decay);
        qm[i >> 2] |= unit_code(m1, am) << (8 * (i & 3));
        qv[i >> 2] |= unit_code(v1, av) << (8 * (i & 3));
        nm[i] = am / 127.0f;
        nv[i] = av / 127.0f;
    }
    store_phase1(x, mst, p, c, vec);
    store_codes<CH>(qm, qv, p, c, vec);
    if (svec) {
#pragma unroll
        for (int i = 0; i < CH / 4; ++i) {
            ((VE_GLOBAL f32x4*)msc)[i] = f32x4{nm[4 * i], nm[4 * i + 1], nm[4 * i + 2], nm[4 * i + 3]};
            ((VE_GLOBAL f32x4*)vsc)[i] = f32x4{nv[4 * i], nv[4 * i + 1], nv[4 * i + 2], nv[4 * i + 3]};
        }
    } else {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            if (i < c.n) {
                msc[i] = nm[i];
                vsc[i] = nv[i];
            }
        }
    }
}

// INLINE: the launch's segments are in the kernel arguments (at most
// kInlineSegs of them), so a wave finds its segment without the chain of
// dependent loads of the binary search in device memory.
template <bool INLINE>
__global__ void __launch_bounds__(256) k_step_small(StepArgs a) {
    if ((int64_t)blockIdx.x >= a.pad_wg0) {  // a padding tile of the same launch
        run_tile(a.pad, (int64_t)blockIdx.x - a.pad_wg0, nullptr, nullptr, a.states, 1, blockIdx.y);
        return;
    }
    constexpr int CH = kSmallChunk;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int64_t gw = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave;
    if (gw >= a.work.total) return;  // whole waves; the kernel has no barrier
    int64_t local;
    Seg sg;
    if constexpr (INLINE) sg = find_inline(a, gw, local);
    else sg = find_global(a, gw, local);
    ve_shard_state st;
    {
        const uint64_t* src = reinterpret_cast<const uint64_t*>(a.states + blockIdx.y);
        uint64_t* dst = reinterpret_cast<uint64_t*>(&st);
#pragma unroll
        for (int i = 0; i < 8; ++i) dst[i] = sload(src + i);
    }
    if (sg.cls == kUnit) {
        step_unit(a, sg, st, local, lane);
        return;
    }
    const int G = sg.group;
    const int64_t k = local * (64 / G) + lane / G;
    const int li = lane & (G - 1);
    const bool active = k < sg.nblocks;
    const Ptrs p = make_ptrs(st, sg.tensor);

    Geo geo;
    ChunkPos cp;
    bool vec = false, has = false;
    float sm = 0.f, sv = 0.f, am = 0.f, av = 0.f;
    In<CH> x;
    if (active) {
        geo = block_geo<CH>(sg, k);
        has = li < geo.nchunks;
        if (has) {
            sm = ((const VE_GLOBAL float*)st.m_scale)[geo.blk];
            sv = ((const VE_GLOBAL float*)st.v_scale)[geo.blk];
            float mst[CH];
            cp = chunk_pos<CH>(geo, sg.shard_base, li);
            vec = vec_ok<CH>(p, cp);
            load_in(x, p, cp, vec);
            load_master(mst, p, cp, vec);
            phase1(x, mst, p, cp, vec, sm, sv, a.sc, am, av);
        }
    }
    am = group_max(am, G);
    av = group_max(av, G);
    if (active) {
        const float im = am > 0.f ? 127.0f / am : 0.f;
        const float iv = av > 0.f ? 127.0f / av : 0.f;
        if (li == 0) {
            ((VE_GLOBAL float*)st.m_scale)[geo.blk] = am / 127.0f;
            ((VE_GLOBAL float*)st.v_scale)[geo.blk] = av / 127.0f;
        }
        if (has) {
            make_opaque(x);
            phase2(x, p, cp, vec, sm, sv, im, iv, a.sc);
        }
    }
}

#ifndef VE_WG_ROTATE
#define VE_WG_ROTATE 1
#endif
#ifndef VE_MASTER_AHEAD
#define VE_MASTER_AHEAD 0  // 0: per shape (4 groups ahead, 8 from 12 groups per thread)
#endif

// One workgroup per block; thread tid owns groups tid, tid + T, ... of
// kWgChunk elements, so wave instruction j covers 64 consecutive groups.
//
// Load order matters: vector loads and stores retire through one in-order
// counter, so waiting for a load also waits for every store issued before
// it.  All input loads are therefore issued first (they stay in registers),
// and each group's master is loaded MA groups ahead of its update, i.e.
// before the stores of the groups in between.
//
// The counter waits are placed by the compiler, and any control flow that
// makes the number of accesses in flight path-dependent turns them into
// full drains (every group's update would then wait for the previous
// group's stores to reach memory).  A block whose chunks are all full and
// aligned -- every block of a contiguous, 16-byte-aligned layout -- is
// therefore handled by a straight-line FAST form: block-relative vector
// accesses only, the loads of idle lanes clamped to the block's last chunk
// (in bounds, result unused), the arithmetic done by every lane, and only
// the stores and the absmax contribution predicated.  Two FAST forms: LINEAR,
// where a lane's chunk in slot k sits at lane0 + k * step (one contiguous run
// per block, or tiles whose rows hold a whole number of workgroup sweeps), so
// a lane keeps three byte offsets in all and the slot part goes into the
// instruction's scalar offset; and TILED, with one offset per chunk.
// Anything else takes the general form.
enum WgMode : int { kWgGeneral = 0, kWgLinear = 1, kWgTiled = 2 };

struct WgItem {
    Seg sg;
    Geo geo;
    Ptrs p;
    FastRsrc fb;  // block-relative buffers (FAST modes)
    float sm, sv;
    float* m_scale;
    float* v_scale;
    int rot;
    int mode;        // WgMode
    uint32_t lane0;  // LINEAR: this lane's element offset in slot 0
    uint32_t step;   // LINEAR: element offset between slots (wave-uniform)
};

// Item (state y, block `local` of segment sg); xw (the launch's work item)
// sets the sweep rotation.
template <int GPT>
__device__ __forceinline__ WgItem wg_item_for(const StepArgs& a, int64_t y, const Seg& sg, int64_t local,
                                              int64_t xw) {
    constexpr int CH = kWgChunk;
    WgItem it;
    it.sg = sg;
    ve_shard_state st;
    {
        static_assert(sizeof(ve_shard_state) == 8 * sizeof(uint64_t), "eight pointers");
        const uint64_t* src = reinterpret_cast<const uint64_t*>(a.states + y);
        uint64_t* dst = reinterpret_cast<uint64_t*>(&st);
#pragma unroll
        for (int i = 0; i < 8; ++i) dst[i] = sload(src + i);
    }
    it.geo = block_geo<CH>(it.sg, local);
    it.p = make_ptrs<true>(st, it.sg.tensor);
    it.sm = sload(st.m_scale + it.geo.blk);
    it.sv = sload(st.v_scale + it.geo.blk);
    it.m_scale = st.m_scale;
    it.v_scale = st.v_scale;
    // Register slot c holds group tid + ((c + rot) mod GPT) * T: neighbouring
    // workgroups start their sweeps at different offsets of their blocks, so
    // the sweep fronts of the resident blocks (whose starts are a multiple of
    // the block size apart) do not all address the same memory channels.
    it.rot = VE_WG_ROTATE ? (int)(xw % GPT) : 0;
    // FAST: every chunk full and naturally aligned, and the block's span
    // small enough for 32-bit buffer offsets.
    const int64_t span = (int64_t)(it.geo.nruns - 1) * it.geo.stride + it.geo.run;
    const bool fast = it.p.aligned && ((it.geo.e0 | it.sg.shard_base | it.geo.run) & (CH - 1)) == 0 &&
                      (it.geo.nruns == 1 || (it.geo.stride & (CH - 1)) == 0) && span < kFastMaxSpan;
    const uint32_t tid = threadIdx.x, cpr = (uint32_t)it.geo.cpr;
    if (!fast) {
        it.mode = kWgGeneral;
    } else if (it.geo.nruns == 1) {
        it.mode = kWgLinear;
        it.lane0 = tid * CH;
        it.step = (uint32_t)blockDim.x * CH;
    } else if (blockDim.x % cpr == 0) {
        it.mode = kWgLinear;
        it.lane0 = (tid / cpr) * (uint32_t)it.geo.stride + (tid % cpr) * CH;
        it.step = (blockDim.x / cpr) * (uint32_t)it.geo.stride;
    } else {
        it.mode = kWgTiled;
    }
    if (fast) {
        const int64_t s0 = it.sg.shard_base + it.geo.e0;
        it.fb.grad = buf_rsrc(it.p.grad + it.geo.e0, 2 * span);
        it.fb.grad_shard = buf_rsrc(it.p.grad_shard + s0, 2 * span);
        it.fb.master = buf_rsrc(it.p.master + s0, 4 * span);
        it.fb.m_q = buf_rsrc(it.p.m_q + s0, span);
        it.fb.v_q = buf_rsrc(it.p.v_q + s0, span);
        it.fb.param = buf_rsrc(it.p.param + s0, 2 * span);
    }
    return it;
}

// Item (state y, block xw of the launch's segment slice).
template <int GPT>
__device__ __forceinline__ WgItem wg_item_at(const StepArgs& a, int64_t y, int64_t xw) {
    int64_t local;
    const Seg sg = find_inline(a, xw, local);
    return wg_item_for<GPT>(a, y, sg, local, xw);
}

template <int T, int GPT>
__device__ __forceinline__ int wg_slot_chunk(const WgItem& it, int c) {
    return (int)threadIdx.x + ((c + it.rot) % GPT) * T;
}

// TILED: element offset of chunk ci, kept per chunk (kNoChunkByte / 4 past
// the block's end).
__device__ __forceinline__ uint32_t tiled_off(const WgItem& it, int ci) {
    constexpr int CH = kWgChunk;
    const uint32_t cpr = (uint32_t)it.geo.cpr;
    const uint32_t ri = (uint32_t)ci / cpr;
    const uint32_t o = ri * (uint32_t)it.geo.stride + ((uint32_t)ci - ri * cpr) * CH;
    return ci < it.geo.nchunks ? o : kNoChunkByte / 4;
}

// Byte offsets of register slot c's chunk.
template <int T, int GPT, int MODE, class Item>
__device__ __forceinline__ ChunkAddr wg_addr(const Item& it, const uint32_t (&off)[GPT], int c) {
    ChunkAddr a;
    if constexpr (MODE == kWgLinear) {
        const int k = (c + it.rot) % GPT;  // wave-uniform slot
        // Recomputed at every use (the opaque copy keeps the compiler from
        // holding each slot's offsets in registers across the block).
        uint32_t l0 = it.lane0;
        opaque(l0);
        const bool ok = (int)threadIdx.x < it.geo.nchunks - k * T;
        const uint32_t so = (uint32_t)k * it.step;
        a.v1 = ok ? l0 : kNoChunkByte;
        a.v2 = ok ? l0 * 2u : kNoChunkByte;
        a.v4 = ok ? l0 * 4u : kNoChunkByte;
        a.s1 = so;
        a.s2 = so * 2u;
        a.s4 = so * 4u;
    } else {
        uint32_t o = off[c];
        opaque(o);
        a.v1 = o;
        a.v2 = o * 2u;
        a.v4 = o * 4u;
        a.s1 = a.s2 = a.s4 = 0;
    }
    return a;
}

// Issue the input loads of every group and the master loads of the first MA
// (FAST modes also record each group's offset).
template <int T, int GPT, int MA, int MODE>
__device__ __forceinline__ void wg_issue(In<kWgChunk> (&x)[GPT], float (&mst)[MA + 1][kWgChunk],
                                         uint32_t (&off)[GPT], const WgItem& it) {
    constexpr int CH = kWgChunk;
#pragma unroll
    for (int c = 0; c < GPT; ++c) {
        const int ci = wg_slot_chunk<T, GPT>(it, c);
        if constexpr (MODE != kWgGeneral) {
            if constexpr (MODE == kWgTiled) off[c] = tiled_off(it, ci);
            const ChunkAddr ad = wg_addr<T, GPT, MODE>(it, off, c);
            load_in_fast(x[c], it.fb, ad);
            if (c < MA) load_master_fast(mst[c % (MA + 1)], it.fb, ad);
            __builtin_amdgcn_sched_barrier(0);  // group-major issue order
        } else if (ci < it.geo.nchunks) {
            const ChunkPos cp = chunk_pos<CH>(it.geo, it.sg.shard_base, ci);
            const bool vec = vec_ok<CH>(it.p, cp);
            load_in(x[c], it.p, cp, vec);
            if (c < MA) load_master(mst[c % (MA + 1)], it.p, cp, vec);
        }
    }
    // every load issued before any arithmetic starts
    if constexpr (MODE != kWgGeneral) __builtin_amdgcn_sched_barrier(0);
}

// Whether a FAST block keeps its fresh moments in registers from phase 1 to
// phase 2 (eight VGPRs per group) instead of recomputing them from the four
// held input registers (more VALU work than the quantisation itself).
// Measured on MI355X: 1.0% faster for 128x128 tiles in 1024 x 4 workgroups,
// 2-3% slower for the 28,672- and 46,080-element row blocks in 512-thread
// workgroups, so it is used for the 1024-thread shapes with few groups only.
#ifndef VE_KEEP_MOMENTS
#define VE_KEEP_MOMENTS 2  // 0: never, 1: always, 2: 1024-thread shapes of up to 8 groups
#endif
template <int T, int GPT>
struct WgKeep {
    static constexpr bool value = VE_KEEP_MOMENTS == 1 || (VE_KEEP_MOMENTS == 2 && T == 1024 && GPT <= 8);
};

// Whether a FAST block stores its gradient-slice copy in phase 2 (from the
// held input registers) instead of in phase 1.  Same bytes, moved from the
// store-heavy phase 1 into the VALU-bound phase 2.
#ifndef VE_LATE_COPY
#define VE_LATE_COPY 2  // 0: never, 1: always, 2: 1024-thread shapes of up to 8 groups
#endif
template <int T, int GPT>
struct WgLateCopy {
    static constexpr bool value = VE_LATE_COPY == 1 || (VE_LATE_COPY == 2 && T == 1024 && GPT <= 8);
};

// One block: phase 1 (inputs already issued), the absmax reduction, phase 2.
template <int T, int GPT, int MA, int MODE>
__device__ __forceinline__ void wg_block(In<kWgChunk> (&x)[GPT], float (&mst)[MA + 1][kWgChunk],
                                         const uint32_t (&off)[GPT], const WgItem& it, float (&red)[2][T / 64],
                                         const StepScalars& sc) {
    constexpr int CH = kWgChunk;
    constexpr bool KEEP = MODE != kWgGeneral && WgKeep<T, GPT>::value;
    constexpr bool LATE = WgLateCopy<T, GPT>::value;
    const int tid = threadIdx.x;
    const int nch = it.geo.nchunks;
    float am = 0.f, av = 0.f;
    float km[KEEP ? GPT : 1][CH], kv[KEEP ? GPT : 1][CH];
#pragma unroll
    for (int c = 0; c < GPT; ++c) {
        const int ci = wg_slot_chunk<T, GPT>(it, c);
        if constexpr (MODE != kWgGeneral) {
            if (c + MA < GPT) load_master_fast(mst[(c + MA) % (MA + 1)], it.fb, wg_addr<T, GPT, MODE>(it, off, c + MA));
            if constexpr (KEEP)
                phase1_fast_k<LATE>(x[c], mst[c % (MA + 1)], it.fb, wg_addr<T, GPT, MODE>(it, off, c), it.sm, it.sv, sc, am,
                              av, km[c], kv[c]);
            else
                phase1_fast<LATE>(x[c], mst[c % (MA + 1)], it.fb, wg_addr<T, GPT, MODE>(it, off, c), it.sm, it.sv, sc, am, av);
            // keep the groups in program order (hoisting later groups' work
            // would run out of registers)
            __builtin_amdgcn_sched_barrier(0);
        } else {
            if (c + MA < GPT) {
                const int cn = wg_slot_chunk<T, GPT>(it, c + MA);
                if (cn < nch) {
                    const ChunkPos cpn = chunk_pos<CH>(it.geo, it.sg.shard_base, cn);
                    load_master(mst[(c + MA) % (MA + 1)], it.p, cpn, vec_ok<CH>(it.p, cpn));
                }
            }
            if (ci < nch) {
                const ChunkPos cp = chunk_pos<CH>(it.geo, it.sg.shard_base, ci);
                phase1(x[c], mst[c % (MA + 1)], it.p, cp, vec_ok<CH>(it.p, cp), it.sm, it.sv, sc, am, av);
            }
        }
    }
    am = wave_max(am);
    av = wave_max(av);
    if ((tid & 63) == 0) {
        red[0][tid >> 6] = am;
        red[1][tid >> 6] = av;
    }
    lds_barrier();
    am = 0.f;
    av = 0.f;
#pragma unroll
    for (int i = 0; i < T / 64; ++i) {
        am = fmaxf(am, red[0][i]);
        av = fmaxf(av, red[1][i]);
    }
    const float im = am > 0.f ? 127.0f / am : 0.f;
    const float iv = av > 0.f ? 127.0f / av : 0.f;
    if (tid == 0) {
        ((VE_GLOBAL float*)it.m_scale)[it.geo.blk] = am / 127.0f;
        ((VE_GLOBAL float*)it.v_scale)[it.geo.blk] = av / 127.0f;
    }
#pragma unroll
    for (int c = 0; c < GPT; ++c) {
        const int ci = wg_slot_chunk<T, GPT>(it, c);
        if constexpr (KEEP) {
            phase2_fast_kept<LATE>(x[c], km[c], kv[c], it.fb, wg_addr<T, GPT, MODE>(it, off, c), im, iv);
            __builtin_amdgcn_sched_barrier(0);
            continue;
        }
        make_opaque(x[c]);
        if constexpr (MODE != kWgGeneral) {
            phase2_fast<LATE>(x[c], it.fb, wg_addr<T, GPT, MODE>(it, off, c), it.sm, it.sv, im, iv, sc);
            __builtin_amdgcn_sched_barrier(0);
        } else if (ci < nch) {
            const ChunkPos cp = chunk_pos<CH>(it.geo, it.sg.shard_base, ci);
            phase2(x[c], it.p, cp, vec_ok<CH>(it.p, cp), it.sm, it.sv, im, iv, sc);
        }
    }
}

// Groups whose master values are in flight ahead of their update: more for
// the FAST forms with many groups per thread; the general form keeps 4 (its
// register use would otherwise set the kernel's occupancy).
template <int GPT, int MODE>
struct WgAhead {
    static constexpr int v0 =
        MODE == kWgGeneral ? 4 : (VE_MASTER_AHEAD > 0 ? VE_MASTER_AHEAD : (GPT >= 12 ? 8 : 4));
    static constexpr int value = v0 < GPT ? v0 : GPT;
};

template <int T, int GPT, int MODE>
__device__ __forceinline__ void wg_one(const WgItem& it, float (&red)[2][T / 64], const StepScalars& sc) {
    constexpr int MA = WgAhead<GPT, MODE>::value;
    In<kWgChunk> x[GPT];
    float mst[MA + 1][kWgChunk];  // ring of master values in flight
    uint32_t off[GPT];
    wg_issue<T, GPT, MA, MODE>(x, mst, off, it);
    wg_block<T, GPT, MA, MODE>(x, mst, off, it, red, sc);
}

template <int T, int GPT>
__global__ void __launch_bounds__(T) k_step_wg(StepArgs a) {
    __shared__ float s_red[2][T / 64];
    const WgItem it = wg_item_at<GPT>(a, blockIdx.y, blockIdx.x);
    if (it.mode == kWgLinear) wg_one<T, GPT, kWgLinear>(it, s_red, a.sc);
    else if (it.mode == kWgTiled) wg_one<T, GPT, kWgTiled>(it, s_red, a.sc);
    else wg_one<T, GPT, kWgGeneral>(it, s_red, a.sc);
}

// Blocks too large for registers: two sweeps, the second re-reading inputs.
__global__ void __launch_bounds__(256) k_step_huge(StepArgs a) {
    constexpr int CH = kWgChunk;
    __shared__ float s_red[2][4];
    const int tid = threadIdx.x, T = blockDim.x;
    int64_t local;
    const Seg sg = find_inline(a, blockIdx.x, local);
    const ve_shard_state st = a.states[blockIdx.y];
    const Geo geo = block_geo<CH>(sg, local);
    const Ptrs p = make_ptrs<true>(st, sg.tensor);
    const float sm = sload(st.m_scale + geo.blk), sv = sload(st.v_scale + geo.blk);
    float am = 0.f, av = 0.f;
    for (int ci = tid; ci < geo.nchunks; ci += T) {
        In<CH> x;
        const ChunkPos cp = chunk_pos<CH>(geo, sg.shard_base, ci);
        load_in(x, p, cp, vec_ok<CH>(p, cp));
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            float m1, v1;
            moments(elem_g(x, i), code_at(x.m[i >> 2], i & 3), code_at(x.v[i >> 2], i & 3), sm, sv, a.sc, m1, v1);
            am = fmaxf(am, fabsf(m1));
            av = fmaxf(av, v1);
        }
    }
    am = wave_max(am);
    av = wave_max(av);
    if ((tid & 63) == 0) {
        s_red[0][tid >> 6] = am;
        s_red[1][tid >> 6] = av;
    }
    __syncthreads();
    am = fmaxf(fmaxf(s_red[0][0], s_red[0][1]), fmaxf(s_red[0][2], s_red[0][3]));
    av = fmaxf(fmaxf(s_red[1][0], s_red[1][1]), fmaxf(s_red[1][2], s_red[1][3]));
    const float im = am > 0.f ? 127.0f / am : 0.f;
    const float iv = av > 0.f ? 127.0f / av : 0.f;
    for (int ci = tid; ci < geo.nchunks; ci += T) {
        In<CH> x;
        float mst[CH];
        const ChunkPos cp = chunk_pos<CH>(geo, sg.shard_base, ci);
        const bool vec = vec_ok<CH>(p, cp);
        load_in(x, p, cp, vec);
        load_master(mst, p, cp, vec);
        float dm = 0.f, dv = 0.f;
        phase1(x, mst, p, cp, vec, sm, sv, a.sc, dm, dv);
        phase2(x, p, cp, vec, sm, sv, im, iv, a.sc);
    }
    if (tid == 0) {
        ((VE_GLOBAL float*)st.m_scale)[geo.blk] = am / 127.0f;
        ((VE_GLOBAL float*)st.v_scale)[geo.blk] = av / 127.0f;
    }
}

// ---------------------------------------------------------------------------
// Persistent form for the row-block shapes (dyn_shape(): 512 threads from 14
// groups per thread, 768 threads, 1024 threads with 7 to 10: row blocks of
// 16K to 49K elements).  The grid holds as many workgroups as the CUs keep
// resident (one per CU here: the LDS staging area takes 114-156 KiB) and
// every workgroup takes its blocks from a ticket counter, one relaxed
// device-scope add per block, so a CU that finishes early takes the next
// block as the hardware dispatcher would, without the gap between one
// workgroup's end and the next one's start.  A block that is one contiguous
// FAST run, its span a multiple of 16 elements, is staged: the block before
// it on the same CU brings its gradient and both code streams (4 of its 8
// input bytes per element, as many register slots as fit the LDS budget)
// into LDS with buffer-to-LDS loads issued in the middle of its own phase 2,
// so the CU keeps HBM requests in flight through its reduction tail and the
// block switch.  Measured on MI355X in one process, outputs bit-identical to
// the one-shot kernel: 28,672-element rows 5.43-5.52 TB/s one-shot (512 x
// 16), 5.72 with tickets alone, 5.88 staged, 5.95 staged in 1024 x 7;
// 46,080-element rows 5.28-5.31 (512 x 24), 5.46, 5.54, 5.61 in 768 x 15.
// A persistent form with a static block order (block i on workgroup i mod
// grid) ran 4% below the one-shot kernel, staged or not: the slowest CUs set
// the end.
//
// sched[0] is the next ticket, sched[1] counts the workgroups that have left;
// the last one resets both, so the next launch on the stream (or a graph
// replay) starts from zero.  Launches that overlap in time must not share
// the counters.
#ifndef VE_DYN_MPRE
#define VE_DYN_MPRE 2  // master groups of a staged block loaded by the block before it
#endif
#ifndef VE_DYN_SLOTS
#define VE_DYN_SLOTS 16  // at most this many staged register slots (T x 16 bytes of LDS each)
#endif
#ifndef VE_DYN_DMA_AT
#define VE_DYN_DMA_AT 8  // phase-2 group before which the next block's loads go out
#endif
#ifndef VE_DYN_LDS_KIB
#define VE_DYN_LDS_KIB 156  // staging budget of the 160 KiB of LDS
#endif
constexpr int kDynLdsBytes = VE_DYN_LDS_KIB * 1024;

template <int T, int GPT>
struct DynCfg {
    static constexpr int SLOT_BYTES = T * kWgChunk * 4;  // gradient (2 B) + m and v codes (1 B each) per element
    static constexpr int FIT = kDynLdsBytes / SLOT_BYTES;
    static constexpr int PF0 = GPT < VE_DYN_SLOTS ? GPT : VE_DYN_SLOTS;
    static constexpr int PF = PF0 < FIT ? PF0 : FIT;  // staged slots
    static constexpr int SPAN = PF * T * kWgChunk;    // staged elements
    static constexpr int LDS = PF * SLOT_BYTES;
    static constexpr int DMA_AT = VE_DYN_DMA_AT < GPT ? VE_DYN_DMA_AT : GPT - 1;
    // master loads in flight ahead of their update: 8 from 12 groups per
    // thread (more spill registers at 768 threads), else 6 (1024 x 7: 0.4%
    // faster than 4), at most GPT
    static constexpr int MA0 = GPT >= 12 ? 8 : 6;
    static constexpr int MA = MA0 < GPT ? MA0 : GPT;
    // of those, the first MPRE of a staged block are loaded by the block
    // before it, with its staging loads, into the master ring (dead in that
    // block's phase 2): the block then starts without an HBM round trip.
    // 28,672-element rows: 2 groups 0.75% faster than none, 1 or 3 less;
    // 46,080-element rows: no change.
    static constexpr int MPRE = VE_DYN_MPRE < MA ? VE_DYN_MPRE : MA;
    // gradient-slice copy stored in phase 2 instead of phase 1 (as
    // WgLateCopy): 768 x 15 0.8% faster that way, 1024 x 7 0.2% slower
    static constexpr bool LATE = T == 768;
    static_assert(T % 256 == 0, "waves split evenly into gradient, m and v pieces");
};

// The fields of a block that the staged path uses (a WgItem's LINEAR subset:
// fewer scalar registers held across the loop).
struct DynItem {
    FastRsrc fb;
    Geo geo;
    float sm, sv;
    float* m_scale;
    float* v_scale;
    int rot;
    uint32_t lane0, step;
    bool staged_ok;  // one contiguous FAST run whose streams can go through LDS
};

template <int GPT>
__device__ __forceinline__ DynItem dyn_item(const StepArgs& a, uint32_t w, uint32_t nx) {
    const uint32_t y = __builtin_amdgcn_readfirstlane(w / nx);
    const WgItem it = wg_item_at<GPT>(a, y, w - y * nx);
    DynItem d;
    d.fb = it.fb;
    d.geo = it.geo;
    d.sm = it.sm;
    d.sv = it.sv;
    d.m_scale = it.m_scale;
    d.v_scale = it.v_scale;
    d.rot = it.rot;
    d.lane0 = it.lane0;
    d.step = it.step;
    // the 16-byte LDS loads need each stream's span to be a multiple of 16 bytes
    d.staged_ok = it.mode == kWgLinear && it.geo.nruns == 1 && (it.geo.run & 15) == 0;
    return d;
}

typedef __attribute__((address_space(3))) void lds_void;

// Stage block `nt`'s first PF register slots (in its rotated slot order) into
// LDS: slot c's gradient at [c * T * 8], its m codes at [2 SPAN + c * T * 4],
// its v codes at [3 SPAN + c * T * 4].  A slot is T / 64 pieces of 1 KiB, one
// per wave: the first half of the waves move its gradient, the next quarter
// its m codes, the last quarter its v codes, 16 bytes per lane; reads past
// the block's span return zeros, which no lane uses.
template <int T, int GPT, class Item>
__device__ __forceinline__ void dyn_stage(const Item& nt, uint8_t* sb) {
    constexpr int W = T / 64;
    constexpr int PF = DynCfg<T, GPT>::PF, SPAN = DynCfg<T, GPT>::SPAN;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const bool gw = wave < W / 2, mw = !gw && wave < 3 * W / 4;
    const __amdgpu_buffer_rsrc_t r = gw ? nt.fb.grad : (mw ? nt.fb.m_q : nt.fb.v_q);
    const int piece = gw ? wave : (mw ? wave - W / 2 : wave - 3 * W / 4);
    const int esz = gw ? 2 : 1;
    const int base = gw ? 0 : (mw ? 2 * SPAN : 3 * SPAN);
#pragma unroll
    for (int c = 0; c < PF; ++c) {
        const int k = (c + nt.rot) % GPT;
        const int src = (k * T * kWgChunk) * esz + piece * 1024 + lane * 16;
        const int dst = base + c * T * kWgChunk * esz + piece * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(sb + dst), 16, src, 0, 0, kBufNT);
    }
}

// One staged or unstaged block: phase 1, absmax, phase 2.  The next ticket is
// taken during phase 1 and the next block staged during phase 2 when
// possible; returns the next ticket and sets stage_next.
template <int T, int GPT, bool STAGED>
__device__ __forceinline__ uint32_t dyn_block(const DynItem& it, const StepArgs& A, uint32_t nx, uint32_t nitems,
                                              bool& stage_next, uint32_t* s_next, uint8_t* sb,
                                              float (&red)[2][T / 64],
                                              float (&mst)[DynCfg<T, GPT>::MA + 1][kWgChunk]) {
    constexpr int CH = kWgChunk;
    constexpr int MODE = kWgLinear;
    constexpr int PF = DynCfg<T, GPT>::PF, SPAN = DynCfg<T, GPT>::SPAN, DMA_AT = DynCfg<T, GPT>::DMA_AT;
    constexpr int MA = DynCfg<T, GPT>::MA, MPRE = DynCfg<T, GPT>::MPRE;
    constexpr bool LATE = DynCfg<T, GPT>::LATE;
    const StepScalars& sc = A.sc;
    const int tid = threadIdx.x;
    In<CH> x[GPT];
    const uint32_t off[GPT] = {};  // unused by LINEAR addressing
#pragma unroll
    for (int c = 0; c < GPT; ++c) {
        const ChunkAddr ad = wg_addr<T, GPT, MODE>(it, off, c);
        if (!STAGED || c >= PF) load_in_fast(x[c], it.fb, ad);
        if (c < MA && !(STAGED && c < MPRE)) load_master_fast(mst[c % (MA + 1)], it.fb, ad);
        __builtin_amdgcn_sched_barrier(0);
    }
    uint32_t ticket = 0;
    if (tid == 0) ticket = atomicAdd(A.sched, 1u);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (STAGED) {
#pragma unroll
        for (int c = 0; c < PF; ++c) {
            // a lane without a chunk takes zeros, as the range-checked loads give it
            const int k = (c + it.rot) % GPT;
            const bool ok = tid < it.geo.nchunks - k * T;
            const uint2 g = *(const uint2*)(sb + c * T * 8 + tid * 8);
            const uint32_t m = *(const uint32_t*)(sb + 2 * SPAN + c * T * 4 + tid * 4);
            const uint32_t v = *(const uint32_t*)(sb + 3 * SPAN + c * T * 4 + tid * 4);
            x[c].g[0] = ok ? g.x : 0u;
            x[c].g[1] = ok ? g.y : 0u;
            x[c].m[0] = ok ? m : 0u;
            x[c].v[0] = ok ? v : 0u;
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    float am = 0.f, av = 0.f;
#pragma unroll
    for (int c = 0; c < GPT; ++c) {
        if (c + MA < GPT) load_master_fast(mst[(c + MA) % (MA + 1)], it.fb, wg_addr<T, GPT, MODE>(it, off, c + MA));
        phase1_fast<LATE>(x[c], mst[c % (MA + 1)], it.fb, wg_addr<T, GPT, MODE>(it, off, c), it.sm, it.sv, sc, am,
                          av);
        __builtin_amdgcn_sched_barrier(0);
    }
    am = wave_max(am);
    av = wave_max(av);
    if ((tid & 63) == 0) {
        red[0][tid >> 6] = am;
        red[1][tid >> 6] = av;
    }
    if (tid == 0) *s_next = ticket;
    lds_barrier();
    const uint32_t wn = *s_next;
    const bool more = wn < nitems;
    const DynItem nt = dyn_item<GPT>(A, more ? wn : 0u, nx);
    stage_next = more && nt.staged_ok;
    am = 0.f;
    av = 0.f;
#pragma unroll
    for (int i = 0; i < T / 64; ++i) {
        am = fmaxf(am, red[0][i]);
        av = fmaxf(av, red[1][i]);
    }
    const float im = am > 0.f ? 127.0f / am : 0.f;
    const float iv = av > 0.f ? 127.0f / av : 0.f;
    if (tid == 0) {
        ((VE_GLOBAL float*)it.m_scale)[it.geo.blk] = am / 127.0f;
        ((VE_GLOBAL float*)it.v_scale)[it.geo.blk] = av / 127.0f;
    }
#pragma unroll
    for (int c = 0; c < GPT; ++c) {
        if (c == DMA_AT) {
            __builtin_amdgcn_sched_barrier(0);
            if (stage_next) {
                dyn_stage<T, GPT>(nt, sb);
#pragma unroll
                for (int c2 = 0; c2 < MPRE; ++c2)
                    load_master_fast(mst[c2 % (MA + 1)], nt.fb, wg_addr<T, GPT, MODE>(nt, off, c2));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        make_opaque(x[c]);
        phase2_fast<LATE>(x[c], it.fb, wg_addr<T, GPT, MODE>(it, off, c), it.sm, it.sv, im, iv, sc);
        __builtin_amdgcn_sched_barrier(0);
    }
    return wn;
}

template <int T, int GPT>
__global__ void __launch_bounds__(T) k_step_dyn(StepArgs a, uint32_t nx, uint32_t nitems) {
    constexpr int GROUP_STORES = DynCfg<T, GPT>::LATE ? 3 : 2;  // phase-2 stores per group
    constexpr int AFTER_DMA = GROUP_STORES * (GPT - DynCfg<T, GPT>::DMA_AT);
    static_assert(AFTER_DMA <= 63, "vmcnt holds at most 63");
    __shared__ float s_red[2][T / 64];
    __shared__ uint32_t s_next;
    __shared__ __attribute__((aligned(16))) uint8_t s_buf[DynCfg<T, GPT>::LDS];
    float mst[DynCfg<T, GPT>::MA + 1][kWgChunk];  // master ring, carried from block to block
    if (threadIdx.x == 0) s_next = atomicAdd(a.sched, 1u);
    __syncthreads();
    uint32_t w = s_next;
    bool staged = false;
    while (w < nitems) {
        const DynItem it = dyn_item<GPT>(a, w, nx);
        uint32_t wn;
        if (it.staged_ok) {
            __builtin_amdgcn_sched_barrier(0);
            // This wave's staging loads (and this block's first master
            // loads) went out before its last AFTER_DMA stores: wait for
            // them (not for the stores), then for every wave.
            // The barrier also separates the previous block's reads of s_red
            // and s_next from this block's writes.
            if (staged) __builtin_amdgcn_s_waitcnt(0x0F70 | (AFTER_DMA & 15) | (((AFTER_DMA >> 4) & 3) << 14));
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            bool sn;
            if (staged) wn = dyn_block<T, GPT, true>(it, a, nx, nitems, sn, &s_next, s_buf, s_red, mst);
            else wn = dyn_block<T, GPT, false>(it, a, nx, nitems, sn, &s_next, s_buf, s_red, mst);
            staged = sn;
        } else {
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_s_barrier();
            if (threadIdx.x == 0) s_next = atomicAdd(a.sched, 1u);  // read after wg_one's barrier
            const uint32_t y = __builtin_amdgcn_readfirstlane(w / nx);
            const WgItem gi = wg_item_at<GPT>(a, y, w - y * nx);
            if (gi.mode == kWgLinear) wg_one<T, GPT, kWgLinear>(gi, s_red, a.sc);
            else if (gi.mode == kWgTiled) wg_one<T, GPT, kWgTiled>(gi, s_red, a.sc);
            else wg_one<T, GPT, kWgGeneral>(gi, s_red, a.sc);
            wn = s_next;
            staged = false;
        }
        w = wn;
    }
    // Every ticket this workgroup will take is taken; the last workgroup out
    // resets the counters for the next launch.
    if (threadIdx.x == 0) {
        const uint32_t left = atomicAdd(a.sched + 1, 1u);
        if (left == gridDim.x - 1) {
            atomicExch(a.sched, 0u);
            atomicExch(a.sched + 1, 0u);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
}

// ---------------------------------------------------------------------------
// Persistent form for short row blocks (2,048 or 4,096 groups: rows of 8K or
// 16K elements): a work item is RPI consecutive blocks of one row-block
// segment, one contiguous span of 8,192 groups that is staged and streamed
// like a long row (1024 x 8), with one absmax, one scale pair and one
// requantisation per block.  Slot c of a thread belongs to block c / SPR
// (no sweep rotation), so every per-block index below is a compile-time
// constant.  Items whose blocks are not all full rows of naturally aligned
// data run block by block through the workgroup code.
// Measured on MI355X, a LLaMA rank of 8,192-element rows with 80 buckets a
// call, against the one-shot 256 x 8 kernel: 5,853-5,902 GB/s against
// 5,509-5,528 on one box, +3 to +5% on others (the host takes this form
// only from about 32 items per CU, where it starts to win).
template <int RPI>
struct RowsItem {
    FastRsrc fb;
    Geo geo;  // nchunks: the item's chunks; blk: its first block's scale slot
    float sm[RPI], sv[RPI];
    float* m_scale;
    float* v_scale;
    int rot;  // always 0
    uint32_t lane0, step;
    int nrows;       // blocks in this item (RPI but at a segment's end)
    bool fast;       // all full rows, aligned: the item runs as one span
    bool staged_ok;  // and its span is a multiple of 16 elements
};

template <int T, int GPT, int RPI>
__device__ __forceinline__ RowsItem<RPI> rows_item(const StepArgs& a, uint32_t w, uint32_t nx, Seg& sg,
                                                   int64_t& lb, uint32_t& y) {
    constexpr int CH = kWgChunk;
    RowsItem<RPI> d;
    y = __builtin_amdgcn_readfirstlane(w / nx);
    int64_t local;
    sg = find_inline(a, w - y * nx, local);
    lb = local * RPI;
    const int64_t rem = sg.nblocks - lb;
    d.nrows = (int)(rem < RPI ? rem : RPI);
    ve_shard_state st;
    {
        const uint64_t* src = reinterpret_cast<const uint64_t*>(a.states + y);
        uint64_t* dst = reinterpret_cast<uint64_t*>(&st);
#pragma unroll
        for (int i = 0; i < 8; ++i) dst[i] = sload(src + i);
    }
    const Ptrs p = make_ptrs<true>(st, sg.tensor);
    const Geo g0 = block_geo<CH>(sg, lb);
    d.geo = g0;
    d.m_scale = st.m_scale;
    d.v_scale = st.v_scale;
#pragma unroll
    for (int r = 0; r < RPI; ++r) {
        d.sm[r] = r < d.nrows ? sload(st.m_scale + g0.blk + r) : 0.f;
        d.sv[r] = r < d.nrows ? sload(st.v_scale + g0.blk + r) : 0.f;
    }
    // full rows only: every block of the item holds block_rows whole rows
    const bool full = sg.tiles == 1 && (sg.panel0 + lb + d.nrows) * sg.block_rows <= sg.rows &&
                      g0.run == T * CH * (GPT / RPI);
    const int64_t span = (int64_t)d.nrows * g0.run;
    d.fast = full && p.aligned && ((g0.e0 | sg.shard_base | g0.run) & (CH - 1)) == 0 && span < kFastMaxSpan;
    d.staged_ok = d.fast && (g0.run & 15) == 0;
    d.geo.nchunks = (int32_t)(span / CH);
    d.rot = 0;
    d.lane0 = threadIdx.x * CH;
    d.step = T * CH;
    if (d.fast) {
        const int64_t s0 = sg.shard_base + g0.e0;
        d.fb.grad = buf_rsrc(p.grad + g0.e0, 2 * span);
        d.fb.grad_shard = buf_rsrc(p.grad_shard + s0, 2 * span);
        d.fb.master = buf_rsrc(p.master + s0, 4 * span);
        d.fb.m_q = buf_rsrc(p.m_q + s0, span);
        d.fb.v_q = buf_rsrc(p.v_q + s0, span);
        d.fb.param = buf_rsrc(p.param + s0, 2 * span);
    }
    return d;
}

// One item of RPI blocks as one span (see dyn_block): per-block absmax
// accumulators, reduction, scales and requantisation.
template <int T, int GPT, bool STAGED, int RPI>
__device__ __forceinline__ bool rows_block(const RowsItem<RPI>& it, const StepArgs& A, uint32_t nx, uint32_t nitems,
                                           RowsItem<RPI>& nt, uint32_t& wn, uint32_t* s_next, uint8_t* sb,
                                           float (&red)[2][RPI][T / 64],
                                           float (&mst)[DynCfg<T, GPT>::MA + 1][kWgChunk]) {
    constexpr int CH = kWgChunk;
    constexpr int MODE = kWgLinear;
    constexpr int SPR = GPT / RPI;  // register slots per block
    static_assert(SPR * RPI == GPT, "whole blocks per thread");
    constexpr int PF = DynCfg<T, GPT>::PF, SPAN = DynCfg<T, GPT>::SPAN, DMA_AT = DynCfg<T, GPT>::DMA_AT;
    constexpr int MA = DynCfg<T, GPT>::MA, MPRE = DynCfg<T, GPT>::MPRE;
    constexpr bool LATE = DynCfg<T, GPT>::LATE;
    const StepScalars& sc = A.sc;
    const int tid = threadIdx.x;
    In<CH> x[GPT];
    const uint32_t off[GPT] = {};  // unused by LINEAR addressing
#pragma unroll
    for (int c = 0; c < GPT; ++c) {
        const ChunkAddr ad = wg_addr<T, GPT, MODE>(it, off, c);
        if (!STAGED || c >= PF) load_in_fast(x[c], it.fb, ad);
        if (c < MA && !(STAGED && c < MPRE)) load_master_fast(mst[c % (MA + 1)], it.fb, ad);
        __builtin_amdgcn_sched_barrier(0);
    }
    uint32_t ticket = 0;
    if (tid == 0) ticket = atomicAdd(A.sched, 1u);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (STAGED) {
#pragma unroll
        for (int c = 0; c < PF; ++c) {
            const bool ok = tid < it.geo.nchunks - c * T;
            const uint2 g = *(const uint2*)(sb + c * T * 8 + tid * 8);
            const uint32_t m = *(const uint32_t*)(sb + 2 * SPAN + c * T * 4 + tid * 4);
            const uint32_t v = *(const uint32_t*)(sb + 3 * SPAN + c * T * 4 + tid * 4);
            x[c].g[0] = ok ? g.x : 0u;
            x[c].g[1] = ok ? g.y : 0u;
            x[c].m[0] = ok ? m : 0u;
            x[c].v[0] = ok ? v : 0u;
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    float am[RPI], av[RPI];
#pragma unroll
    for (int r = 0; r < RPI; ++r) am[r] = av[r] = 0.f;
#pragma unroll
    for (int c = 0; c < GPT; ++c) {
        if (c + MA < GPT) load_master_fast(mst[(c + MA) % (MA + 1)], it.fb, wg_addr<T, GPT, MODE>(it, off, c + MA));
        phase1_fast<LATE>(x[c], mst[c % (MA + 1)], it.fb, wg_addr<T, GPT, MODE>(it, off, c), it.sm[c / SPR],
                          it.sv[c / SPR], sc, am[c / SPR], av[c / SPR]);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = 0; r < RPI; ++r) {
        am[r] = wave_max(am[r]);
        av[r] = wave_max(av[r]);
        if ((tid & 63) == 0) {
            red[0][r][tid >> 6] = am[r];
            red[1][r][tid >> 6] = av[r];
        }
    }
    if (tid == 0) *s_next = ticket;
    lds_barrier();
    wn = *s_next;
    const bool more = wn < nitems;
    Seg nsg;
    int64_t nlb;
    uint32_t ny;
    nt = rows_item<T, GPT, RPI>(A, more ? wn : 0u, nx, nsg, nlb, ny);
    const bool stage_next = more && nt.staged_ok;
    float im[RPI], iv[RPI];
#pragma unroll
    for (int r = 0; r < RPI; ++r) {
        float bm = 0.f, bv = 0.f;
#pragma unroll
        for (int i = 0; i < T / 64; ++i) {
            bm = fmaxf(bm, red[0][r][i]);
            bv = fmaxf(bv, red[1][r][i]);
        }
        im[r] = bm > 0.f ? 127.0f / bm : 0.f;
        iv[r] = bv > 0.f ? 127.0f / bv : 0.f;
        if (tid == r && r < it.nrows) {
            ((VE_GLOBAL float*)it.m_scale)[it.geo.blk + r] = bm / 127.0f;
            ((VE_GLOBAL float*)it.v_scale)[it.geo.blk + r] = bv / 127.0f;
        }
    }
#pragma unroll
    for (int c = 0; c < GPT; ++c) {
        if (c == DMA_AT) {
            __builtin_amdgcn_sched_barrier(0);
            if (stage_next) {
                dyn_stage<T, GPT>(nt, sb);
#pragma unroll
                for (int c2 = 0; c2 < MPRE; ++c2)
                    load_master_fast(mst[c2 % (MA + 1)], nt.fb, wg_addr<T, GPT, MODE>(nt, off, c2));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        make_opaque(x[c]);
        phase2_fast<LATE>(x[c], it.fb, wg_addr<T, GPT, MODE>(it, off, c), it.sm[c / SPR], it.sv[c / SPR],
                          im[c / SPR], iv[c / SPR], sc);
        __builtin_amdgcn_sched_barrier(0);
    }
    return stage_next;
}

template <int T, int GPT, int RPI>
__global__ void __launch_bounds__(T) k_step_rows(StepArgs a, uint32_t nx, uint32_t nitems) {
    constexpr int GROUP_STORES = DynCfg<T, GPT>::LATE ? 3 : 2;  // phase-2 stores per group
    constexpr int AFTER_DMA = GROUP_STORES * (GPT - DynCfg<T, GPT>::DMA_AT);
    static_assert(AFTER_DMA <= 63, "vmcnt holds at most 63");
    __shared__ float s_red[2][RPI][T / 64];
    __shared__ float s_red1[2][T / 64];  // the block-by-block fallback's
    __shared__ uint32_t s_next;
    __shared__ __attribute__((aligned(16))) uint8_t s_buf[DynCfg<T, GPT>::LDS];
    float mst[DynCfg<T, GPT>::MA + 1][kWgChunk];  // master ring, carried from item to item
    if (threadIdx.x == 0) s_next = atomicAdd(a.sched, 1u);
    __syncthreads();
    uint32_t w = s_next;
    bool staged = false;
    while (w < nitems) {
        Seg sg;
        int64_t lb;
        uint32_t y;
        const RowsItem<RPI> it = rows_item<T, GPT, RPI>(a, w, nx, sg, lb, y);
        uint32_t wn;
        if (it.fast) {
            __builtin_amdgcn_sched_barrier(0);
            // as in k_step_dyn: wait for this wave's staging loads, then for every wave
            if (staged) __builtin_amdgcn_s_waitcnt(0x0F70 | (AFTER_DMA & 15) | (((AFTER_DMA >> 4) & 3) << 14));
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            RowsItem<RPI> nt;
            if (staged) staged = rows_block<T, GPT, true, RPI>(it, a, nx, nitems, nt, wn, &s_next, s_buf, s_red, mst);
            else staged = rows_block<T, GPT, false, RPI>(it, a, nx, nitems, nt, wn, &s_next, s_buf, s_red, mst);
        } else {
            // block by block through the workgroup code.  (With the general
            // form alone here the kernel spills no registers, yet runs 1.3%
            // slower on 8,192-element rows.)
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_s_barrier();
            if (threadIdx.x == 0) s_next = atomicAdd(a.sched, 1u);  // read after the blocks' barriers
            for (int r = 0; r < it.nrows; ++r) {
                const WgItem gi = wg_item_for<GPT>(a, y, sg, lb + r, lb + r);
                if (r > 0) __syncthreads();  // the previous block's reads of s_red1
                if (gi.mode == kWgLinear) wg_one<T, GPT, kWgLinear>(gi, s_red1, a.sc);
                else if (gi.mode == kWgTiled) wg_one<T, GPT, kWgTiled>(gi, s_red1, a.sc);
                else wg_one<T, GPT, kWgGeneral>(gi, s_red1, a.sc);
            }
            wn = s_next;
            staged = false;
        }
        w = wn;
    }
    // as in k_step_dyn: the last workgroup out resets the counters
    if (threadIdx.x == 0) {
        const uint32_t left = atomicAdd(a.sched + 1, 1u);
        if (left == gridDim.x - 1) {
            atomicExch(a.sched, 0u);
            atomicExch(a.sched + 1, 0u);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
static inline unsigned grid_x(int64_t n) { return (unsigned)n; }

hipError_t launch_step_small(const StepArgs& a0, int n_states, hipStream_t s) {
    StepArgs a = a0;
    a.pad_wg0 = (a.work.total + 3) / 4;
    const dim3 grid(grid_x(a.pad_wg0 + a.pad.n_tiles), n_states);
    if (a.n_inline > 0) hipLaunchKernelGGL(k_step_small<true>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_step_small<false>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int T, int GPT>
static hipError_t launch_wg_t(const StepArgs& a, int n_states, int dyn_cu, hipStream_t s) {
    if constexpr (dyn_shape(T, GPT)) {
        if (dyn_cu > 0) {
            // resident workgroups per CU of the persistent kernel (its LDS and
            // registers decide), read once per process
            static const int occ = [] {
                int n = 0;
                if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_step_dyn<T, GPT>, T, 0) != hipSuccess || n < 1)
                    n = 1;
                return n < kDynMaxPerCu ? n : kDynMaxPerCu;
            }();
            const int64_t items = a.work.total * n_states;
            const int64_t grid = std::min<int64_t>(items, (int64_t)dyn_cu * occ);
            hipLaunchKernelGGL((k_step_dyn<T, GPT>), dim3((unsigned)grid), dim3(T), 0, s, a, (uint32_t)a.work.total,
                               (uint32_t)items);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((k_step_wg<T, GPT>), dim3(grid_x(a.work.total), n_states), dim3(T), 0, s, a);
    return hipGetLastError();
}

// Resident workgroups per CU of a persistent item kernel (its LDS and
// registers decide), at most kDynMaxPerCu.
template <class K>
static int item_occupancy(K kernel) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kItemThreads, 0) != hipSuccess || n < 1) n = 1;
    return n < kDynMaxPerCu ? n : kDynMaxPerCu;
}

hipError_t launch_step_items(const StepArgs& a, int n_states, int form, int dyn_cu, hipStream_t s) {
    constexpr int T = kItemThreads, G = kItemGpt;
    if (dyn_cu < 1) return hipErrorInvalidValue;
    const int64_t items = a.work.total * n_states;
    const uint32_t nx = (uint32_t)a.work.total, ni = (uint32_t)items;
    auto grid = [&](int occ) { return dim3((unsigned)std::min<int64_t>(items, (int64_t)dyn_cu * occ)); };
    if (form == kItemRows4) {
        static const int occ = item_occupancy(k_step_rows<T, G, 4>);
        hipLaunchKernelGGL((k_step_rows<T, G, 4>), grid(occ), dim3(T), 0, s, a, nx, ni);
    } else if (form == kItemRows2) {
        static const int occ = item_occupancy(k_step_rows<T, G, 2>);
        hipLaunchKernelGGL((k_step_rows<T, G, 2>), grid(occ), dim3(T), 0, s, a, nx, ni);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

bool wg_config_supported(int threads, int gpt) {
#define VE_WG_CASE(T, G) if (threads == T && gpt == G) return true;
    VE_WG_SHAPES(VE_WG_CASE)
#undef VE_WG_CASE
    return false;
}

bool wg_dynamic_shape(int threads, int gpt) { return dyn_shape(threads, gpt); }

hipError_t launch_step_wg(const StepArgs& a, int n_states, int threads, int gpt, int dyn_grid, hipStream_t s) {
#define VE_WG_CASE(T, G) if (threads == T && gpt == G) return launch_wg_t<T, G>(a, n_states, dyn_grid, s);
    VE_WG_SHAPES(VE_WG_CASE)
#undef VE_WG_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_step_huge(const StepArgs& a, int n_states, hipStream_t s) {
    hipLaunchKernelGGL(k_step_huge, dim3(grid_x(a.work.total), n_states), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_runs_copy(const RunArgs& r, const uint16_t* const* grad_ptrs, uint16_t* out, hipStream_t s) {
    hipLaunchKernelGGL(k_runs, dim3(grid_x(r.n_tiles), 1), dim3(256), 0, s, r, grad_ptrs, out,
                       (const ve_shard_state*)nullptr, 0);
    return hipGetLastError();
}

hipError_t launch_runs_pad(const RunArgs& r, const ve_shard_state* states, int n_states, hipStream_t s) {
    hipLaunchKernelGGL(k_runs, dim3(grid_x(r.n_tiles), n_states), dim3(256), 0, s, r,
                       (const uint16_t* const*)nullptr, (uint16_t*)nullptr, states, 1);
    return hipGetLastError();
}

}  // namespace ve
