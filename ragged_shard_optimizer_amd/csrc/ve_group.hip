// ve_group.hip -- DBuffer group operations: zero, scale, accumulate.
//
// The DBuffer applies one operation to all of its tensors in one pass
// (veScale-FSDP talk notes, "3. DBuffer"; Dutch summary, "C. Distributed
// Buffer": identical operations such as add, scale and zero are fused across
// tensors).  Here one launch covers a rank chunk or a whole bucket, for any
// number of buckets that share a plan (grid.y), over the same run tables as
// the group copy-in: each run is a tensor piece (dst in the bucket, src in
// the tensor) or padding.
//
// Element arithmetic, fp32: the bf16 operands are widened exactly, one IEEE
// operation is applied (scale: alpha*x; accumulate: fma(alpha, g, x), one
// rounding) and the result is rounded to bf16 to nearest even
// (v_cvt_pk_bf16_f32).  Padding is written 0.
//
// Bound: HBM.  Algorithmic bytes per tensor element: zero 2 (write), scale 4
// (read + write), accumulate 6 (bucket read + write, gradient read); 2 per
// padding element (write).  A tile is up to 4096 elements of one run, cut at
// 128-byte positions of the bucket (run_tile_span); a thread
// moves two 16-byte vectors, lane-contiguous, so every wave access covers
// 1 KB of whole cache lines and carries the streaming hint.  A tile whose
// bucket or gradient address is not 16-byte aligned (ragged pieces of 1-D
// tensors) falls back to 2-byte accesses, still lane-contiguous.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ve_device.h"
#include "ve_internal.h"

namespace ve {
namespace {

template <int OP>
__device__ __forceinline__ float apply(float x, float g, float alpha) {
    if constexpr (OP == VE_GROUP_SCALE) return alpha * x;
    else return __builtin_fmaf(alpha, g, x);
}

// Two bf16 elements per dword.
template <int OP>
__device__ __forceinline__ uint32_t apply2(uint32_t x, uint32_t g, float alpha) {
    return pack_bf16x2(apply<OP>(bf_lo(x), bf_lo(g), alpha), apply<OP>(bf_hi(x), bf_hi(g), alpha));
}

template <int OP>
__global__ void __launch_bounds__(256) k_group(RunArgs r, const ve_group_operand* ops, float alpha) {
    constexpr int V = 8;                        // bf16 per 16-byte vector
    constexpr int PER = kRunTile / (256 * V);   // vectors per thread
    constexpr bool NT = VE_NONTEMPORAL;
    const int tid = threadIdx.x;
    const int64_t tile = blockIdx.x;
    const int ri = r.tile_run[tile];
    const Run rn = r.runs[ri];
    int64_t t0, n;
    run_tile_span(rn.dst, rn.len, tile - r.tile_prefix[ri], t0, n);
    const int len = (int)n;
    const ve_group_operand od = ops[blockIdx.y];
    VE_GLOBAL uint16_t* d = (VE_GLOBAL uint16_t*)(od.bucket + rn.dst + t0);
    // zero, and padding under every op: plain fill, nothing read
    const bool fill = OP == VE_GROUP_ZERO || rn.tensor < 0;
    const VE_GLOBAL uint16_t* g = nullptr;
    if (OP == VE_GROUP_ACCUMULATE && !fill) {
        // wave-uniform, read-only for the kernel's lifetime: a scalar load
        const uint64_t gp = ((const __attribute__((address_space(4))) uint64_t*)od.grad_ptrs)[rn.tensor];
        g = (const VE_GLOBAL uint16_t*)gp + rn.src + t0;
    }
    const bool vec = ((((uintptr_t)d) | ((uintptr_t)g)) & 15) == 0;
    const int nvec = vec ? len / V : 0;

    if (nvec > 0) {
        u32x4 xv[PER], gv[PER];
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            xv[q] = u32x4{0, 0, 0, 0};
            gv[q] = u32x4{0, 0, 0, 0};
            const int v = q * 256 + tid;
            if (!fill && v < nvec) {
                xv[q] = ldv<NT>((const VE_GLOBAL u32x4*)(d + v * V));
                if (OP == VE_GROUP_ACCUMULATE) gv[q] = ldv<NT>((const VE_GLOBAL u32x4*)(g + v * V));
            }
        }
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int v = q * 256 + tid;
            if (v >= nvec) break;
            u32x4 y = u32x4{0, 0, 0, 0};
            if (!fill) {
                y.x = apply2<OP>(xv[q].x, gv[q].x, alpha);
                y.y = apply2<OP>(xv[q].y, gv[q].y, alpha);
                y.z = apply2<OP>(xv[q].z, gv[q].z, alpha);
                y.w = apply2<OP>(xv[q].w, gv[q].w, alpha);
            }
            stv<NT>((VE_GLOBAL u32x4*)(d + v * V), y);
        }
    }
    // what the vectors did not cover: the run's last partial vector, or the
    // whole tile when an address is misaligned
    for (int i = nvec * V + tid; i < len; i += 256) {
        uint16_t y = 0;
        if (!fill) {
            const uint32_t x = d[i];
            const uint32_t gg = OP == VE_GROUP_ACCUMULATE ? (uint32_t)g[i] : 0u;
            y = (uint16_t)apply2<OP>(x, gg, alpha);   // low half: the element itself
        }
        d[i] = y;
    }
}

}  // namespace

hipError_t launch_group(const RunArgs& r, int op, float alpha, const ve_group_operand* ops, int n_ops,
                        hipStream_t s) {
    const dim3 grid((unsigned)r.n_tiles, (unsigned)n_ops);
    switch (op) {
        case VE_GROUP_ZERO:
            hipLaunchKernelGGL(k_group<VE_GROUP_ZERO>, grid, dim3(256), 0, s, r, ops, alpha);
            break;
        case VE_GROUP_SCALE:
            hipLaunchKernelGGL(k_group<VE_GROUP_SCALE>, grid, dim3(256), 0, s, r, ops, alpha);
            break;
        case VE_GROUP_ACCUMULATE:
            hipLaunchKernelGGL(k_group<VE_GROUP_ACCUMULATE>, grid, dim3(256), 0, s, r, ops, alpha);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ve
