// ve_stream.hip -- plain device-to-device copy with 16-byte non-temporal
// accesses: the streaming reference the HBM-bound kernels of this library
// are measured against (read + write bytes over its time is the practical
// bandwidth of one MI355X for a 1:1 read/write mix).
//
// Every thread moves four 16-byte vectors per sweep, lane-contiguous, so
// each wave access covers 1 KB of whole cache lines; the grid strides over
// the buffer.  Measured on MI355X the rate depends on how far the sweep
// fronts of a grid-stride loop drift apart over a long buffer: a 1 GiB copy
// reaches ~5.9 TB/s in one launch, larger single launches less, and the
// same bytes cut into launches of 256 MiB ~6.1 TB/s.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ve_device.h"
#include "ve_internal.h"

namespace ve {
namespace {

constexpr int kCopyUnroll = 4;

__global__ void __launch_bounds__(256) k_stream_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                     int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * 256 * kCopyUnroll;
    for (int64_t i = (int64_t)blockIdx.x * 256 * kCopyUnroll + threadIdx.x; i < n; i += stride) {
        u32x4 v[kCopyUnroll];
#pragma unroll
        for (int k = 0; k < kCopyUnroll; ++k)
            if (i + k * 256 < n) v[k] = ldv<true>((const VE_GLOBAL u32x4*)src + i + k * 256);
#pragma unroll
        for (int k = 0; k < kCopyUnroll; ++k)
            if (i + k * 256 < n) stv<true>((VE_GLOBAL u32x4*)dst + i + k * 256, v[k]);
    }
}

}  // namespace

hipError_t launch_stream_copy(const void* src, void* dst, int64_t vectors, int grid, hipStream_t s) {
    hipLaunchKernelGGL(k_stream_copy, dim3(grid), dim3(256), 0, s, (const u32x4*)src, (u32x4*)dst, vectors);
    return hipGetLastError();
}

}  // namespace ve
