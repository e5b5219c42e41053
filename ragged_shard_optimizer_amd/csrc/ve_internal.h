// ve_internal.h -- tables shared by the host side of libve and its kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ve.h"

namespace ve {

// Elements per chunk: the unit a lane moves with 16-byte vector accesses
// (16 int8 codes, 2 x 8 bf16, 4 x 4 fp32).
constexpr int kChunk = 16;
// A block with at most this many chunks is handled by a group of <= 64 lanes
// of one wave (one chunk per lane); larger blocks take a whole workgroup.
constexpr int kSmallMaxChunks = 64;
// Largest chunks-per-thread instantiation of the workgroup path.
constexpr int kWgMaxChunksPerThread = 12;
constexpr int kWgMaxThreads = 1024;
// Entries of a work-prefix table staged in LDS (larger tables are searched
// in global memory).
constexpr int kLdsPrefixCap = 2048;
// Elements per tile of the run copier (copy-in and padding fill).
constexpr int kRunTile = 4096;

enum SegClass : int32_t { kSmall = 0, kWg = 1, kHuge = 2 };

// One tensor piece on one rank ("segment"), in device-visible form.
struct Seg {
    int64_t shard_base;  // shard coordinate of tensor element 0 (may be < 0)
    int64_t elem_lo;     // piece = tensor elements [elem_lo, elem_hi)
    int64_t elem_hi;
    int64_t rows, cols;
    int64_t block_rows, block_cols;
    int64_t panel0;      // first row panel of the piece
    int64_t block0;      // rank-local index of the piece's first block
    int64_t nblocks;     // panels * tiles
    int32_t tensor;      // index into the caller's tensor list / grad_ptrs
    int32_t tiles;       // tiles per panel = cols / block_cols
    int32_t cls;         // SegClass
    int32_t group;       // small path: lanes per block (power of two <= 64)
    int32_t max_chunks;  // chunks of a full block
    int32_t pad_;
};

// A contiguous copy (tensor >= 0) or zero fill (tensor == -1) of `len`
// elements to output position `dst`, reading tensor elements from `src`.
struct Run {
    int64_t dst;
    int64_t src;
    int64_t len;
    int32_t tensor;
    int32_t pad_;
};

// A class-homogeneous work list on one rank: work item w belongs to
// seg_idx[i] where prefix[i] <= w < prefix[i+1].
struct WorkList {
    const int32_t* seg_idx;  // device
    const int64_t* prefix;   // device, n + 1 entries
    int32_t n;
    int64_t total;           // prefix[n]
};

// Per-step scalars, computed on the host in double and rounded once.
struct StepScalars {
    float beta1, beta2, omb1, omb2;  // omb = 1 - beta (exact in fp32)
    float step_size;                 // lr / (1 - beta1^t)
    float inv_sqrt_bc2;              // 1 / sqrt(1 - beta2^t)
    float eps;
    float decay;                     // 1 - lr * weight_decay
};

struct StepArgs {
    const ve_shard_state* states;  // device [n_states]
    const Seg* segs;               // device, this rank's segments
    WorkList work;
    StepScalars sc;
};

struct RunArgs {
    const Run* runs;              // device
    const int64_t* tile_prefix;   // device, n_runs + 1
    const int32_t* tile_run;      // device, one run index per tile
    int32_t n_runs;
    int64_t n_tiles;
};

// Launchers (ve_kernels.hip).  Return the hipError_t of the launch.
hipError_t launch_step_small(const StepArgs& a, int n_states, hipStream_t s);
hipError_t launch_step_wg(const StepArgs& a, int n_states, int threads, int chunks_per_thread,
                          hipStream_t s);
hipError_t launch_step_huge(const StepArgs& a, int n_states, hipStream_t s);
// Copy-in: out = bucket; grad pointers from `grad_ptrs`.
hipError_t launch_runs_copy(const RunArgs& r, const uint16_t* const* grad_ptrs, uint16_t* out,
                            hipStream_t s);
// Padding fill of the step: zero grad_shard and param_shard of every state.
hipError_t launch_runs_pad(const RunArgs& r, const ve_shard_state* states, int n_states,
                           hipStream_t s);

// (threads, chunks per thread) pairs instantiated for the workgroup path.
bool wg_config_supported(int threads, int chunks_per_thread);

}  // namespace ve
