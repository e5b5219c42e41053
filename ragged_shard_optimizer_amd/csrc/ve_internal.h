// ve_internal.h -- tables shared by the host side of libve and its kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ve.h"

namespace ve {

// Elements per lane-chunk: 4 on both paths (a dword of codes, 8 bytes of
// bf16, 16 bytes of fp32 per lane, so that the 64 lanes of a wave touch one
// contiguous span per access).  Small blocks are latency-bound (a ragged
// rank holds ~700 K elements), and 4-element chunks give them four times the
// waves of 16-element ones.  The small-block code also takes 16-element
// chunks (kernel helpers are written for both).
constexpr int kSmallChunk = 4;
constexpr int kWgChunk = 4;
// A block with at most this many chunks (256 elements) is handled by a group of
// <= 64 lanes of one wave (one chunk per lane); larger blocks take a whole
// workgroup.
constexpr int kSmallMaxChunks = 64;
constexpr int kWgMaxThreads = 1024;
// Workgroup shapes of the step that run in the persistent form (one
// workgroup per CU taking blocks from a ticket counter).
constexpr bool dyn_shape(int threads, int gpt) {
    // (1024 x 12 and more spill registers in that form)
    return (threads == 512 && gpt >= 14) || threads == 768 || (threads == 1024 && gpt >= 7 && gpt <= 10);
}
constexpr size_t kSchedStride = 64;  // bytes of scheduler counters per rank in a plan's device tables

// Instantiated workgroup shapes (threads, 4-element groups per thread).  The
// largest capacity, 1024 x 16 groups = 65,536 elements, bounds the blocks
// held in registers; larger blocks take the two-pass path.
#define VE_WG_SHAPES(X)                                                                         \
    X(256, 1) X(256, 2) X(256, 4) X(256, 8) X(256, 12) X(256, 16) X(256, 24) X(256, 32)         \
    X(512, 2) X(512, 4) X(512, 6) X(512, 8) X(512, 10) X(512, 12) X(512, 14) X(512, 16)         \
    X(512, 20) X(512, 24)                                                                       \
    X(768, 10) X(768, 15)                                                                       \
    X(1024, 2) X(1024, 4) X(1024, 6) X(1024, 7) X(1024, 8) X(1024, 10) X(1024, 12) X(1024, 14) X(1024, 16)
constexpr int64_t kWgMaxGroups = 1024 * 16;
// The workgroup-path kernels take their segment table in the kernel
// arguments (read through the scalar cache), so a workgroup finds its block
// without a dependent chain of memory loads; a class with more segments is
// launched in slices of at most this many.
constexpr int kInlineSegs = 16;
// Elements per tile of the run copier (copy-in, padding fill, group ops).
#ifndef VE_RUN_TILE
#define VE_RUN_TILE 4096
#endif
constexpr int kRunTile = VE_RUN_TILE;
// Tiles are cut at multiples of kRunAlign elements of the destination (128
// bytes of bf16), so that no cache line is written by two workgroups (which
// run on different XCDs, whose L2s would each write back a partial line):
// the first tile of a run is short by the run's offset mod kRunAlign.
constexpr int kRunAlign = 64;
__host__ __device__ inline int64_t run_head(int64_t dst) { return dst & (kRunAlign - 1); }
__host__ __device__ inline int64_t run_tiles(int64_t dst, int64_t len) {
    return len <= 0 ? 0 : (len + run_head(dst) + kRunTile - 1) / kRunTile;
}
// Tile j of a run covers run elements [t0, t0 + n), 0 < n <= kRunTile.
__host__ __device__ inline void run_tile_span(int64_t dst, int64_t len, int64_t j, int64_t& t0, int64_t& n) {
    const int64_t h = run_head(dst);
    const int64_t end = (j + 1) * kRunTile - h;
    t0 = j == 0 ? 0 : j * kRunTile - h;
    n = (end < len ? end : len) - t0;
}
// A dispatch's grid is at most 2^32 - 1 work-items per dimension.
constexpr int64_t kMaxGridItems = 0xFFFFFFFFll;
constexpr int64_t kMaxRunTiles = kMaxGridItems / 256;  // run kernels: 256 threads per tile

// kUnit: one-element blocks (a block's maximum is the element itself), on
// the small-block work list with kUnitPerWave blocks per wave item.
enum SegClass : int32_t { kSmall = 0, kWg = 1, kHuge = 2, kUnit = 3 };
constexpr int kUnitPerWave = 64 * kSmallChunk;

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
    int32_t max_chunks;  // small-path chunks of a full block
    int32_t max_groups;  // 4-element groups of a full block (workgroup path)
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

struct RunArgs {
    const Run* runs;              // device
    const int64_t* tile_prefix;   // device, n_runs + 1
    const int32_t* tile_run;      // device, one run index per tile
    int32_t n_runs;
    int64_t n_tiles;
};

struct StepArgs {
    const ve_shard_state* states;  // device [n_states]
    const Seg* segs;               // device, this rank's segments
    WorkList work;
    StepScalars sc;
    RunArgs pad;                   // small-block path: padding tiles fused into the launch (n_tiles 0: none)
    int64_t pad_wg0;               // small-block path: first workgroup of the padding tiles
    uint32_t* sched;               // workgroup path, persistent form: [next ticket, workgroups done], zero between launches
    int32_t n_inline;              // workgroup paths: segments given inline below
    int64_t inl_prefix[kInlineSegs + 1];  // work-item prefix, inl_prefix[0] = 0
    Seg inl_segs[kInlineSegs];
};


// Launchers (ve_kernels.hip).  Return the hipError_t of the launch.
// Small-block step; a.pad's tiles (zero fill of grad_shard and param_shard)
// run as extra workgroups of the same launch.
hipError_t launch_step_small(const StepArgs& a, int n_states, hipStream_t s);
// dyn_cu > 0 (the device's CU count) runs a shape that wg_dynamic_shape()
// accepts in its persistent form, as many workgroups as the CUs hold at once
// (at most kDynMaxPerCu per CU), scheduled through a.sched.
hipError_t launch_step_wg(const StepArgs& a, int n_states, int threads, int groups_per_thread, int dyn_cu,
                          hipStream_t s);
constexpr int kDynMaxPerCu = 8;
// Work a launch needs for the persistent forms (option wg_dynamic = 1):
// blocks per CU for the row-block form, items per CU for row items.
constexpr int kDynMinPerCu = 5, kItemMinPerCu = 32;
bool wg_dynamic_shape(int threads, int groups_per_thread);
// Persistent form over items of several blocks, 8,192 groups an item, in
// kItemThreads x kItemGpt workgroups: 2 or 4 consecutive whole-row blocks
// of 4,096 or 2,048 groups (kItemRows2 / kItemRows4).  a.inl_prefix counts
// items, a.sched as above, dyn_cu > 0.
constexpr int kItemThreads = 1024, kItemGpt = 8, kItemGroups = kItemThreads * kItemGpt;
enum ItemForm : int { kItemNone = 0, kItemRows2 = 2, kItemRows4 = 4 };
constexpr int item_blocks(int form) { return form; }
hipError_t launch_step_items(const StepArgs& a, int n_states, int form, int dyn_cu, hipStream_t s);
hipError_t launch_step_huge(const StepArgs& a, int n_states, hipStream_t s);
// Copy-in: out = bucket; grad pointers from `grad_ptrs`.
hipError_t launch_runs_copy(const RunArgs& r, const uint16_t* const* grad_ptrs, uint16_t* out,
                            hipStream_t s);
// Padding fill of the step: zero grad_shard and param_shard of every state.
hipError_t launch_runs_pad(const RunArgs& r, const ve_shard_state* states, int n_states,
                           hipStream_t s);

// Process-wide launch options (ve_set_option / ve_get_option; each starts
// from its environment variable, read once, else its default).
enum Option : int {
    kOptWgThreads = 0,  // "wg_threads" (VE_WG_THREADS): step workgroup threads, 0 = by block size
    kOptWgGpt,          // "wg_gpt" (VE_WG_GPT): step groups per thread, 0 = by block size
    kOptGemmSplit,      // "gemm_split" (VE_GEMM_SPLIT): 0 = never split a product's short last round
    kOptGemmCfg,        // "gemm_cfg" (VE_GEMM_CFG): product configuration, -1 = by shape
    kOptGemmXcd,        // "gemm_xcd" (VE_GEMM_XCD): 0 = plain tile order instead of the XCD-aware one
    kOptWgDynamic,      // "wg_dynamic" (VE_WG_DYNAMIC): 0 = one-shot launches only; 1 = persistent forms where a
                        // launch has enough work; 2 = persistent forms whatever the work
    kOptWgRows,         // "wg_rows" (VE_WG_ROWS): 0 = no multi-block items for blocks of 2,048 / 4,096 groups
    kNumOptions
};
int64_t option(Option o);

// Record the thread-local message ve_last_error() returns; returns `st`.
ve_status fail(ve_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// DBuffer group operation `op` (a ve_group_op) over the run tiles, for
// ops[0 .. n_ops) (ve_group.hip).
hipError_t launch_group(const RunArgs& r, int op, float alpha, const ve_group_operand* ops, int n_ops,
                        hipStream_t s);

// Streaming copy of `vectors` 16-byte vectors with `grid` workgroups of 256
// threads (ve_stream.hip).
hipError_t launch_stream_copy(const void* src, void* dst, int64_t vectors, int grid, hipStream_t s);

// (threads, groups per thread) pairs instantiated for the workgroup path.
bool wg_config_supported(int threads, int groups_per_thread);

}  // namespace ve
