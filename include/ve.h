/*
 * ve.h -- C ABI of the MI355X RaggedShard shard-step library (libve.so).
 *
 * The library runs the data-parallel hot path of veScale-FSDP ("veScale-FSDP:
 * Flexible and High-Performance FSDP at Scale") on one rank's slice of a
 * planned DBuffer bucket:
 *
 *   1. group copy-in of per-parameter bf16 gradients into the flat, padded
 *      bucket slice (talk notes, "3. DBuffer": tensors enter the buffer
 *      through group-level operators, zero-copy);
 *   2. a block-wise 8-bit AdamW step on the local shard, one absmax scale per
 *      RaggedShard quantisation block, so no rank needs another rank's data
 *      (talk notes, "1. RaggedShard": sync-free block-wise quantisation;
 *      "Case study: 8-bit Adam and distributed Muon");
 *   3. write-back of the bf16 parameter shard for the next all-gather;
 *
 * and the DBuffer's other group operations (zero, scale, accumulate) over a
 * rank chunk or a whole bucket, the structure-aware planner that produces
 * bucket layouts (host only), and Muon's Newton-Schulz iteration on one
 * gathered matrix (MFMA).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Bucket: m = fsdp_size equal chunks of S = shard_elems elements; rank r
 *    owns bucket elements [r*S, (r+1)*S) ("shard coordinates" 0..S-1).
 *    Equal chunks are what in-place all-gather / reduce-scatter need
 *    (talk notes, "3. DBuffer").
 *  - Tensor k is a row-major rows x cols matrix (1-D: numel x 1) stored
 *    contiguously at bucket elements [offset, offset + rows*cols).  Padding
 *    exists only between tensors (talk notes, "2. Structure-aware planning";
 *    Dutch summary, "2B").
 *  - RaggedShard block of tensor k: the shard unit is a row panel of
 *    block_rows rows (block_rows*cols elements); a chunk boundary may cut a
 *    tensor only at a unit boundary.  The quantisation block is the
 *    block_rows x block_cols tile inside a panel (block_cols divides cols;
 *    block_cols == cols gives whole-row blocks).  A last panel with fewer
 *    than block_rows rows is a shorter block with its own scale.
 *  - Piece: tensor k's intersection with rank r's chunk, tensor elements
 *    [elem_start, elem_end), stored at shard coordinates
 *    [shard_offset, shard_offset + elem_end - elem_start).
 *  - Rank-local block order (index into m_scale / v_scale): pieces by
 *    ascending bucket offset; inside a piece, panels top to bottom, and
 *    inside a panel, tiles left to right.  B_r is the rank's block count.
 *  - Pointers named "device" are device (or managed) memory on the plan's
 *    device; "host" pointers are host memory.  The caller owns every data
 *    buffer and pointer table; the library never allocates or copies per
 *    call.  Device arrays of pointers cannot be inspected from the host:
 *    entries the call reads must be valid, or the kernel faults.
 *  - Streams: `stream` is a hipStream_t (NULL = the null stream).  No call
 *    synchronises; device-side faults surface at the caller's next sync.
 *  - Errors: every entry point returns a ve_status; on failure
 *    ve_last_error() returns a thread-local message.  No C++ exception
 *    crosses the ABI.  A call rejected by its argument checks has launched
 *    nothing; a VE_ERR_DEVICE from a launch may leave earlier launches of
 *    the same call queued.
 *  - Concurrency: a loaded plan is immutable; calls on different streams
 *    with disjoint output buffers may overlap.
 */
#ifndef VE_H
#define VE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    VE_OK = 0,
    VE_ERR_INVALID_ARG = 1,  /* NULL / out-of-range argument */
    VE_ERR_LAYOUT = 2,       /* the bucket layout breaks a RaggedShard invariant */
    VE_ERR_OOM = 3,          /* device allocation for the plan tables failed */
    VE_ERR_DEVICE = 4,       /* a HIP runtime call or kernel launch failed */
    VE_ERR_UNSUPPORTED = 5   /* valid layout outside this build's limits */
} ve_status;

typedef struct ve_plan ve_plan; /* opaque; created by ve_plan_load */

/* One tensor of the bucket (any order; the library sorts by offset). */
typedef struct {
    int64_t rows, cols;             /* dim 0 and prod(dims[1:]); both >= 1 */
    int64_t block_rows, block_cols; /* RaggedShard block: >= 1, block_cols | cols */
    int64_t offset;                 /* first element's bucket offset */
} ve_tensor_spec;

/* AdamW hyper-parameters (fp32, as the step consumes them). */
typedef struct {
    float lr, beta1, beta2, eps, weight_decay;
} ve_adam_hparams;

/* One bucket's buffers on one rank.  All members are device pointers.
 * Arrays of S elements must be 16-byte aligned for the vector path (any
 * alignment is correct, misaligned ones are slower). */
typedef struct {
    const uint16_t* const* grad_ptrs; /* device array [n_tensors] of bf16 gradient
                                         pointers, tensor k's element e at
                                         grad_ptrs[k][e]; entries of tensors without
                                         a piece on the rank are not read (may be NULL) */
    uint16_t* grad_shard;  /* bf16 [S] out: copied-in gradient slice, padding 0 */
    float* master;         /* fp32 [S] in/out: master weights (padding untouched) */
    int8_t* m_q;           /* int8 [S] in/out: first-moment codes */
    int8_t* v_q;           /* int8 [S] in/out: second-moment codes (0..127) */
    float* m_scale;        /* fp32 [B_r] in/out: first-moment block scales */
    float* v_scale;        /* fp32 [B_r] in/out: second-moment block scales */
    uint16_t* param_shard; /* bf16 [S] out: RNE(master), padding 0 */
} ve_shard_state;

/* Validate a bucket layout and upload its per-rank segment tables to
 * `device` (host specs[n_tensors]).  Checks: shapes and blocks positive,
 * block_cols | cols; tensors disjoint and inside [0, fsdp_size*shard_elems);
 * every chunk boundary inside a tensor on a unit boundary (talk notes,
 * "1. RaggedShard").  VE_ERR_LAYOUT names the tensor and boundary that
 * fail.  VE_ERR_UNSUPPORTED: a block of more than 2^30 elements.
 * device == -1 builds a host-only plan: validation, ve_plan_query and
 * ve_dbuffer_slice work, kernel entry points return VE_ERR_INVALID_ARG.
 * The device tables also hold 64 bytes of step scheduler counters per rank.
 * On success *out owns the tables until ve_plan_free. */
ve_status ve_plan_load(const ve_tensor_spec* specs, int32_t n_tensors, int32_t fsdp_size,
                       int64_t shard_elems, int32_t device, ve_plan** out);

/* Release a plan (NULL is a no-op).  No call may still be using it. */
ve_status ve_plan_free(ve_plan* plan);

/* Per-rank sizes (host outputs; any may be NULL): valid elements, B_r, and
 * the number of pieces. */
ve_status ve_plan_query(const ve_plan* plan, int32_t rank, int64_t* valid_elems,
                        int64_t* n_blocks, int32_t* n_segments);

/* Group copy-in (talk notes, "3. DBuffer").  rank >= 0: bucket is bf16 [S],
 * receives rank's pieces at their shard coordinates; rank == -1: bucket is
 * bf16 [fsdp_size*S], receives every tensor.  Padding is written as 0.
 * grad_ptrs: device array as in ve_shard_state. */
ve_status ve_dbuffer_copy_in(const ve_plan* plan, int32_t rank, const uint16_t* const* grad_ptrs,
                             uint16_t* bucket, void* stream);

/* The fused shard step on `rank` for n_states buckets that share this plan
 * (states is a DEVICE array [n_states]; a few launches on `stream`: one per
 * workgroup block shape among the rank's pieces, one for small blocks that
 * also zero-fills the padding, one per slice of blocks too large for
 * registers, and a separate padding fill when there are no small blocks).
 * For every
 * piece element: copy the gradient into grad_shard, dequantise the moments
 * with the block's stored scales, update the Adam moments, update master
 * with decoupled weight decay and bias correction for step `step` (>= 1),
 * write param_shard = bf16_rne(master); then requantise each block's fresh
 * moments with a new absmax scale (scale = amax/127, code =
 * clamp(rint(x*127/amax), -127, 127); amax 0 gives scale 0 and code 0).
 * Padding of grad_shard and param_shard is written 0; master and the codes
 * at padding are not touched.
 * Blocks of the row-block shapes and row items (see the options "wg_dynamic"
 * and "wg_rows") are handed out to persistent workgroups by
 * two counters that the plan holds per rank (zero between launches), which
 * admit one launch at a time: a call for a rank on another stream than the
 * rank's previous such call first waits, on the GPU, for that call (the
 * library records an event after each call; host threads are serialised
 * per plan).  Calls for different ranks or plans are not ordered.  Under
 * stream capture nothing is recorded or waited on: replays of a captured
 * step must not overlap other calls for the same plan and rank.  With the
 * option "wg_dynamic" at 0 the step uses no counters. */
ve_status ve_shard_adam8bit_step(const ve_plan* plan, int32_t rank, const ve_shard_state* states,
                                 int32_t n_states, const ve_adam_hparams* hp, int64_t step,
                                 void* stream);

/* Zero-copy extraction (talk notes, "3. DBuffer"; Korean summary, "2.3"):
 * where tensor `tensor`'s piece on `rank` sits (host outputs).  rank == -1
 * refers to the whole bucket (shard_offset = offset, [0, numel)).  If the
 * rank holds none of the tensor: *shard_offset = -1, *elem_start =
 * *elem_end = 0 and VE_OK. */
ve_status ve_dbuffer_slice(const ve_plan* plan, int32_t rank, int32_t tensor,
                           int64_t* shard_offset, int64_t* elem_start, int64_t* elem_end);

/* DBuffer group operations: one operation applied to every tensor of a
 * chunk (or of the whole bucket) in one launch, the way the DBuffer fuses
 * identical operations such as add, scale and zero across its tensors
 * (talk notes, "3. DBuffer"; Dutch summary, "C. Distributed Buffer"). */
typedef enum {
    VE_GROUP_ZERO = 0,       /* x = 0 on every element, padding included */
    VE_GROUP_SCALE = 1,      /* x = alpha * x on tensor elements (e.g. averaging) */
    VE_GROUP_ACCUMULATE = 2  /* x = x + alpha * g on tensor elements (gradient accumulation) */
} ve_group_op;

/* One bucket operand of a group operation.  Both members are device pointers. */
typedef struct {
    uint16_t* bucket;                 /* bf16 [S] (rank >= 0) or [fsdp_size*S] (rank == -1), in/out */
    const uint16_t* const* grad_ptrs; /* VE_GROUP_ACCUMULATE: device array as in ve_shard_state
                                         (tensor k's element e at grad_ptrs[k][e]; entries of
                                         tensors without a piece in the range may be NULL);
                                         ignored by the other operations (may be NULL) */
} ve_group_operand;

/* Apply `op` to n_operands buckets that share this plan (operands is a
 * DEVICE array [n_operands]; one launch).  rank >= 0: each bucket is rank's
 * chunk, bf16 [S]; rank == -1: the whole bucket, bf16 [fsdp_size*S].
 * Arithmetic per tensor element, in fp32: the bf16 operands are widened,
 * one IEEE operation is applied (scale: the product alpha*x; accumulate: the
 * fused multiply-add fma(alpha, g, x), one rounding) and the result is
 * stored as bf16, rounded to nearest even.  Padding is written 0 by every
 * operation.  NaN inputs give NaN outputs (payload unspecified).  Buckets
 * must not overlap each other or the gradients.  Errors: unknown op, rank
 * out of [-1, fsdp_size), n_operands < 0 or a NULL operands array with
 * n_operands > 0 give VE_ERR_INVALID_ARG; n_operands == 0 is a no-op. */
ve_status ve_dbuffer_group_op(const ve_plan* plan, int32_t rank, int32_t op, float alpha,
                              const ve_group_operand* operands, int32_t n_operands, void* stream);

/* Launch options (process-wide tuning knobs for measurement; the defaults
 * are the measured choices).  Each option starts from its environment
 * variable, read once, else from its default:
 *   "wg_threads" (VE_WG_THREADS, 0) and "wg_gpt" (VE_WG_GPT, 0): pin the
 *       step's workgroup shape (threads, 4-element groups per thread) for
 *       blocks that fit it, when that shape is built; 0 = chosen by block size;
 *   "gemm_split" (VE_GEMM_SPLIT, 1): 0 = never cut a product's short last
 *       round of tiles along K;
 *   "gemm_cfg" (VE_GEMM_CFG, -1): pin a product configuration (0, 2: register
 *       staged 128^2 / 256^2 tiles; 6, 9: direct-to-LDS 4 waves of 128^2 /
 *       8 waves of 128x64; 13: 8 waves of 128x64, P direct to LDS in three
 *       stages, Q through registers; 14: direct-to-LDS 128^2 tiles of 2
 *       waves of 128x64, two workgroups a CU); -1 = chosen by shape;
 *   "gemm_xcd" (VE_GEMM_XCD, 1): 0 = plain tile order instead of the
 *       XCD-aware one;
 *   "wg_dynamic" (VE_WG_DYNAMIC, 1): how the step's row-block shapes
 *       (blocks of 4,097 to 12,288 groups: 512 threads with 14 to 24 groups
 *       per thread, 768 threads, 1024 threads with 7 to 10) and the row
 *       items below launch.  1: persistent workgroups (one or a few per
 *       CU) taking work from the plan's per-rank counters, for launches
 *       with at least 5 such blocks (or 32 row items) per CU, one
 *       workgroup per block below that (the persistent forms' fixed cost
 *       exceeds their gain there); 2: persistent whatever the amount of
 *       work; 0: never (no counters, no ordering of calls, see
 *       ve_shard_adam8bit_step).  Same results in every case;
 *   "wg_rows" (VE_WG_ROWS, 1): 0 = whole-row blocks of 2,048 or 4,096
 *       groups (rows of 8K or 16K elements) run one workgroup per block
 *       instead of persistent items of 4 or 2 consecutive blocks (same
 *       results, slower; needs "wg_dynamic" and no pinned shape).
 * ve_set_option changes a value for every later call of the process
 * (calls already queued are unaffected); ve_get_option reads it.  Errors:
 * an unknown name or a NULL value pointer gives VE_ERR_INVALID_ARG. */
ve_status ve_set_option(const char* name, int64_t value);
ve_status ve_get_option(const char* name, int64_t* value);

/* Streaming reference (not part of the method): copy `bytes` bytes from
 * `src` to `dst` (device pointers, both 16-byte aligned, bytes a multiple
 * of 16, not overlapping) with 16-byte non-temporal accesses on `stream`.
 * It is the measured bandwidth that the HBM-bound kernels above are
 * compared with: read + write bytes over its time.  Errors: a NULL or
 * misaligned buffer, a size that is negative or not a multiple of 16, or
 * overlapping buffers give VE_ERR_INVALID_ARG; bytes == 0 is a no-op. */
ve_status ve_stream_copy(void* dst, const void* src, int64_t bytes, void* stream);

/* Structure-aware bucket planner (talk notes, "2. Structure-aware planning
 * algorithm"; Dutch summary, "2B"; Korean summary, "2.2").  Host only: no
 * device is touched.  Reads rows, cols and block_rows of the host array
 * specs[n_tensors] (block_cols and offset are ignored on input) and writes
 * every tensor's offset and *shard_elems = S; the result passes
 * ve_plan_load's checks for fsdp_size.
 *   Order: by shard unit (min(block_rows, rows) * cols elements), largest
 *   first, ties in input order.  Placement: each tensor at the smallest
 *   multiple of `align` after the previous tensor at which every chunk
 *   boundary inside it falls on one of its unit boundaries; padding only
 *   between tensors.  S: the smallest multiple of `align` for which the
 *   ordered tensors fit in fsdp_size chunks; for this order no smaller S
 *   admits a valid placement.
 *   *lower_bound (may be NULL): the smallest S any layout, in any order,
 *   could have: at least total/fsdp_size rounded up to `align`, and a
 *   multiple of the unit of every tensor longer than 2S (such a tensor
 *   crosses two chunk boundaries wherever it lies).
 * Errors: NULL specs or shard_elems, n_tensors < 1, fsdp_size < 1, align
 * outside [1, 2^20] or a non-positive shape or block: VE_ERR_INVALID_ARG;
 * a bucket beyond 2^52 / fsdp_size elements: VE_ERR_UNSUPPORTED.  On error
 * the outputs are not written. */
ve_status ve_plan_layout(ve_tensor_spec* specs, int32_t n_tensors, int32_t fsdp_size, int64_t align,
                         int64_t* shard_elems, int64_t* lower_bound);

/* Grouping of a model's tensors into buckets (talk notes, "2. Structure-
 * aware planning algorithm": RaggedShard tensors are grouped into
 * communication buffers; Dutch summary, "2B").  Host only.  specs[n_tensors]
 * lists the model's tensors in model order (rows, cols, block_rows read;
 * offset written); unit_of[k] numbers the wrapper unit (e.g. the decoder
 * layer) tensor k belongs to, 0, 1, 2, ... in tensor order.  A bucket is a
 * run of consecutive units, laid out by the rules of ve_plan_layout; a
 * dynamic program over the split points picks the runs that minimise,
 * first, the summed padding above `tolerance` (a fraction of each bucket),
 * then the number of buckets, largest first.  A run holds at most
 * `max_units` units and, when it holds several, at most twice the elements
 * of the largest unit.  Outputs: bucket_of[k] (bucket of tensor k),
 * specs[k].offset (offset inside its bucket), shard_elems[b] (S of bucket
 * b; the caller provides one entry per unit), *n_buckets.  Errors: NULL
 * arguments, n_tensors < 1, fsdp_size < 1, align outside [1, 2^20],
 * max_units < 1, tolerance outside [0, 1), a unit numbering that is not
 * 0, 1, 2, ... or a non-positive shape give VE_ERR_INVALID_ARG; sizes
 * beyond 2^52 / fsdp_size elements give VE_ERR_UNSUPPORTED. */
ve_status ve_plan_buckets(ve_tensor_spec* specs, const int32_t* unit_of, int32_t n_tensors, int32_t fsdp_size,
                          int64_t align, int32_t max_units, double tolerance, int32_t* bucket_of,
                          int64_t* shard_elems, int32_t* n_buckets);

/* Muon's Newton-Schulz orthogonalisation of one gathered 2-D matrix, the
 * dense work of the root rank in distributed Muon (talk notes, "Case study:
 * 8-bit Adam and distributed Muon": the full matrix is gathered on one rank,
 * iterated and redistributed; Dutch summary, "Muon-optimalisator").  The
 * iteration is the published Muon quintic: X0 = G / (|G|_F + eps) in the
 * wide orientation (a tall G is transposed), then `steps` times
 * A = X X^T, B = b A + c A A, X = a X + B X with (a, b, c) =
 * (3.4445, -4.7750, 2.0315); the result is returned in G's orientation.
 * Precision: X, A and B are bf16; products accumulate in fp32 on the MFMA
 * units; each stored result is rounded once from fp32 to bf16 (nearest
 * even); the Frobenius norm is accumulated in fp64 and 1/(|G|_F + eps) is
 * rounded to fp32.
 *   G, out: device, bf16 rows x cols row-major (out may not alias G or the
 *   workspace).  steps in [0, 64] (0: out = bf16(G / (|G|_F + eps))).
 *   workspace: device, 256-byte aligned, at least ve_muon_workspace_bytes
 *   bytes, owned by the caller; its contents are scratch (two copies of X
 *   and of X^T, A, B, and when the longer side is at least 1024 a further
 *   64 MiB for the fp32 K slices of products whose last (or only) round of
 *   tiles is split along the contraction).
 * Errors: NULL pointers, a non-positive shape, steps outside [0, 64], eps
 * negative or not finite, a short or misaligned workspace:
 * VE_ERR_INVALID_ARG; a matrix beyond one launch: VE_ERR_UNSUPPORTED;
 * launch failures: VE_ERR_DEVICE. */
ve_status ve_muon_workspace_bytes(int64_t rows, int64_t cols, int64_t* bytes);
ve_status ve_muon_newton_schulz(const uint16_t* G, uint16_t* out, int64_t rows, int64_t cols, int32_t steps,
                                float eps, void* workspace, int64_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * iteration as ve_muon_newton_schulz, bit for bit, with its workspace in a
 * static device array of 200 MiB that each GPU the library runs on holds
 * until the process ends (so any matrix whose ve_muon_workspace_bytes is at
 * most 200 MiB, e.g. 2048 x 7168 or 3,400 x 3,400).  G and out as above; the
 * call allocates nothing.  Calls on one GPU share that array: calls that
 * overlap on one GPU (two streams or threads) race.  Errors: as
 * ve_muon_newton_schulz; a larger workspace need gives VE_ERR_UNSUPPORTED;
 * no current device gives VE_ERR_DEVICE. */
ve_status ve_muon_newton_schulz_noalloc(const uint16_t* G, uint16_t* out, int64_t rows, int64_t cols,
                                        int32_t steps, float eps, void* stream);

/* The product kernel the iteration runs on: C = bf16(alpha * P Q^T + beta * D)
 * with P (M x K), Q (N x K), D and C (M x N) and CT = C^T (N x M), all bf16
 * row-major device arrays with leading dimensions ld* (>= the row length).
 * D may be NULL (beta ignored); C or CT may be NULL, not both.  fp32
 * accumulation on the MFMA units, one rounding to bf16.  symmetric != 0
 * declares P Q^T symmetric (M == N, C required, D symmetric if given): only
 * the output tiles on or above the diagonal are computed, each mirrored.
 * Errors: NULL P or Q, no output, a non-positive size, a short leading
 * dimension, symmetric without M == N and C: VE_ERR_INVALID_ARG. */
ve_status ve_gemm_bf16_nt(const uint16_t* P, int64_t ldp, const uint16_t* Q, int64_t ldq, const uint16_t* D,
                          int64_t ldd, uint16_t* C, int64_t ldc, uint16_t* CT, int64_t ldct, int64_t M, int64_t N,
                          int64_t K, float alpha, float beta, int32_t symmetric, void* stream);

/* Thread-local message of this thread's last failing call ("" if none). */
const char* ve_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VE_H */
