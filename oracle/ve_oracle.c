/*
 * ve_oracle.c -- plain CPU reference for the RaggedShard shard step.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or table with the GPU library.
 *
 * What it computes, following veScale-FSDP (MLSys 2026 talk notes,
 * notes.yuuk.io; Dutch and Korean gist.science summaries of the same paper):
 *
 *  - Bucket layout.  A bucket is a flat buffer of m equal chunks of S
 *    elements; rank r owns [r*S, (r+1)*S).  Each tensor is one contiguous
 *    range [offset, offset+numel) of it; padding lives only between tensors
 *    (talk notes "2. Structure-aware planning"; Dutch summary "2B").  A
 *    tensor may be cut between ranks only at a RaggedShard unit boundary,
 *    i.e. a multiple of block_rows*cols elements from its first element
 *    (talk notes "1. RaggedShard": block-wise uneven sharding whose shard
 *    boundaries coincide with block boundaries).
 *
 *  - Group copy-in.  The rank's chunk of the gradient bucket is filled from
 *    the per-parameter gradients; padding is zero (talk notes "3. DBuffer":
 *    tensors are placed into the buffer by group-level operators).
 *
 *  - Block-wise 8-bit AdamW on the local shard.  Every quantisation block
 *    (a block_rows x block_cols tile of one tensor) is quantised on its own,
 *    with one absmax scale per moment, so no rank needs another rank's data
 *    (talk notes "1. RaggedShard", sync-free block-wise quantisation, and
 *    "Case study: 8-bit Adam").  The pages give no formula; the reading
 *    taken here is textbook AdamW with decoupled weight decay and bias
 *    correction, both moments stored as symmetric linear int8 codes with
 *    127 levels and one fp32 scale amax/127 per block.  The fresh moments
 *    (not their quantised images) drive this step's update.
 *
 *  - Write-back of the parameter shard as bf16 for the next all-gather.
 *
 *  - Bucket planning: the smallest chunk length S at which the tensors fit
 *    (in a given order, or in any order) by exhaustive search over offsets.
 *
 *  - DBuffer group operations (zero, scale, accumulate) applied to every
 *    tensor of a chunk or of the whole bucket at once (talk notes
 *    "3. DBuffer"; Dutch summary "C"), in fp32 as described at
 *    ora_group_op.
 *
 * Arithmetic: every update of the shard step is carried out in double
 * precision.  Stored
 * results take their storage type: fp32 master, fp32 scales, bf16 param
 * (round-to-nearest-even of the stored fp32 master).  The int8 codes are
 * integers decided by floating point, so that decision is taken in the
 * storage precision of the moments (fp32): the fresh moments are rounded to
 * fp32, the block absmax and 127/absmax are fp32, and the code is
 * rint(fp32(moment * (127/absmax))) clamped to [-127, 127].
 *
 * Block order on a rank (the index of m_scale / v_scale): the rank's tensor
 * pieces in ascending bucket offset; inside a piece, row panels top to
 * bottom, and inside a panel, tiles left to right.
 */
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t rows, cols, block_rows, block_cols, offset;
} ora_tensor;

static _Thread_local char g_msg[512];
const char* ora_last_error(void) { return g_msg; }

static int fail(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_msg, sizeof g_msg, fmt, ap);
    va_end(ap);
    return 1;
}

/* ---- bf16 <-> fp32 (bit patterns) ------------------------------------- */
static float bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint16_t f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN */
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

/* ---- layout --------------------------------------------------------------- */
/* Tensor k's piece on rank r: tensor elements [*lo, *hi).  Returns 0 if none. */
static int piece(const ora_tensor* t, int64_t S, int64_t r, int64_t* lo, int64_t* hi) {
    int64_t n = t->rows * t->cols;
    int64_t a = t->offset, b = t->offset + n;
    int64_t c0 = r * S, c1 = c0 + S;
    int64_t x = a > c0 ? a : c0;
    int64_t y = b < c1 ? b : c1;
    if (x >= y) return 0;
    *lo = x - a;
    *hi = y - a;
    return 1;
}

/* (offset, index) pairs sort by offset; no shared state, so independent
 * buckets can be stepped from several threads at once. */
typedef struct {
    int64_t offset;
    int index;
} ora_key;
static int by_offset(const void* a, const void* b) {
    int64_t x = ((const ora_key*)a)->offset, y = ((const ora_key*)b)->offset;
    if (x != y) return (x > y) - (x < y);
    return ((const ora_key*)a)->index - ((const ora_key*)b)->index;
}

/* indices of the tensors sorted by bucket offset (caller frees) */
static int* offset_order(const ora_tensor* t, int n) {
    int* idx = (int*)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
    ora_key* keys = (ora_key*)malloc(sizeof(ora_key) * (size_t)(n > 0 ? n : 1));
    for (int i = 0; i < n; ++i) {
        keys[i].offset = t[i].offset;
        keys[i].index = i;
    }
    qsort(keys, (size_t)n, sizeof(ora_key), by_offset);
    for (int i = 0; i < n; ++i) idx[i] = keys[i].index;
    free(keys);
    return idx;
}

/* Layout checks: shapes and tiles well formed; tensors inside the bucket and
 * disjoint; every cut between ranks on a unit boundary of its tensor. */
int ora_validate(const ora_tensor* t, int n, int m, int64_t S) {
    if (n < 0 || m < 1 || S < 1) return fail("bad bucket: n=%d m=%d S=%lld", n, m, (long long)S);
    for (int k = 0; k < n; ++k) {
        const ora_tensor* x = &t[k];
        if (x->rows < 1 || x->cols < 1 || x->block_rows < 1 || x->block_cols < 1)
            return fail("tensor %d: non-positive shape or block (rows=%lld cols=%lld)", k, (long long)x->rows, (long long)x->cols);
        if (x->cols % x->block_cols != 0)
            return fail("tensor %d: block_cols %lld does not divide cols %lld", k, (long long)x->block_cols, (long long)x->cols);
        if (x->offset < 0 || x->offset + x->rows * x->cols > (int64_t)m * S)
            return fail("tensor %d: [%lld, +%lld) leaves the bucket", k, (long long)x->offset, (long long)(x->rows * x->cols));
    }
    int* idx = offset_order(t, n);
    for (int i = 1; i < n; ++i) {
        const ora_tensor* p = &t[idx[i - 1]];
        const ora_tensor* q = &t[idx[i]];
        if (p->offset + p->rows * p->cols > q->offset) {
            int a = idx[i - 1], b = idx[i];
            free(idx);
            return fail("tensors %d and %d overlap at %lld", a, b, (long long)q->offset);
        }
    }
    free(idx);
    for (int k = 0; k < n; ++k) {
        const ora_tensor* x = &t[k];
        int64_t unit = x->block_rows * x->cols, numel = x->rows * x->cols;
        for (int64_t r = 0; r < m; ++r) {
            int64_t lo, hi;
            if (!piece(x, S, r, &lo, &hi)) continue;
            if (lo % unit != 0)
                return fail("tensor %d: rank %lld piece starts at element %lld, not a unit boundary", k, (long long)r, (long long)lo);
            if (hi != numel && hi % unit != 0)
                return fail("tensor %d: rank %lld piece ends at element %lld, not a unit boundary", k, (long long)r, (long long)hi);
        }
    }
    return 0;
}

/* Number of quantisation blocks and valid elements on rank r. */
int64_t ora_rank_blocks(const ora_tensor* t, int n, int64_t S, int64_t r, int64_t* valid) {
    int64_t nb = 0, nv = 0;
    for (int k = 0; k < n; ++k) {
        int64_t lo, hi;
        if (!piece(&t[k], S, r, &lo, &hi)) continue;
        int64_t unit = t[k].block_rows * t[k].cols;
        int64_t panels = (hi - lo + unit - 1) / unit;
        nb += panels * (t[k].cols / t[k].block_cols);
        nv += hi - lo;
    }
    if (valid) *valid = nv;
    return nb;
}

/* Zero-copy extraction: where tensor k's local piece sits in rank r's shard
 * (r = -1: in the whole bucket).  Returns 0 if the rank holds none of it. */
int ora_slice(const ora_tensor* t, int n, int m, int64_t S, int64_t r, int k,
              int64_t* shard_off, int64_t* lo, int64_t* hi) {
    (void)n;
    if (r < 0) {
        *shard_off = t[k].offset;
        *lo = 0;
        *hi = t[k].rows * t[k].cols;
        return 1;
    }
    (void)m;
    if (!piece(&t[k], S, r, lo, hi)) return 0;
    *shard_off = t[k].offset + *lo - r * S;
    return 1;
}

/* Group copy-in: out[0, S) (r >= 0) or out[0, m*S) (r = -1) receives every
 * tensor element that lands there; everything else is zero.  grads[k] holds
 * tensor k's elements starting at element grad_base[k]. */
void ora_copy_in(const ora_tensor* t, int n, int m, int64_t S, int64_t r,
                 const uint16_t* const* grads, const int64_t* grad_base, uint16_t* out) {
    int64_t len = r < 0 ? (int64_t)m * S : S;
    int64_t c0 = r < 0 ? 0 : r * S;
    for (int64_t j = 0; j < len; ++j) out[j] = 0;
    for (int k = 0; k < n; ++k) {
        int64_t lo = 0, hi = t[k].rows * t[k].cols;
        if (r >= 0 && !piece(&t[k], S, r, &lo, &hi)) continue;
        for (int64_t e = lo; e < hi; ++e) out[t[k].offset + e - c0] = grads[k][e - grad_base[k]];
    }
}

/* ---- quantiser ------------------------------------------------------------ */
/* Symmetric linear int8 code of one block with one absmax scale:
 * scale = amax/127 and q = clamp(rint(x * (127/amax)), -127, 127), all in
 * fp32 (a block whose amax is 0 gets scale 0 and all-zero codes). */
void ora_quantize(const float* x, int64_t n, int8_t* q, float* scale) {
    float am = 0.0f;
    for (int64_t i = 0; i < n; ++i)
        if (fabsf(x[i]) > am) am = fabsf(x[i]);
    /* one division rounded once to fp32 == the correctly rounded fp32 quotient */
    *scale = (float)((double)am / 127.0);
    const float inv = am > 0.0f ? (float)(127.0 / (double)am) : 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float y = (float)((double)x[i] * (double)inv); /* exact product, one rounding */
        y = rintf(y);                                  /* round half to even */
        if (y > 127.0f) y = 127.0f;
        if (y < -127.0f) y = -127.0f;
        q[i] = (int8_t)y;
    }
}

/* ---- DBuffer group operations ---------------------------------------------- */
/* One operation over every tensor of rank r's chunk (r = -1: the whole
 * bucket), the way the DBuffer applies an identical operation to all of its
 * tensors at once (talk notes "3. DBuffer"; Dutch summary "C": add, scale
 * and zero fused across tensors):
 *   op 0 zero:       every element of the chunk, padding included, becomes 0;
 *   op 1 scale:      x = alpha * x on tensor elements (gradient averaging);
 *   op 2 accumulate: x = x + alpha * g on tensor elements, g the
 *                    per-parameter gradient (gradient accumulation);
 * and padding becomes 0 for every op.  The pages fix no precision; the
 * reading taken is that of elementwise arithmetic on bf16 tensors in a
 * PyTorch system: the operands are widened to fp32, the operation is one
 * IEEE fp32 operation (a product, or a fused multiply-add with a single
 * rounding), and the result is rounded to bf16 to nearest-even. */
int ora_group_op(const ora_tensor* t, int n, int m, int64_t S, int64_t r, int op, float alpha,
                 const uint16_t* const* grads, const int64_t* grad_base, uint16_t* bucket) {
    if (op < 0 || op > 2) return fail("unknown group op %d", op);
    if (r < -1 || r >= m) return fail("rank %lld out of range [-1, %d)", (long long)r, m);
    const int64_t len = r < 0 ? (int64_t)m * S : S;
    const int64_t c0 = r < 0 ? 0 : r * S;
    char* covered = (char*)calloc((size_t)len, 1);
    if (!covered) return fail("out of host memory");
    for (int k = 0; k < n; ++k) {
        int64_t lo = 0, hi = t[k].rows * t[k].cols;
        if (r >= 0 && !piece(&t[k], S, r, &lo, &hi)) continue;
        for (int64_t e = lo; e < hi; ++e) {
            const int64_t pos = t[k].offset + e - c0;
            covered[pos] = 1;
            const float x = bf16_to_f32(bucket[pos]);
            if (op == 0) {
                bucket[pos] = 0;
            } else if (op == 1) {
                bucket[pos] = f32_to_bf16(alpha * x);
            } else {
                const float g = bf16_to_f32(grads[k][e - grad_base[k]]);
                bucket[pos] = f32_to_bf16(fmaf(alpha, g, x));
            }
        }
    }
    for (int64_t j = 0; j < len; ++j)
        if (!covered[j]) bucket[j] = 0;
    free(covered);
    return 0;
}

/* ---- bucket planning by exhaustive search ----------------------------------- */
/* A layout of tensors (n_k elements, shard unit u_k elements) in a bucket of
 * m chunks of S elements is valid when every offset is a multiple of `align`,
 * the tensors do not overlap and end by m*S, and every chunk boundary j*S
 * strictly inside tensor k lies a multiple of u_k from its first element
 * (talk notes "1. RaggedShard" and "2. Structure-aware planning";
 * padding only between tensors).  The search below tries every offset of
 * every tensor, so it only serves tiny buckets. */
static int boundaries_ok(int64_t o, int64_t n, int64_t u, int64_t m, int64_t S) {
    for (int64_t j = 1; j < m; ++j) {
        const int64_t b = j * S;
        if (b > o && b < o + n && (b - o) % u != 0) return 0;
    }
    return 1;
}

/* Can tensors order[i..cnt) be placed at or after `cursor`, in this order? */
static int place_from(const int64_t* n, const int64_t* u, const int* order, int i, int cnt, int64_t cursor,
                      int64_t m, int64_t S, int64_t align, int64_t rest) {
    if (i == cnt) return 1;
    const int k = order[i];
    int64_t o = (cursor + align - 1) / align * align;
    for (; o + rest <= m * S; o += align) {
        if (!boundaries_ok(o, n[k], u[k], m, S)) continue;
        if (place_from(n, u, order, i + 1, cnt, o + n[k], m, S, align, rest - n[k])) return 1;
    }
    return 0;
}

/* Smallest S (a multiple of align, at most s_max) for which the tensors fit
 * in the given order; 0 if none does. */
int64_t ora_plan_min_shard(const int64_t* n, const int64_t* u, const int* order, int cnt, int64_t m,
                           int64_t align, int64_t s_max) {
    int64_t total = 0;
    for (int i = 0; i < cnt; ++i) total += n[i];
    for (int64_t S = align; S <= s_max; S += align) {
        if (m * S < total) continue;
        if (place_from(n, u, order, 0, cnt, 0, m, S, align, total)) return S;
    }
    return 0;
}

static int next_permutation(int* a, int cnt) {
    int i = cnt - 2;
    while (i >= 0 && a[i] >= a[i + 1]) --i;
    if (i < 0) return 0;
    int j = cnt - 1;
    while (a[j] <= a[i]) --j;
    int t = a[i]; a[i] = a[j]; a[j] = t;
    for (int l = i + 1, r = cnt - 1; l < r; ++l, --r) { t = a[l]; a[l] = a[r]; a[r] = t; }
    return 1;
}

/* Smallest S over every order of the tensors (cnt <= 8). */
int64_t ora_plan_min_shard_any_order(const int64_t* n, const int64_t* u, int cnt, int64_t m, int64_t align,
                                     int64_t s_max) {
    if (cnt < 1 || cnt > 8) return fail("any-order search needs 1..8 tensors"), -1;
    int order[8];
    for (int i = 0; i < cnt; ++i) order[i] = i;
    int64_t best = 0;
    do {
        const int64_t lim = best ? best - align : s_max;
        if (lim < align) break;
        const int64_t S = ora_plan_min_shard(n, u, order, cnt, m, align, lim);
        if (S) best = S;
    } while (next_permutation(order, cnt));
    return best;
}

/* ---- the shard step --------------------------------------------------------- */
typedef struct {
    double lr, beta1, beta2, eps, wd;
} ora_hparams;

/* Is block b in the ascending list sel[0..nsel) (every block when sel is NULL)? */
static int selected(int64_t b, const int64_t* sel, int64_t nsel) {
    if (!sel) return 1;
    int64_t lo = 0, hi = nsel;
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo) / 2;
        if (sel[mid] < b) lo = mid + 1; else hi = mid;
    }
    return lo < nsel && sel[lo] == b;
}

/* One step of block-wise 8-bit AdamW on rank r's shard.
 *
 * grads[k] / grad_base[k]: per-parameter bf16 gradients (see ora_copy_in);
 * only tensors with a piece on r are read.
 * grad_shard, master, m_q, v_q, param_shard: length S, shard coordinates.
 * m_scale, v_scale: one entry per block of the rank (block order above).
 * t: step number, >= 1.
 * sel / nsel: if sel is non-NULL only those block indices (ascending) are
 * processed (used to check samples of very large shards, and by callers
 * that split the blocks over threads); padding is then untouched.
 */
int ora_shard_step(const ora_tensor* T, int n, int m, int64_t S, int64_t r,
                   const uint16_t* const* grads, const int64_t* grad_base,
                   uint16_t* grad_shard, float* master, int8_t* m_q, int8_t* v_q,
                   float* m_scale, float* v_scale, uint16_t* param_shard,
                   const ora_hparams* hp, int64_t t, const int64_t* sel, int64_t nsel) {
    if (t < 1) return fail("step %lld < 1", (long long)t);
    if (r < 0 || r >= m) return fail("rank %lld out of range [0, %d)", (long long)r, m);
    const double b1 = hp->beta1, b2 = hp->beta2;
    const double bc1 = 1.0 - pow(b1, (double)t);
    const double bc2 = 1.0 - pow(b2, (double)t);
    const double decay = 1.0 - hp->lr * hp->wd;

    int* idx = offset_order(T, n);
    int64_t blk = 0;
    float* m1f = NULL;
    float* v1f = NULL;
    int8_t* codes = NULL;
    int64_t* pos = NULL;
    int64_t* src = NULL;
    int64_t cap = 0;
    char* covered = sel ? NULL : (char*)calloc((size_t)S, 1);

    for (int ii = 0; ii < n; ++ii) {
        const int k = idx[ii];
        const ora_tensor* x = &T[k];
        int64_t lo, hi;
        if (!piece(x, S, r, &lo, &hi)) continue;
        const int64_t R = x->rows, C = x->cols, br = x->block_rows, bc = x->block_cols;
        const int64_t unit = br * C;
        const int64_t shard_base = x->offset - r * S; /* shard position of tensor element 0 */
        for (int64_t p = lo / unit; p * unit < hi; ++p) {
            const int64_t r0 = p * br, r1 = (r0 + br < R) ? r0 + br : R;
            for (int64_t j = 0; j < C / bc; ++j, ++blk) {
                if (!selected(blk, sel, nsel)) continue;
                const int64_t nb = (r1 - r0) * bc;
                if (nb > cap) {
                    cap = nb;
                    m1f = (float*)realloc(m1f, sizeof(float) * (size_t)cap);
                    v1f = (float*)realloc(v1f, sizeof(float) * (size_t)cap);
                    codes = (int8_t*)realloc(codes, (size_t)cap);
                    pos = (int64_t*)realloc(pos, sizeof(int64_t) * (size_t)cap);
                    src = (int64_t*)realloc(src, sizeof(int64_t) * (size_t)cap);
                }
                /* the block's elements: rows r0..r1-1, cols j*bc..(j+1)*bc-1 */
                int64_t q = 0;
                for (int64_t row = r0; row < r1; ++row)
                    for (int64_t col = j * bc; col < (j + 1) * bc; ++col, ++q) {
                        int64_t e = row * C + col;
                        pos[q] = shard_base + e;
                        src[q] = e - grad_base[k];
                    }
                const double sm_old = m_scale[blk], sv_old = v_scale[blk];
                for (q = 0; q < nb; ++q) {
                    const uint16_t gbits = grads[k][src[q]];
                    const double g = (double)bf16_to_f32(gbits);
                    /* dequantise the stored moments */
                    const double m0 = (double)m_q[pos[q]] * sm_old;
                    const double v0 = (double)v_q[pos[q]] * sv_old;
                    /* Adam moments */
                    const double m1 = b1 * m0 + (1.0 - b1) * g;
                    const double v1 = b2 * v0 + (1.0 - b2) * g * g;
                    /* AdamW: decoupled decay, bias-corrected step */
                    const double p0 = (double)master[pos[q]];
                    const double upd = (hp->lr / bc1) * m1 / (sqrt(v1) / sqrt(bc2) + hp->eps);
                    const float p1 = (float)(p0 * decay - upd);
                    master[pos[q]] = p1;
                    param_shard[pos[q]] = f32_to_bf16(p1);
                    grad_shard[pos[q]] = gbits;
                    if (covered) covered[pos[q]] = 1;
                    m1f[q] = (float)m1;
                    v1f[q] = (float)v1;
                }
                float sm, sv;
                ora_quantize(m1f, nb, codes, &sm);
                for (q = 0; q < nb; ++q) m_q[pos[q]] = codes[q];
                ora_quantize(v1f, nb, codes, &sv);
                for (q = 0; q < nb; ++q) v_q[pos[q]] = codes[q];
                m_scale[blk] = sm;
                v_scale[blk] = sv;
            }
        }
    }
    if (covered) {
        for (int64_t j = 0; j < S; ++j)
            if (!covered[j]) {
                grad_shard[j] = 0;
                param_shard[j] = 0;
            }
        free(covered);
    }
    free(m1f);
    free(v1f);
    free(codes);
    free(pos);
    free(src);
    free(idx);
    return 0;
}
