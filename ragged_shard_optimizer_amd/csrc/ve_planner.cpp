// ve_planner.cpp -- the structure-aware bucket planner (host only).
//
// Problem (veScale-FSDP talk notes, "2. Structure-aware planning
// algorithm"; Dutch summary, "2B"; Korean summary, "2.2"): place the tensors
// of a bucket in a flat buffer of m equal chunks of S elements so that every
// tensor is contiguous, padding lies only between tensors, and every chunk
// boundary that falls inside a tensor lies on one of its RaggedShard unit
// boundaries (a multiple of block_rows*cols elements from its first
// element); make the buffer, m*S, as small as possible.  The pages state the
// problem is NP-hard and solve it with a heuristic order plus dynamic
// programming over placements.
//
// The algorithm here:
//  1. order: by shard unit, largest first (ties keep the input order);
//  2. placement DP: for a given S, state i = "the first i tensors of the
//     order are placed"; its value would be the set of reachable end
//     offsets, but a smaller end offset is never worse for the rest of the
//     order (padding can always be added), so only the minimum is kept and
//     each tensor goes to its earliest feasible offset;
//  3. S: the smallest multiple of the alignment for which step 2 fits the
//     whole order in m chunks, scanned upward from a lower bound.
// For the chosen order the result is therefore optimal.  Feasibility is not
// monotone in S (moving the boundaries can turn a wasteful crossing into an
// aligned one), so the scan is exhaustive, not a bisection.
//
// Lower bound for any order: S >= ceil(total/m), and a tensor longer than 2S
// crosses two chunk boundaries wherever it lies, which requires S to be a
// multiple of its unit.

#include <algorithm>
#include <cstdint>
#include <numeric>
#include <vector>

#include "ve.h"
#include "ve_internal.h"

namespace {

constexpr int64_t kI64Max = INT64_MAX;

struct Item {
    int64_t n;  // elements
    int64_t u;  // shard unit in elements
};

int64_t ceil_to(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// lcm, or -1 if it exceeds `cap`
int64_t lcm_capped(int64_t a, int64_t b, int64_t cap) {
    const int64_t g = std::gcd(a, b);
    const int64_t q = a / g;
    if (q > cap / b) return -1;
    return q * b;
}

// Smallest S' >= S (a multiple of A) that is a multiple of the unit of every
// tensor longer than 2 S'; -1 if the multiples exceed `cap`.
int64_t next_forced_ok(const std::vector<Item>& it, int64_t S, int64_t A, int64_t cap) {
    while (S <= cap) {
        int64_t step = A, drop = kI64Max;
        for (const Item& x : it) {
            if (x.n > 2 * S) {
                step = lcm_capped(step, x.u, cap);
                if (step < 0) return -1;
                drop = std::min(drop, (x.n - 1) / 2 + 1);  // from here on x is no longer forced
            }
        }
        if (S % step == 0) return S;
        const int64_t s2 = ceil_to(S, step);
        // a smaller S may satisfy the shorter forced list that applies past `drop`
        S = (drop != kI64Max && s2 > drop) ? ceil_to(drop, A) : s2;
    }
    return -1;
}

// Earliest offset >= c, a multiple of A, at which a tensor of n elements and
// unit u can start (every chunk boundary strictly inside it on a unit
// boundary); -1 if none starts before `end`.
int64_t earliest(int64_t c, int64_t n, int64_t u, int64_t S, int64_t A, int64_t L, int64_t end) {
    const int64_t off = ceil_to(c, A);
    const bool any_crossings = S % u == 0;  // then every later boundary aligns once the first does
    for (int64_t w = off / S * S; w < end; w += S) {
        const int64_t lo = std::max(off, w);
        if (lo + n <= w + S) return lo;       // fits inside this chunk
        const int64_t b = w + S;              // first boundary it would cross
        const int64_t o = b - (b - lo) / L * L;  // smallest o >= lo with o = b (mod L)
        if (o < b && (any_crossings || o + n <= b + S)) return o;
    }
    return -1;
}

// The placement DP for one S: offsets in `order` order, or false.
bool place(const std::vector<Item>& it, const std::vector<int32_t>& order, int64_t m, int64_t S, int64_t A,
           std::vector<int64_t>& offs) {
    const int64_t end = m * S;
    int64_t cursor = 0;
    for (size_t i = 0; i < order.size(); ++i) {
        const Item& x = it[(size_t)order[i]];
        const int64_t L = std::lcm(x.u, A);
        const int64_t o = earliest(cursor, x.n, x.u, S, A, L, end);
        if (o < 0 || o + x.n > end) return false;
        offs[i] = o;
        cursor = o + x.n;
    }
    return true;
}

}  // namespace

extern "C" ve_status ve_plan_layout(ve_tensor_spec* specs, int32_t n_tensors, int32_t fsdp_size, int64_t align,
                                    int64_t* shard_elems, int64_t* lower_bound) {
    using ve::fail;
    if (!specs || !shard_elems) return fail(VE_ERR_INVALID_ARG, "specs or shard_elems is NULL");
    if (n_tensors < 1) return fail(VE_ERR_INVALID_ARG, "n_tensors %d < 1", n_tensors);
    if (fsdp_size < 1) return fail(VE_ERR_INVALID_ARG, "fsdp_size %d < 1", fsdp_size);
    if (align < 1 || align > (1 << 20)) return fail(VE_ERR_INVALID_ARG, "align %lld outside [1, 2^20]", (long long)align);
    const int64_t m = fsdp_size;
    // the bucket m*S must stay far from int64 overflow
    const int64_t cap = (int64_t(1) << 52) / m;
    std::vector<Item> it((size_t)n_tensors);
    int64_t total = 0;
    for (int32_t k = 0; k < n_tensors; ++k) {
        const ve_tensor_spec& t = specs[k];
        if (t.rows < 1 || t.cols < 1 || t.block_rows < 1 || t.block_cols < 1)
            return fail(VE_ERR_INVALID_ARG, "tensor %d: non-positive shape or block", k);
        if (t.rows > cap / t.cols) return fail(VE_ERR_UNSUPPORTED, "tensor %d is too large", k);
        const int64_t n = t.rows * t.cols;
        it[(size_t)k] = Item{n, std::min(t.block_rows, t.rows) * t.cols};
        total += n;
        if (total > cap) return fail(VE_ERR_UNSUPPORTED, "bucket of more than 2^52/fsdp_size elements");
    }
    std::vector<int32_t> order((size_t)n_tensors);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(),
                     [&](int32_t a, int32_t b) { return it[(size_t)a].u > it[(size_t)b].u; });

    const int64_t s0 = std::max(align, ceil_to((total + m - 1) / m, align));
    int64_t S = next_forced_ok(it, s0, align, cap);
    if (S < 0) return fail(VE_ERR_UNSUPPORTED, "no shard size within 2^52/fsdp_size elements");
    if (lower_bound) *lower_bound = S;
    std::vector<int64_t> offs((size_t)n_tensors);
    while (!place(it, order, m, S, align, offs)) {
        S = next_forced_ok(it, S + align, align, cap);
        if (S < 0) return fail(VE_ERR_UNSUPPORTED, "no shard size within 2^52/fsdp_size elements");
    }
    for (size_t i = 0; i < order.size(); ++i) specs[order[i]].offset = offs[i];
    *shard_elems = S;
    return VE_OK;
}
