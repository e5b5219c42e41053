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
#include <atomic>
#include <cmath>
#include <cstdint>
#include <map>
#include <numeric>
#include <thread>
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

// One bucket: the order (largest unit first), S and the offsets (in the
// items' own order).  False if no S within `cap` works.
bool plan_bucket(const std::vector<Item>& it, int64_t m, int64_t align, int64_t cap, int64_t& S, int64_t& lb,
                 std::vector<int64_t>& offsets) {
    const size_t n = it.size();
    int64_t total = 0;
    for (const Item& x : it) total += x.n;
    std::vector<int32_t> order(n);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return it[(size_t)a].u > it[(size_t)b].u; });
    const int64_t s0 = std::max(align, ceil_to((total + m - 1) / m, align));
    S = next_forced_ok(it, s0, align, cap);
    if (S < 0) return false;
    lb = S;
    std::vector<int64_t> offs(n);
    while (!place(it, order, m, S, align, offs)) {
        S = next_forced_ok(it, S + align, align, cap);
        if (S < 0) return false;
    }
    offsets.assign(n, 0);
    for (size_t i = 0; i < n; ++i) offsets[(size_t)order[i]] = offs[i];
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
    int64_t S = 0, lb = 0;
    std::vector<int64_t> offs;
    if (!plan_bucket(it, m, align, cap, S, lb, offs))
        return fail(VE_ERR_UNSUPPORTED, "no shard size within 2^52/fsdp_size elements");
    if (lower_bound) *lower_bound = lb;
    for (int32_t k = 0; k < n_tensors; ++k) specs[k].offset = offs[(size_t)k];
    *shard_elems = S;
    return VE_OK;
}

// Grouping of a model's tensors into buckets (the DBuffers the collectives
// run on).  The pages state the problem -- group RaggedShard tensors into
// communication buffers -- and solve it with a heuristic order and dynamic
// programming (talk notes, "2. Structure-aware planning algorithm"; Dutch
// summary, "2B").  Reading taken: the model's wrapper units (e.g. one
// decoder layer each) stay in model order and a bucket is a run of
// consecutive units, planned with ve_plan_layout's rules; the dynamic
// program over the split points chooses the runs.  Objective, compared in
// order: (1) the padding above `tolerance` of each bucket, summed; (2) the
// number of buckets, more being better (smaller buffers, overlap of
// communication with compute).  A run holds at most `max_units` units and,
// when it holds more than one, at most twice the elements of the largest
// unit (the memory of one all-gathered buffer).  Runs of identical units
// (equal shape lists) are planned once.
extern "C" ve_status ve_plan_buckets(ve_tensor_spec* specs, const int32_t* unit_of, int32_t n_tensors,
                                     int32_t fsdp_size, int64_t align, int32_t max_units, double tolerance,
                                     int32_t* bucket_of, int64_t* shard_elems, int32_t* n_buckets) {
    using ve::fail;
    if (!specs || !unit_of || !bucket_of || !shard_elems || !n_buckets)
        return fail(VE_ERR_INVALID_ARG, "NULL argument");
    if (n_tensors < 1) return fail(VE_ERR_INVALID_ARG, "n_tensors %d < 1", n_tensors);
    if (fsdp_size < 1) return fail(VE_ERR_INVALID_ARG, "fsdp_size %d < 1", fsdp_size);
    if (align < 1 || align > (1 << 20)) return fail(VE_ERR_INVALID_ARG, "align %lld outside [1, 2^20]", (long long)align);
    if (max_units < 1) return fail(VE_ERR_INVALID_ARG, "max_units %d < 1", max_units);
    if (!(tolerance >= 0.0 && tolerance < 1.0)) return fail(VE_ERR_INVALID_ARG, "tolerance outside [0, 1)");
    if (unit_of[0] != 0) return fail(VE_ERR_INVALID_ARG, "unit_of[0] must be 0");
    for (int32_t k = 1; k < n_tensors; ++k)
        if (unit_of[k] != unit_of[k - 1] && unit_of[k] != unit_of[k - 1] + 1)
            return fail(VE_ERR_INVALID_ARG, "unit_of must number the units 0, 1, 2, ... in tensor order");
    const int64_t m = fsdp_size;
    const int64_t cap = (int64_t(1) << 52) / m;
    std::vector<Item> it((size_t)n_tensors);
    for (int32_t k = 0; k < n_tensors; ++k) {
        const ve_tensor_spec& t = specs[k];
        if (t.rows < 1 || t.cols < 1 || t.block_rows < 1)
            return fail(VE_ERR_INVALID_ARG, "tensor %d: non-positive shape or block", k);
        if (t.rows > cap / t.cols) return fail(VE_ERR_UNSUPPORTED, "tensor %d is too large", k);
        it[(size_t)k] = Item{t.rows * t.cols, std::min(t.block_rows, t.rows) * t.cols};
    }
    const int32_t U = unit_of[n_tensors - 1] + 1;
    std::vector<int32_t> first((size_t)U + 1, n_tensors);
    for (int32_t k = n_tensors - 1; k >= 0; --k) first[(size_t)unit_of[k]] = k;
    std::vector<double> usize((size_t)U, 0.0);
    for (int32_t k = 0; k < n_tensors; ++k) usize[(size_t)unit_of[k]] += (double)it[(size_t)k].n;
    const double largest = *std::max_element(usize.begin(), usize.end());

    // Candidate runs, each planned once per distinct shape list (on several
    // host threads: the plans are independent), before the DP reads them.
    struct Plan {
        int64_t S = 0, pad = 0;
        std::vector<int64_t> offs;
        bool ok = false;
    };
    auto key_of = [&](int32_t i, int32_t j) {
        std::vector<int64_t> key;
        key.reserve((size_t)(first[(size_t)j] - first[(size_t)i]) * 3);
        for (int32_t k = first[(size_t)i]; k < first[(size_t)j]; ++k)
            key.insert(key.end(), {specs[k].rows, specs[k].cols, specs[k].block_rows});
        return key;
    };
    auto admissible = [&](int32_t i, int32_t j) {
        if (j - i > max_units) return false;
        double tot = 0.0;
        for (int32_t u = i; u < j; ++u) tot += usize[(size_t)u];
        return j - i == 1 || tot <= 2.0 * largest;
    };
    std::map<std::vector<int64_t>, Plan> memo;  // node addresses stay valid
    std::vector<std::pair<int32_t, int32_t>> todo;  // one representative run per distinct key
    std::vector<Plan*> slot;                        // its plan
    std::vector<Plan*> cand((size_t)U * (size_t)max_units, nullptr);
    for (int32_t j = 1; j <= U; ++j)
        for (int32_t i = j - 1; i >= 0 && admissible(i, j); --i) {
            auto ins = memo.emplace(key_of(i, j), Plan{});
            if (ins.second) {
                todo.emplace_back(i, j);
                slot.push_back(&ins.first->second);
            }
            cand[(size_t)(j - 1) * (size_t)max_units + (size_t)(j - 1 - i)] = &ins.first->second;
        }
    auto work = [&](size_t t) {
        const int32_t i = todo[t].first, j = todo[t].second;
        std::vector<Item> sub(it.begin() + first[(size_t)i], it.begin() + first[(size_t)j]);
        int64_t total = 0;
        for (const Item& x : sub) total += x.n;
        Plan& p = *slot[t];
        int64_t lb = 0;
        if (total <= cap && plan_bucket(sub, m, align, cap, p.S, lb, p.offs)) {
            p.ok = true;
            p.pad = m * p.S - total;
        }
    };
    {
        const size_t nthr = std::min<size_t>(todo.size(), std::max(1u, std::min(16u, std::thread::hardware_concurrency())));
        std::atomic<size_t> next{0};
        std::vector<std::thread> pool;
        for (size_t w = 0; w + 1 < nthr; ++w)
            pool.emplace_back([&] {
                for (size_t t; (t = next++) < todo.size();) work(t);
            });
        for (size_t t; (t = next++) < todo.size();) work(t);
        for (auto& th : pool) th.join();
    }
    auto run_plan = [&](int32_t i, int32_t j) -> const Plan& {
        return *cand[(size_t)(j - 1) * (size_t)max_units + (size_t)(j - 1 - i)];
    };
    // best[j]: (excess padding, -buckets) of units [0, j)
    const double inf = 1e300;
    std::vector<double> ex((size_t)U + 1, inf);
    std::vector<int32_t> nb((size_t)U + 1, 0), prev((size_t)U + 1, -1);
    ex[0] = 0.0;
    for (int32_t j = 1; j <= U; ++j) {
        double tot = 0.0;
        for (int32_t i = j - 1; i >= 0 && admissible(i, j); --i) {
            tot += usize[(size_t)i];
            if (ex[(size_t)i] >= inf) continue;
            const Plan& p = run_plan(i, j);
            if (!p.ok) continue;
            const double excess = std::max(0.0, (double)p.pad - tolerance * (tot + (double)p.pad));
            const double e = ex[(size_t)i] + excess;
            const int32_t b = nb[(size_t)i] + 1;
            // equal excess up to the rounding of the sums: more buckets win
            const double eq = 1e-9 * (1.0 + std::fabs(ex[(size_t)j] < inf ? ex[(size_t)j] : 0.0));
            if (e < ex[(size_t)j] - eq || (e <= ex[(size_t)j] + eq && b > nb[(size_t)j])) {
                ex[(size_t)j] = e;
                nb[(size_t)j] = b;
                prev[(size_t)j] = i;
            }
        }
        if (ex[(size_t)j] >= inf) return fail(VE_ERR_UNSUPPORTED, "unit %d cannot be planned", j - 1);
    }
    std::vector<std::pair<int32_t, int32_t>> runs;
    for (int32_t j = U; j > 0; j = prev[(size_t)j]) runs.emplace_back(prev[(size_t)j], j);
    std::reverse(runs.begin(), runs.end());
    for (size_t b = 0; b < runs.size(); ++b) {
        const Plan& p = run_plan(runs[b].first, runs[b].second);
        shard_elems[b] = p.S;
        for (int32_t k = first[(size_t)runs[b].first]; k < first[(size_t)runs[b].second]; ++k) {
            bucket_of[k] = (int32_t)b;
            specs[k].offset = p.offs[(size_t)(k - first[(size_t)runs[b].first])];
        }
    }
    *n_buckets = (int32_t)runs.size();
    return VE_OK;
}
