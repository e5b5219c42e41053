// ve_host.cpp -- host side of libve: layout validation, per-rank segment and
// run tables, and the C entry points declared in include/ve.h.
//
// A plan is built once per bucket layout (the planner runs once at
// initialisation; veScale-FSDP talk notes, "2. Structure-aware planning").
// For every rank it derives the pieces ("segments") of the tensors that fall
// in the rank's chunk, the rank-local block numbering, the block-size class
// of each segment, and the copy / padding runs, and uploads all of it to the
// device in one allocation.  Entry points afterwards only launch kernels.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "ve.h"
#include "ve_internal.h"

using namespace ve;

namespace {
thread_local std::string g_err;

struct OptionDef {
    const char* name;
    const char* env;
    int64_t dflt;
};
constexpr OptionDef kOptionDefs[kNumOptions] = {
    {"wg_threads", "VE_WG_THREADS", 0}, {"wg_gpt", "VE_WG_GPT", 0}, {"gemm_split", "VE_GEMM_SPLIT", 1},
    {"gemm_cfg", "VE_GEMM_CFG", -1},    {"gemm_xcd", "VE_GEMM_XCD", 1},     {"wg_dynamic", "VE_WG_DYNAMIC", 1},
    {"wg_rows", "VE_WG_ROWS", 1},
};
std::atomic<int64_t> g_options[kNumOptions];
std::once_flag g_options_once;

void seed_options() {
    for (int i = 0; i < kNumOptions; ++i) {
        const char* e = std::getenv(kOptionDefs[i].env);
        g_options[i].store(e ? std::atoll(e) : kOptionDefs[i].dflt, std::memory_order_relaxed);
    }
}

int option_index(const char* name) {
    if (!name) return -1;
    for (int i = 0; i < kNumOptions; ++i)
        if (std::strcmp(name, kOptionDefs[i].name) == 0) return i;
    return -1;
}
}  // namespace

int64_t ve::option(Option o) {
    std::call_once(g_options_once, seed_options);
    return g_options[o].load(std::memory_order_relaxed);
}

ve_status ve::fail(ve_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

namespace {

// host-side copies of one work list / run table, with byte offsets into the
// single device allocation filled in at upload
struct HostWork {
    std::vector<int32_t> seg_idx;
    std::vector<int64_t> prefix{0};
    size_t off_idx = 0, off_pref = 0;
};

struct HostRuns {
    std::vector<Run> runs;
    std::vector<int64_t> tile_prefix{0};
    std::vector<int32_t> tile_run;
    size_t off_runs = 0, off_pref = 0, off_tiles = 0;
    int64_t zero_elems = 0;
};

struct RankTables {
    std::vector<Seg> segs;
    size_t off_segs = 0;
    HostWork small, wg, huge;
    HostRuns copy;  // pieces + padding of the rank slice
    HostRuns pad;   // padding only (the step's zero fill)
    int64_t valid = 0, nblocks = 0;
};

void add_run(HostRuns& h, int64_t dst, int64_t src, int64_t len, int32_t tensor) {
    if (len <= 0) return;
    Run r{dst, src, len, tensor, 0};
    const int32_t ri = (int32_t)h.runs.size();
    h.runs.push_back(r);
    const int64_t tiles = run_tiles(dst, len);
    h.tile_prefix.push_back(h.tile_prefix.back() + tiles);
    for (int64_t t = 0; t < tiles; ++t) h.tile_run.push_back(ri);
    if (tensor < 0) h.zero_elems += len;
}

int32_t next_pow2(int32_t x) {
    int32_t g = 1;
    while (g < x) g <<= 1;
    return g;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

struct ve_plan {
    int device = 0;
    int32_t m = 0;
    int64_t S = 0;
    std::vector<ve_tensor_spec> specs;
    std::vector<int32_t> order;  // tensor indices by ascending offset
    std::vector<RankTables> ranks;
    HostRuns whole;              // rank == -1 copy-in
    char* dev = nullptr;         // one device allocation holding every table
    size_t dev_bytes = 0;
    size_t off_sched = 0;        // per rank, kSchedStride bytes: the persistent step's two counters (zero at rest)
    int n_cu = 0;                // compute units of `device`
    // Per rank: the stream of the last step call that used the counters and
    // an event recorded after its launches, so that a call on another stream
    // waits for it (the counters admit one launch at a time).
    struct SchedOrder {
        hipEvent_t done = nullptr;
        hipStream_t stream = nullptr;
        bool used = false;
    };
    mutable std::mutex sched_mu;
    mutable std::vector<SchedOrder> sched_order;

    template <class T>
    const T* dptr(size_t off) const { return reinterpret_cast<const T*>(dev + off); }
};

namespace {

// -------------------------------------------------------------------------
// validation (the RaggedShard layout rules; talk notes "1. RaggedShard" and
// "2. Structure-aware planning")
ve_status validate(const ve_tensor_spec* sp, int32_t n, int32_t m, int64_t S, std::vector<int32_t>& order) {
    if (n < 0) return fail(VE_ERR_INVALID_ARG, "n_tensors %d < 0", n);
    if (m < 1) return fail(VE_ERR_INVALID_ARG, "fsdp_size %d < 1", m);
    if (S < 1) return fail(VE_ERR_INVALID_ARG, "shard_elems %lld < 1", (long long)S);
    if (S > INT64_MAX / m) return fail(VE_ERR_INVALID_ARG, "bucket size overflows");
    const int64_t total = S * m;
    for (int32_t k = 0; k < n; ++k) {
        const ve_tensor_spec& t = sp[k];
        if (t.rows < 1 || t.cols < 1 || t.block_rows < 1 || t.block_cols < 1)
            return fail(VE_ERR_LAYOUT, "tensor %d: shape %lldx%lld / block %lldx%lld must be positive", k,
                        (long long)t.rows, (long long)t.cols, (long long)t.block_rows, (long long)t.block_cols);
        if (t.cols % t.block_cols != 0)
            return fail(VE_ERR_LAYOUT, "tensor %d: block_cols %lld does not divide cols %lld", k,
                        (long long)t.block_cols, (long long)t.cols);
        if (t.rows > total / t.cols) return fail(VE_ERR_LAYOUT, "tensor %d: larger than the bucket", k);
        const int64_t numel = t.rows * t.cols;
        if (t.offset < 0 || t.offset > total - numel)
            return fail(VE_ERR_LAYOUT, "tensor %d: elements [%lld, %lld) leave the bucket [0, %lld)", k,
                        (long long)t.offset, (long long)(t.offset + numel), (long long)total);
        const int64_t br = std::min(t.block_rows, t.rows);
        const int64_t block_elems = br * t.block_cols;
        if (block_elems > (int64_t(1) << 30))
            return fail(VE_ERR_UNSUPPORTED, "tensor %d: quantisation block of %lld elements exceeds 2^30", k,
                        (long long)block_elems);
        if (br > INT32_MAX || t.cols / t.block_cols > INT32_MAX)
            return fail(VE_ERR_UNSUPPORTED, "tensor %d: block geometry beyond 32-bit counters", k);
    }
    order.resize((size_t)n);
    for (int32_t k = 0; k < n; ++k) order[(size_t)k] = k;
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return sp[a].offset < sp[b].offset; });
    for (int32_t i = 1; i < n; ++i) {
        const ve_tensor_spec& a = sp[order[(size_t)i - 1]];
        const ve_tensor_spec& b = sp[order[(size_t)i]];
        if (a.offset + a.rows * a.cols > b.offset)
            return fail(VE_ERR_LAYOUT, "tensors %d and %d overlap at bucket offset %lld", order[(size_t)i - 1],
                        order[(size_t)i], (long long)b.offset);
    }
    // every chunk boundary strictly inside a tensor sits on one of its units
    for (int32_t k = 0; k < n; ++k) {
        const ve_tensor_spec& t = sp[k];
        // a block taller than the tensor is the whole tensor (clamped: no overflow)
        const int64_t numel = t.rows * t.cols, unit = std::min(t.block_rows, t.rows) * t.cols;
        for (int64_t b = (t.offset / S + 1) * S; b < t.offset + numel; b += S) {
            if ((b - t.offset) % unit != 0)
                return fail(VE_ERR_LAYOUT,
                            "tensor %d: chunk boundary at bucket offset %lld cuts it at element %lld, "
                            "not a multiple of its unit %lld (block_rows %lld x cols %lld)",
                            k, (long long)b, (long long)(b - t.offset), (long long)unit, (long long)t.block_rows,
                            (long long)t.cols);
        }
    }
    return VE_OK;
}

void build_rank(ve_plan& P, int32_t r, RankTables& rt) {
    const int64_t c0 = (int64_t)r * P.S, c1 = c0 + P.S;
    int64_t cursor = 0;  // shard coordinate covered so far (for padding runs)
    int64_t block0 = 0;
    for (int32_t k : P.order) {
        const ve_tensor_spec& t = P.specs[(size_t)k];
        const int64_t numel = t.rows * t.cols;
        const int64_t a = std::max(t.offset, c0), b = std::min(t.offset + numel, c1);
        if (a >= b) continue;
        Seg s{};
        s.shard_base = t.offset - c0;
        s.elem_lo = a - t.offset;
        s.elem_hi = b - t.offset;
        s.rows = t.rows;
        s.cols = t.cols;
        s.block_rows = std::min(t.block_rows, t.rows);
        s.block_cols = t.block_cols;
        const int64_t unit = s.block_rows * t.cols;
        s.panel0 = s.elem_lo / unit;
        const int64_t panels = ceil_div(s.elem_hi, unit) - s.panel0;
        s.tiles = (int32_t)(t.cols / t.block_cols);
        s.nblocks = panels * s.tiles;
        s.block0 = block0;
        s.tensor = k;
        const int64_t br = s.block_rows;
        // lane-chunks of a full block: whole-row blocks are one run, tiles br runs
        auto chunks_of = [&](int64_t ch) {
            return s.tiles == 1 ? ceil_div(br * t.cols, ch) : br * ceil_div(t.block_cols, ch);
        };
        const int64_t chunks = chunks_of(kSmallChunk), groups = chunks_of(kWgChunk);
        s.max_chunks = (int32_t)std::min<int64_t>(chunks, INT32_MAX);
        s.max_groups = (int32_t)std::min<int64_t>(groups, INT32_MAX);
        if (br * t.cols == 1) {  // one-element blocks (then block_cols == cols == 1)
            s.cls = kUnit;
            s.group = 1;
        } else if (chunks <= kSmallMaxChunks) {
            s.cls = kSmall;
            s.group = next_pow2((int32_t)chunks);
        } else if (groups <= kWgMaxGroups) {
            s.cls = kWg;
            s.group = 0;
        } else {
            s.cls = kHuge;
            s.group = 0;
        }
        const int32_t si = (int32_t)rt.segs.size();
        rt.segs.push_back(s);
        block0 += s.nblocks;
        rt.valid += s.elem_hi - s.elem_lo;
        HostWork& w = (s.cls == kSmall || s.cls == kUnit) ? rt.small : (s.cls == kWg ? rt.wg : rt.huge);
        const int64_t items = s.cls == kSmall  ? ceil_div(s.nblocks, 64 / s.group)
                              : s.cls == kUnit ? ceil_div(s.nblocks, kUnitPerWave)
                                               : s.nblocks;
        w.seg_idx.push_back(si);
        w.prefix.push_back(w.prefix.back() + items);
        const int64_t dst = a - c0;
        add_run(rt.copy, cursor, 0, dst - cursor, -1);
        add_run(rt.pad, cursor, 0, dst - cursor, -1);
        add_run(rt.copy, dst, s.elem_lo, b - a, k);
        cursor = b - c0;
    }
    add_run(rt.copy, cursor, 0, P.S - cursor, -1);
    add_run(rt.pad, cursor, 0, P.S - cursor, -1);
    rt.nblocks = block0;
}

void build_whole(ve_plan& P) {
    int64_t cursor = 0;
    for (int32_t k : P.order) {
        const ve_tensor_spec& t = P.specs[(size_t)k];
        add_run(P.whole, cursor, 0, t.offset - cursor, -1);
        add_run(P.whole, t.offset, 0, t.rows * t.cols, k);
        cursor = t.offset + t.rows * t.cols;
    }
    add_run(P.whole, cursor, 0, P.S * P.m - cursor, -1);
}

// layout of the single device allocation
struct Packer {
    std::vector<char> buf;
    template <class T>
    size_t put(const std::vector<T>& v) {
        size_t off = (buf.size() + 255) & ~size_t(255);
        buf.resize(off + sizeof(T) * v.size());
        if (!v.empty()) std::memcpy(buf.data() + off, v.data(), sizeof(T) * v.size());
        return off;
    }
};

void pack_runs(Packer& pk, HostRuns& h) {
    h.off_runs = pk.put(h.runs);
    h.off_pref = pk.put(h.tile_prefix);
    h.off_tiles = pk.put(h.tile_run);
}

void pack_work(Packer& pk, HostWork& w) {
    w.off_idx = pk.put(w.seg_idx);
    w.off_pref = pk.put(w.prefix);
}

RunArgs run_args(const ve_plan& P, const HostRuns& h) {
    RunArgs r;
    r.runs = P.dptr<Run>(h.off_runs);
    r.tile_prefix = P.dptr<int64_t>(h.off_pref);
    r.tile_run = P.dptr<int32_t>(h.off_tiles);
    r.n_runs = (int32_t)h.runs.size();
    r.n_tiles = h.tile_prefix.back();
    return r;
}

// Point the step arguments at one class's work list (small-block path).
void set_work(StepArgs& a, const ve_plan& P, const HostWork& w) {
    a.work.seg_idx = P.dptr<int32_t>(w.off_idx);
    a.work.prefix = P.dptr<int64_t>(w.off_pref);
    a.work.n = (int32_t)w.seg_idx.size();
    a.work.total = w.prefix.back();
    a.n_inline = 0;
}

// Copy segments [i0, i1) of a class's work list into the step arguments
// (workgroup paths); returns the number of work items of the slice.
int64_t set_inline(StepArgs& a, const RankTables& rt, const HostWork& w, size_t i0, size_t i1) {
    a.n_inline = (int32_t)(i1 - i0);
    for (size_t i = i0; i < i1; ++i) {
        a.inl_segs[i - i0] = rt.segs[(size_t)w.seg_idx[i]];
        a.inl_prefix[i - i0] = w.prefix[i] - w.prefix[i0];
    }
    a.inl_prefix[i1 - i0] = w.prefix[i1] - w.prefix[i0];
    a.work.total = a.inl_prefix[i1 - i0];
    return a.work.total;
}

// Persistent multi-block item form of a workgroup-path segment (ItemForm),
// kItemNone for none: segments of whole-row blocks (one tile a panel) of
// 2,048 or 4,096 groups run items of 4 or 2 consecutive blocks, 8,192
// groups, as one contiguous span (option wg_rows; needs the persistent
// form and no pinned shape; k_step_rows gives the measurements).
int item_form(const Seg& sg) {
    if (option(kOptWgRows) == 0 || option(kOptWgDynamic) == 0) return kItemNone;
    if (option(kOptWgThreads) > 0 && option(kOptWgGpt) > 0) return kItemNone;
    if (sg.tiles != 1) return kItemNone;
    if (sg.max_groups == kItemGroups / 4) return kItemRows4;
    if (sg.max_groups == kItemGroups / 2) return kItemRows2;
    return kItemNone;
}

// Items of item_blocks(form) blocks over segments [i0, i1) of a class's work
// list (a segment's last item may hold fewer blocks); with `a`, writes the
// item prefix into its inline table (after set_inline) and the item total.
int64_t item_prefix(const RankTables& rt, const HostWork& w, size_t i0, size_t i1, int form, StepArgs* a) {
    const int64_t per = item_blocks(form);
    int64_t tot = 0;
    for (size_t i = i0; i < i1; ++i) {
        if (a) a->inl_prefix[i - i0] = tot;
        tot += ceil_div(rt.segs[(size_t)w.seg_idx[i]].nblocks, per);
    }
    if (a) {
        a->inl_prefix[i1 - i0] = tot;
        a->work.total = tot;
    }
    return tot;
}

// Workgroup path shape: threads and 4-element groups per thread for blocks
// of up to `groups` groups (each run of segments with one shape is a launch).
// Measured on MI355X over the model workloads:
//   2,049 .. 4,096 groups (128x128 tiles): 1024 threads x 4 (two resident
//     workgroups per CU) beat 512 x 8 by ~2%;
//   4,097 .. 12,288 groups (row blocks of 16K..48K elements), persistent
//     form: the shape with the fewest idle lanes, then the most threads.
//     28,672-element rows: 1024 x 7 5.95 TB/s, 512 x 14 5.90, 512 x 16 and
//     768 x 10 5.85; 46,080-element rows: 768 x 15 5.61, 512 x 24 5.57.
//     With the persistent form off (option wg_dynamic = 0): 512 threads
//     with 16, 20 or 24 groups, which beat 1024 threads there by 1-2%;
//   larger: 1024 threads x 14 / 16;
//   up to 2,048 groups: the largest workgroup that gives each thread at
//     least 6 groups (fewer leave the per-block prologue exposed), else 256.
// The options wg_threads / wg_gpt pin it (launch-shape tuning) for blocks
// that fit the pinned shape.
void wg_shape(int32_t groups, int& threads, int& gpt, bool persistent) {
    const int64_t ot = option(kOptWgThreads), og = option(kOptWgGpt);
    if (ot > 0 && og > 0 && ot <= kWgMaxThreads && og <= 64) {
        threads = (int)ot;
        gpt = (int)og;
        if (wg_config_supported(threads, gpt) && (int64_t)threads * gpt >= groups) return;
    }
    auto fit = [&](int t, int min_g, int& g) {
        for (g = std::max(min_g, (int)ceil_div(groups, t)); g <= 32; ++g)
            if (wg_config_supported(t, g)) return true;
        return false;
    };
    int g = 0;
    if (groups > 2048 && groups <= 4096 && fit(1024, 1, g)) {
        threads = 1024;
        gpt = g;
        return;
    }
    if (groups > 4096 && groups <= 12288 && persistent) {
        // idle fraction (t * g - groups) / (t * g), compared as fractions
        int64_t bt = 0, bg = 0;
        auto better = [&](int64_t t, int64_t gg) {
            if (bt == 0) return true;
            const int64_t a = (t * gg - groups) * (bt * bg), b = (bt * bg - groups) * (t * gg);
            return a < b || (a == b && t > bt);
        };
#define VE_WG_CASE(T, G) \
        if (dyn_shape(T, G) && (int64_t)(T) * (G) >= groups && better(T, G)) { bt = T; bg = G; }
        VE_WG_SHAPES(VE_WG_CASE)
#undef VE_WG_CASE
        if (bt > 0) {
            threads = (int)bt;
            gpt = (int)bg;
            return;
        }
    }
    if (groups > 4096 && groups <= 12288 && fit(512, 16, g)) {
        threads = 512;
        gpt = g;
        return;
    }
    if (groups > 12288 && fit(1024, 1, g)) {
        threads = 1024;
        gpt = g;
        return;
    }
    for (int t : {1024, 512}) {
        if (ceil_div(groups, t) >= 6 && fit(t, 1, g)) {
            threads = t;
            gpt = g;
            return;
        }
    }
    for (int t : {256, 512, 1024}) {
        if (fit(t, 1, g)) {
            threads = t;
            gpt = g;
            return;
        }
    }
    threads = 1024;  // unreachable for blocks classed kWg (groups <= kWgMaxGroups)
    gpt = 16;
}

struct DeviceGuard {
    int prev = -1;
    bool ok = false;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        ok = hipSetDevice(dev) == hipSuccess;
    }
    ~DeviceGuard() {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

ve_status launch_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return VE_OK;
    return fail(VE_ERR_DEVICE, "%s launch failed: %s", what, hipGetErrorString(e));
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
extern "C" {

const char* ve_last_error(void) { return g_err.c_str(); }

ve_status ve_set_option(const char* name, int64_t value) {
    const int i = option_index(name);
    if (i < 0) return fail(VE_ERR_INVALID_ARG, "unknown option %s", name ? name : "(NULL)");
    std::call_once(g_options_once, seed_options);
    g_options[i].store(value, std::memory_order_relaxed);
    return VE_OK;
}

ve_status ve_get_option(const char* name, int64_t* value) {
    const int i = option_index(name);
    if (i < 0) return fail(VE_ERR_INVALID_ARG, "unknown option %s", name ? name : "(NULL)");
    if (!value) return fail(VE_ERR_INVALID_ARG, "value is NULL");
    *value = option((Option)i);
    return VE_OK;
}

ve_status ve_plan_load(const ve_tensor_spec* specs, int32_t n_tensors, int32_t fsdp_size, int64_t shard_elems,
                       int32_t device, ve_plan** out) {
    try {
        if (!out) return fail(VE_ERR_INVALID_ARG, "out is NULL");
        *out = nullptr;
        if (n_tensors > 0 && !specs) return fail(VE_ERR_INVALID_ARG, "specs is NULL");
        int ndev = 0;
        if (device != -1 && (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev))
            return fail(VE_ERR_INVALID_ARG, "device %d not available (%d devices)", device, ndev);
        auto P = new ve_plan();
        P->device = device;
        P->m = fsdp_size;
        P->S = shard_elems;
        P->specs.assign(specs, specs + (n_tensors > 0 ? n_tensors : 0));
        ve_status st = validate(P->specs.data(), n_tensors, fsdp_size, shard_elems, P->order);
        if (st != VE_OK) {
            delete P;
            return st;
        }
        P->ranks.resize((size_t)fsdp_size);
        P->sched_order.resize((size_t)fsdp_size);
        for (int32_t r = 0; r < fsdp_size; ++r) build_rank(*P, r, P->ranks[(size_t)r]);
        build_whole(*P);
        Packer pk;
        for (auto& rt : P->ranks) {
            rt.off_segs = pk.put(rt.segs);
            pack_work(pk, rt.small);
            pack_work(pk, rt.wg);
            pack_work(pk, rt.huge);
            pack_runs(pk, rt.copy);
            pack_runs(pk, rt.pad);
        }
        pack_runs(pk, P->whole);
        // one 64-byte line of scheduler counters per rank, zero at load
        P->off_sched = pk.put(std::vector<uint32_t>((size_t)fsdp_size * kSchedStride / sizeof(uint32_t), 0u));
        P->dev_bytes = std::max<size_t>(pk.buf.size(), 256);
        if (device == -1) {  // host-only plan: layout queries, no kernels
            *out = P;
            return VE_OK;
        }
        DeviceGuard g(device);
        if (!g.ok) {
            delete P;
            return fail(VE_ERR_DEVICE, "hipSetDevice(%d) failed", device);
        }
        if (hipDeviceGetAttribute(&P->n_cu, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
            P->n_cu <= 0) {
            delete P;
            return fail(VE_ERR_DEVICE, "cannot read the compute-unit count of device %d", device);
        }
        if (hipMalloc((void**)&P->dev, P->dev_bytes) != hipSuccess) {
            delete P;
            return fail(VE_ERR_OOM, "hipMalloc of %zu bytes of plan tables failed", pk.buf.size());
        }
        if (!pk.buf.empty() && hipMemcpy(P->dev, pk.buf.data(), pk.buf.size(), hipMemcpyHostToDevice) != hipSuccess) {
            (void)hipFree(P->dev);
            delete P;
            return fail(VE_ERR_DEVICE, "upload of plan tables failed");
        }
        *out = P;
        return VE_OK;
    } catch (const std::bad_alloc&) {
        return fail(VE_ERR_OOM, "host allocation failed while building the plan");
    } catch (...) {
        return fail(VE_ERR_DEVICE, "unexpected host exception in ve_plan_load");
    }
}

ve_status ve_plan_free(ve_plan* plan) {
    if (!plan) return VE_OK;
    ve_status st = VE_OK;
    if (plan->dev && plan->device >= 0) {
        DeviceGuard g(plan->device);
        for (auto& o : plan->sched_order)
            if (o.done && hipEventDestroy(o.done) != hipSuccess) st = fail(VE_ERR_DEVICE, "hipEventDestroy failed");
        if (hipFree(plan->dev) != hipSuccess) st = fail(VE_ERR_DEVICE, "hipFree of plan tables failed");
    }
    delete plan;
    return st;
}

ve_status ve_plan_query(const ve_plan* plan, int32_t rank, int64_t* valid_elems, int64_t* n_blocks,
                        int32_t* n_segments) {
    if (!plan) return fail(VE_ERR_INVALID_ARG, "plan is NULL");
    if (rank < 0 || rank >= plan->m) return fail(VE_ERR_INVALID_ARG, "rank %d outside [0, %d)", rank, plan->m);
    const RankTables& rt = plan->ranks[(size_t)rank];
    if (valid_elems) *valid_elems = rt.valid;
    if (n_blocks) *n_blocks = rt.nblocks;
    if (n_segments) *n_segments = (int32_t)rt.segs.size();
    return VE_OK;
}

ve_status ve_dbuffer_slice(const ve_plan* plan, int32_t rank, int32_t tensor, int64_t* shard_offset,
                           int64_t* elem_start, int64_t* elem_end) {
    if (!plan) return fail(VE_ERR_INVALID_ARG, "plan is NULL");
    if (!shard_offset || !elem_start || !elem_end) return fail(VE_ERR_INVALID_ARG, "output pointer is NULL");
    if (rank < -1 || rank >= plan->m) return fail(VE_ERR_INVALID_ARG, "rank %d outside [-1, %d)", rank, plan->m);
    if (tensor < 0 || tensor >= (int32_t)plan->specs.size())
        return fail(VE_ERR_INVALID_ARG, "tensor %d outside [0, %zu)", tensor, plan->specs.size());
    const ve_tensor_spec& t = plan->specs[(size_t)tensor];
    const int64_t numel = t.rows * t.cols;
    if (rank < 0) {
        *shard_offset = t.offset;
        *elem_start = 0;
        *elem_end = numel;
        return VE_OK;
    }
    const int64_t c0 = (int64_t)rank * plan->S;
    const int64_t a = std::max(t.offset, c0), b = std::min(t.offset + numel, c0 + plan->S);
    if (a >= b) {
        *shard_offset = -1;
        *elem_start = *elem_end = 0;
    } else {
        *shard_offset = a - c0;
        *elem_start = a - t.offset;
        *elem_end = b - t.offset;
    }
    return VE_OK;
}

ve_status ve_dbuffer_copy_in(const ve_plan* plan, int32_t rank, const uint16_t* const* grad_ptrs, uint16_t* bucket,
                             void* stream) {
    if (!plan) return fail(VE_ERR_INVALID_ARG, "plan is NULL");
    if (rank < -1 || rank >= plan->m) return fail(VE_ERR_INVALID_ARG, "rank %d outside [-1, %d)", rank, plan->m);
    if (!bucket) return fail(VE_ERR_INVALID_ARG, "bucket is NULL");
    if (!plan->dev) return fail(VE_ERR_INVALID_ARG, "host-only plan (device -1) cannot launch kernels");
    const HostRuns& h = rank < 0 ? plan->whole : plan->ranks[(size_t)rank].copy;
    bool needs_grads = false;
    for (const Run& r : h.runs) needs_grads |= r.tensor >= 0;
    if (needs_grads && !grad_ptrs) return fail(VE_ERR_INVALID_ARG, "grad_ptrs is NULL");
    if (h.tile_prefix.back() == 0) return VE_OK;
    if (h.tile_prefix.back() > kMaxRunTiles)
        return fail(VE_ERR_UNSUPPORTED, "%lld tiles exceed one launch", (long long)h.tile_prefix.back());
    DeviceGuard g(plan->device);
    if (!g.ok) return fail(VE_ERR_DEVICE, "hipSetDevice(%d) failed", plan->device);
    (void)hipGetLastError();
    return launch_status(launch_runs_copy(run_args(*plan, h), grad_ptrs, bucket, (hipStream_t)stream), "copy-in");
}

ve_status ve_dbuffer_group_op(const ve_plan* plan, int32_t rank, int32_t op, float alpha,
                              const ve_group_operand* operands, int32_t n_operands, void* stream) {
    if (!plan) return fail(VE_ERR_INVALID_ARG, "plan is NULL");
    if (rank < -1 || rank >= plan->m) return fail(VE_ERR_INVALID_ARG, "rank %d outside [-1, %d)", rank, plan->m);
    if (op != VE_GROUP_ZERO && op != VE_GROUP_SCALE && op != VE_GROUP_ACCUMULATE)
        return fail(VE_ERR_INVALID_ARG, "unknown group op %d", op);
    if (n_operands < 0 || n_operands > 65535)
        return fail(VE_ERR_INVALID_ARG, "n_operands %d outside [0, 65535]", n_operands);
    if (n_operands > 0 && !operands) return fail(VE_ERR_INVALID_ARG, "operands is NULL");
    if (!plan->dev) return fail(VE_ERR_INVALID_ARG, "host-only plan (device -1) cannot launch kernels");
    const HostRuns& h = rank < 0 ? plan->whole : plan->ranks[(size_t)rank].copy;
    if (n_operands == 0 || h.tile_prefix.back() == 0) return VE_OK;
    if (h.tile_prefix.back() > kMaxRunTiles)
        return fail(VE_ERR_UNSUPPORTED, "%lld tiles exceed one launch", (long long)h.tile_prefix.back());
    DeviceGuard g(plan->device);
    if (!g.ok) return fail(VE_ERR_DEVICE, "hipSetDevice(%d) failed", plan->device);
    (void)hipGetLastError();
    return launch_status(launch_group(run_args(*plan, h), op, alpha, operands, n_operands, (hipStream_t)stream),
                         "group op");
}

ve_status ve_stream_copy(void* dst, const void* src, int64_t bytes, void* stream) {
    if (bytes < 0) return fail(VE_ERR_INVALID_ARG, "bytes %lld < 0", (long long)bytes);
    if (bytes == 0) return VE_OK;
    if (!dst || !src) return fail(VE_ERR_INVALID_ARG, "NULL buffer");
    if ((((uintptr_t)dst | (uintptr_t)src | (uintptr_t)bytes) & 15) != 0)
        return fail(VE_ERR_INVALID_ARG, "buffers and size must be multiples of 16 bytes");
    const uintptr_t d = (uintptr_t)dst, s0 = (uintptr_t)src;
    if (d < s0 + (uintptr_t)bytes && s0 < d + (uintptr_t)bytes) return fail(VE_ERR_INVALID_ARG, "buffers overlap");
    const int64_t vectors = bytes / 16;
    // 16 workgroups per CU of a 256-CU device (measured best of 1024..4096),
    // fewer when the buffer is small
    const int64_t grid = std::min<int64_t>(4096, (vectors + 1023) / 1024);
    (void)hipGetLastError();
    return launch_status(launch_stream_copy(src, dst, vectors, (int)grid, (hipStream_t)stream), "stream copy");
}

ve_status ve_shard_adam8bit_step(const ve_plan* plan, int32_t rank, const ve_shard_state* states, int32_t n_states,
                                 const ve_adam_hparams* hp, int64_t step, void* stream) {
    if (!plan) return fail(VE_ERR_INVALID_ARG, "plan is NULL");
    if (rank < 0 || rank >= plan->m) return fail(VE_ERR_INVALID_ARG, "rank %d outside [0, %d)", rank, plan->m);
    if (!states) return fail(VE_ERR_INVALID_ARG, "states is NULL");
    if (n_states < 1 || n_states > 65535) return fail(VE_ERR_INVALID_ARG, "n_states %d outside [1, 65535]", n_states);
    if (!hp) return fail(VE_ERR_INVALID_ARG, "hparams is NULL");
    if (step < 1) return fail(VE_ERR_INVALID_ARG, "step %lld < 1", (long long)step);
    if (!(hp->beta1 >= 0.f && hp->beta1 < 1.f) || !(hp->beta2 >= 0.f && hp->beta2 < 1.f))
        return fail(VE_ERR_INVALID_ARG, "betas (%g, %g) outside [0, 1)", (double)hp->beta1, (double)hp->beta2);
    if (!std::isfinite(hp->lr) || !std::isfinite(hp->eps) || !std::isfinite(hp->weight_decay) || hp->eps <= 0.f)
        return fail(VE_ERR_INVALID_ARG, "lr / eps / weight_decay must be finite and eps > 0");
    if (!plan->dev) return fail(VE_ERR_INVALID_ARG, "host-only plan (device -1) cannot launch kernels");
    const RankTables& rt = plan->ranks[(size_t)rank];
    if ((rt.small.prefix.back() + 3) / 4 * 256 > kMaxGridItems || rt.wg.prefix.back() * kWgMaxThreads > kMaxGridItems ||
        rt.huge.prefix.back() * 256 > kMaxGridItems || rt.pad.tile_prefix.back() > kMaxRunTiles)
        return fail(VE_ERR_UNSUPPORTED, "rank %d has more blocks than one launch covers", rank);

    // A rank with small blocks and padding zero-fills the padding in the
    // small-block launch (one launch fewer), when the grid allows it.
    const int64_t small_wgs = (rt.small.prefix.back() + 3) / 4;
    const bool fuse_pad = small_wgs > 0 && rt.pad.tile_prefix.back() > 0 &&
                          (small_wgs + rt.pad.tile_prefix.back()) * 256 <= kMaxGridItems;
    StepArgs a{};
    a.states = states;
    a.segs = plan->dptr<Seg>(rt.off_segs);
    a.sched = reinterpret_cast<uint32_t*>(plan->dev + plan->off_sched + (size_t)rank * kSchedStride);
    const double b1 = hp->beta1, b2 = hp->beta2, lr = hp->lr;
    a.sc.beta1 = hp->beta1;
    a.sc.beta2 = hp->beta2;
    a.sc.omb1 = 1.0f - hp->beta1;  // exact: Sterbenz for beta in [0.5, 1); rounded once otherwise
    a.sc.omb2 = 1.0f - hp->beta2;
    a.sc.step_size = (float)(lr / (1.0 - std::pow(b1, (double)step)));
    a.sc.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(1.0 - std::pow(b2, (double)step)));
    a.sc.eps = hp->eps;
    a.sc.decay = (float)(1.0 - lr * (double)hp->weight_decay);

    DeviceGuard g(plan->device);
    if (!g.ok) return fail(VE_ERR_DEVICE, "hipSetDevice(%d) failed", plan->device);
    (void)hipGetLastError();
    hipStream_t s = (hipStream_t)stream;
    ve_status st;
    if (rt.wg.prefix.back() > 0) {
        // One launch per run of consecutive segments whose blocks take the same
        // shape (a rank's segments are sorted by block size, so a rank holding
        // the end of one tensor and most of a tensor with smaller blocks gets
        // two launches instead of running every block in the larger shape).
        // Segments of whole-row blocks of 2,048 or 4,096 groups (rows of 8K
        // or 16K elements) and of 128 x 128 tiles run persistent with items
        // of several blocks (form != kItemNone); see item_form().
        struct WgLaunch {
            size_t i0, i1;
            int threads, gpt, form;
            bool dyn;
        };
        std::vector<WgLaunch> runs;
        bool any_dyn = false;
        const size_t n = rt.wg.seg_idx.size();
        auto shape_of = [&](size_t i, int& t, int& g, int& r) {
            const Seg& sg = rt.segs[(size_t)rt.wg.seg_idx[i]];
            wg_shape(sg.max_groups, t, g, option(kOptWgDynamic) != 0);
            r = item_form(sg);
        };
        // Persistent launches pay a fixed cost (about 9 us a launch, 13 us with
        // row items) that only enough work hides: measured on MI355X, LLaMA
        // rows, against the one-shot launch: 28,672-element rows from about
        // 5 blocks per CU on (6 buckets of rank 0: 23.6 against 24.0 us a
        // bucket; 1 bucket: 37.0 against 28.0 us), row items from about 32
        // per CU on (48 buckets of rank 36: 20.7 against 21.1 us a bucket;
        // 16 buckets: 21.8 against 21.0).  Below that, the run takes the
        // one-shot shapes; wg_dynamic = 2 keeps the persistent forms anyway.
        const int64_t dyn_opt = option(kOptWgDynamic);
        auto push_runs = [&](size_t i0, size_t i1, bool persistent) {
            for (size_t a0 = i0; a0 < i1;) {
                int threads = 256, gpt = 1;
                wg_shape(rt.segs[(size_t)rt.wg.seg_idx[a0]].max_groups, threads, gpt, persistent);
                size_t a1 = a0 + 1;
                for (int t1, g1; a1 < i1; ++a1) {
                    wg_shape(rt.segs[(size_t)rt.wg.seg_idx[a1]].max_groups, t1, g1, persistent);
                    if (t1 != threads || g1 != gpt) break;
                }
                runs.push_back({a0, a1, threads, gpt, kItemNone, false});
                a0 = a1;
            }
        };
        for (size_t i0 = 0; i0 < n;) {
            int threads = 256, gpt = 1, form = kItemNone;
            shape_of(i0, threads, gpt, form);
            size_t i1 = i0 + 1;
            for (int t1, g1, f1; i1 < n && i1 - i0 < (size_t)kInlineSegs; ++i1) {
                shape_of(i1, t1, g1, f1);
                if (t1 != threads || g1 != gpt || f1 != form) break;
            }
            const int64_t items = form != kItemNone ? item_prefix(rt, rt.wg, i0, i1, form, nullptr)
                                                    : rt.wg.prefix[i1] - rt.wg.prefix[i0];
            // Row-block shapes run persistent, the resident workgroups taking
            // blocks from the rank's counters; tickets stay below 2^31.
            const bool fits = items * n_states + (int64_t)kDynMaxPerCu * plan->n_cu < (int64_t(1) << 31);
            const bool candidate = dyn_opt != 0 && (form != kItemNone || wg_dynamic_shape(threads, gpt));
            const int64_t min_work = (form != kItemNone ? kItemMinPerCu : kDynMinPerCu) * (int64_t)plan->n_cu;
            if (candidate && (!fits || (dyn_opt != 2 && items * n_states < min_work))) {
                push_runs(i0, i1, false);  // one-shot shapes
            } else {
                const bool dyn = items > 0 && candidate;
                runs.push_back({i0, i1, threads, gpt, form, dyn});
                any_dyn = any_dyn || dyn;
            }
            i0 = i1;
        }
        // The counters admit one launch at a time.  Launches on one stream
        // run one after another; a call on another stream than the rank's
        // last one that used them first waits (on the GPU) for that call's
        // launches.  Under stream capture no event is recorded or waited on:
        // a captured step must not overlap other calls for this plan and rank.
        std::unique_lock<std::mutex> order_lock;
        bool capturing = false;
        if (any_dyn) {
            order_lock = std::unique_lock<std::mutex>(plan->sched_mu);
            hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
            if (hipStreamIsCapturing(s, &cs) != hipSuccess)
                return fail(VE_ERR_DEVICE, "hipStreamIsCapturing failed");
            capturing = cs != hipStreamCaptureStatusNone;
            const auto& o = plan->sched_order[(size_t)rank];
            if (!capturing && o.used && o.stream != s && hipStreamWaitEvent(s, o.done, 0) != hipSuccess)
                return fail(VE_ERR_DEVICE, "hipStreamWaitEvent on the rank's previous step failed");
        }
        for (const WgLaunch& w : runs) {
            if (w.form != kItemNone) {
                if (set_inline(a, rt, rt.wg, w.i0, w.i1) == 0) continue;
                item_prefix(rt, rt.wg, w.i0, w.i1, w.form, &a);
                if ((st = launch_status(launch_step_items(a, n_states, w.form, plan->n_cu, s),
                                        "multi-block item step")) != VE_OK)
                    return st;
                continue;
            }
            if (set_inline(a, rt, rt.wg, w.i0, w.i1) == 0) continue;
            if ((st = launch_status(launch_step_wg(a, n_states, w.threads, w.gpt, w.dyn ? plan->n_cu : 0, s),
                                    "workgroup step")) != VE_OK)
                return st;
        }
        if (any_dyn && !capturing) {
            auto& o = plan->sched_order[(size_t)rank];
            if (!o.done && hipEventCreateWithFlags(&o.done, hipEventDisableTiming) != hipSuccess)
                return fail(VE_ERR_DEVICE, "hipEventCreateWithFlags failed");
            if (hipEventRecord(o.done, s) != hipSuccess) return fail(VE_ERR_DEVICE, "hipEventRecord failed");
            o.stream = s;
            o.used = true;
        }
    }
    if (rt.small.prefix.back() > 0) {
        set_work(a, *plan, rt.small);
        // few segments: hand them to the kernel inline (no table lookups)
        if (rt.small.seg_idx.size() <= (size_t)kInlineSegs) set_inline(a, rt, rt.small, 0, rt.small.seg_idx.size());
        if (fuse_pad) a.pad = run_args(*plan, rt.pad);  // the padding fill rides along
        if ((st = launch_status(launch_step_small(a, n_states, s), "small-block step")) != VE_OK) return st;
        a.pad = RunArgs{};
    }
    if (rt.huge.prefix.back() > 0) {
        for (size_t i0 = 0; i0 < rt.huge.seg_idx.size(); i0 += kInlineSegs) {
            const size_t i1 = std::min(rt.huge.seg_idx.size(), i0 + (size_t)kInlineSegs);
            if (set_inline(a, rt, rt.huge, i0, i1) == 0) continue;
            if ((st = launch_status(launch_step_huge(a, n_states, s), "large-block step")) != VE_OK) return st;
        }
    }
    if (rt.pad.tile_prefix.back() > 0 && !fuse_pad) {
        if ((st = launch_status(launch_runs_pad(run_args(*plan, rt.pad), states, n_states, s), "padding fill")) != VE_OK)
            return st;
    }
    return VE_OK;
}

}  // extern "C"
