"""Benchmark of the fused RaggedShard shard step on one MI355X.

One step = one ``ve_shard_adam8bit_step`` call over every bucket of the
workload on one rank (group copy-in of the bf16 gradients, block-wise 8-bit
AdamW with one absmax scale per block, bf16 parameter write-back).  Default
workload: LLaMA-3-70B-shaped buckets, 80 layers, 1-row blocks, FSDP size 128,
rank 0 (6,709,248 elements and 234 blocks of 28,672 per bucket).  Inputs are
synthetic, seeded, resident in HBM before timing.

Prints one JSON line on stdout; progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--workload llama|gptoss|deepseek|adversarial]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak
METRIC = "fused shard-step HBM GB/s and params/s on 1 GPU; % of HBM peak"
# algorithmic bytes: per valid element, per quantisation block, per padding element
BYTES_PER_ELEM = 18   # grad read 2 + grad-slice write 2 + master r/w 8 + codes r/w 4 + bf16 param write 2
BYTES_PER_BLOCK = 16  # two fp32 scales read + written
BYTES_PER_PAD = 4     # two bf16 zero writes
# DBuffer group operations: algorithmic bytes per tensor element (padding: one bf16 write)
GROUP_BYTES = {"zero": 2, "scale": 4, "accumulate": 6}
GROUP_PAD_BYTES = 2


def log(msg):
    print(msg, file=sys.stderr, flush=True)


STEP_SOURCES = ("ve_kernels.hip", "ve_device.h", "ve_internal.h", "ve_host.cpp")
GROUP_SOURCES = ("ve_group.hip", "ve_device.h", "ve_internal.h", "ve_host.cpp")
MUON_SOURCES = ("ve_muon.hip", "ve_muon.h", "ve_muon_host.cpp", "ve_device.h", "ve_internal.h")


def strip_comments(src: str) -> str:
    """C/C++ source without its comments, each run of blank space made one
    space: what the compiler sees, up to layout.  String and character
    literals are kept as they are."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(files=STEP_SOURCES):
    """Hash of the kernel sources with comments and layout removed, so that
    a profile stays valid across comment edits and is dropped by any code
    change."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "ragged_shard_optimizer_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(strip_comments(fh.read()).encode())
    return h.hexdigest()[:16]


def _profile(name, files):
    """A committed rocprofv3 counter summary, if it was taken on the current
    kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("kernel_source_hash") != kernel_source_hash(files):
        return None
    return d


def measured_traffic(workload):
    """HBM bytes per launch of the step kernel from the committed counters."""
    d = _profile(f"shard_step_{workload}_traffic.json", STEP_SOURCES)
    return None if d is None else d.get("hbm_bytes_per_launch")


def measured_group_traffic(workload):
    """{op: HBM bytes per launch} of the group kernels from the committed counters."""
    d = _profile(f"dbuffer_group_{workload}_traffic.json", GROUP_SOURCES)
    return None if d is None else d.get("hbm_bytes_per_launch")


def host_cores():
    """(threads the CPU legs use, CPUs visible to this process): the visible
    CPUs, capped by OMP_NUM_THREADS when that is set (the machine's CPU share)."""
    try:
        visible = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        visible = os.cpu_count() or 1
    share = os.environ.get("OMP_NUM_THREADS", "")
    threads = min(visible, int(share)) if share.isdigit() and int(share) > 0 else visible
    return threads, visible


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(cfg, lay, rank, budget_s=8.0):
    """The oracle (plain C, fp64 updates) on a bounded sample of the same
    workload: bucket 0 of the rank's shard, with the workload's seeded
    inputs (the rank's gradient pieces, its master shard), stepped over and
    over for about ``budget_s`` seconds per leg.  Two legs: one host thread,
    and the rank's blocks split over every host thread this process may use
    (bit-identical results).  Input generation is not timed."""
    import oracle
    from synth import HPARAMS
    from synth.data import host_master, host_piece_grads
    spec, S = lay.spec_array(), lay.shard
    hp = dict(HPARAMS)
    grads, bases = host_piece_grads(cfg, lay, 0, rank, step=1)
    st = oracle.new_state(spec, S, rank, host_master(cfg, lay, 0, rank))
    nb, nv = oracle.rank_blocks(spec, S, rank)
    alg = BYTES_PER_ELEM * nv + BYTES_PER_BLOCK * nb + BYTES_PER_PAD * (S - nv)
    threads, visible = host_cores()
    step = 1
    oracle.shard_step(spec, lay.fsdp, S, rank, grads, st, hp, step, bases=bases)  # warm (step 1 from zero)
    legs = {}
    for name, nthr in (("single_thread", 1), ("all_threads", threads)):
        done, t0 = 0, time.perf_counter()
        while True:
            step += 1
            oracle.shard_step_threads(spec, lay.fsdp, S, rank, grads, st, hp, step, bases=bases, threads=nthr)
            done += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
        legs[name] = {"threads": nthr, "steps": done, "seconds": round(el, 3),
                      "value": round(alg * done / el / 1e9, 4), "params_per_s": round(nv * done / el, 1)}
        log(f"[bench] oracle {name} ({nthr} threads): {legs[name]['value']} GB/s")
    best = legs["all_threads"]
    return {"value": best["value"], "unit": "GB/s", "cores": best["threads"], "kind": "oracle",
            "params_per_s": best["params_per_s"],
            "single_thread": legs["single_thread"], "all_threads": legs["all_threads"],
            "host": {"cpus_visible": visible, "cpu_model": cpu_model()},
            "sample": f"bucket 0 of rank {rank} ({nv} elements, {nb} blocks; the workload's seeded gradient "
                      f"pieces and master shard), stepped repeatedly for ~{budget_s:.0f} s on 1 thread and "
                      f"~{budget_s:.0f} s on {best['threads']} threads (blocks split over the threads); "
                      f"value is the {best['threads']}-thread rate"}


def time_group_ops(torch, ve, plan, rank, states, lay, valid, steps, warmup, traffic=None):
    """Each DBuffer group operation over every bucket's rank chunk (the
    states' gradient slices) in one launch: HIP events on the launch stream,
    algorithmic bytes per launch over the mean launch time."""
    stream = torch.cuda.current_stream()
    bufs = [st["grad_shard"] for st in states]
    gts = [st["grad_table"] for st in states]
    S, nbk = lay.shard, len(states)
    out = {}
    for name, op, alpha in (("zero", ve.GROUP_ZERO, 0.0), ("scale", ve.GROUP_SCALE, 0.999),
                            ("accumulate", ve.GROUP_ACCUMULATE, 1.0)):
        table = ve.group_table(plan, rank, bufs, gts if op == ve.GROUP_ACCUMULATE else None)
        for _ in range(warmup):
            plan.group_op(rank, op, alpha, table, stream)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            a.record(stream)
            plan.group_op(rank, op, alpha, table, stream)
            b.record(stream)
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in ev) / steps
        per_elem = GROUP_BYTES[name]
        alg = nbk * (S * per_elem if name == "zero" else per_elem * valid + GROUP_PAD_BYTES * (S - valid))
        gbs = alg / (ms / 1e3) / 1e9
        t = None if not traffic or name not in traffic else traffic[name] / (ms / 1e3) / 1e9
        out[name] = {"ms": round(ms, 5), "alg_bytes": alg, "achieved": round(gbs, 2),
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if t is None else round(t, 2)}
        log(f"[bench] group {name}: {ms:.4f} ms, {gbs:.1f} GB/s")
    return {"bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s", "buckets": nbk,
            "bytes_per_elem": GROUP_BYTES, "bytes_per_pad": GROUP_PAD_BYTES, "ops": out}


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
# Muon's published quintic coefficients (a, b, c) of X <- a X + (b A + c A^2) X
NS_COEFFS = (3.4445, -4.7750, 2.0315)


def ns_flops(rows, cols, steps=5):
    """Work of the Newton-Schulz iteration counted the minimal way, two flops
    per multiply-add: with m = min(rows, cols) and n = max, each step is
    X X^T (symmetric, m*m*n multiply-adds), A A (symmetric, m^3) and B X
    (2*m*m*n)."""
    m, n = min(rows, cols), max(rows, cols)
    return steps * (3 * m * m * n + m * m * m)


def time_muon(torch, ve, dev, rows=8192, cols=28672, steps=3, warmup=1, name="LLaMA-3-70B MLP"):
    """Muon's Newton-Schulz iteration (5 steps) on one gathered matrix (by
    default of the LLaMA-3-70B MLP shape), HIP events on the launch stream;
    flops counted the minimal way (symmetric products at half cost)."""
    stream = torch.cuda.current_stream()
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    G = torch.randn(rows, cols, generator=g, device=dev).to(torch.bfloat16).view(torch.int16)
    out = torch.empty_like(G)
    ws = torch.empty(ve.muon_workspace_bytes(rows, cols), dtype=torch.uint8, device=dev)
    for _ in range(warmup):
        ve.muon_newton_schulz(G, out, 5, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        ve.muon_newton_schulz(G, out, 5, workspace=ws, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    flops = ns_flops(rows, cols)
    tf = flops / (ms / 1e3) / 1e12
    log(f"[bench] muon newton-schulz {rows}x{cols}: {ms:.3f} ms, {tf:.1f} TFLOP/s")
    del G, out, ws
    torch.cuda.empty_cache()
    # context: the same iteration in torch (hipBLASLt products with the scalars
    # fused into addmm), timed the same way
    m, n = min(rows, cols), max(rows, cols)
    X = torch.randn(m, n, device=dev, dtype=torch.bfloat16, generator=g) / (m * n) ** 0.5
    a_, b_, c_ = NS_COEFFS

    def torch_ns(X):
        for _ in range(5):
            A = X @ X.t()
            B = torch.addmm(A, A, A, beta=b_, alpha=c_)
            X = torch.addmm(X, B, X, beta=a_)
        return X
    torch_ns(X)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        torch_ns(X)
    t1.record(stream)
    torch.cuda.synchronize()
    tms = t0.elapsed_time(t1) / steps
    log(f"[bench] torch addmm iteration for comparison: {tms:.3f} ms")
    del X
    torch.cuda.empty_cache()
    return {"workload": f"Muon Newton-Schulz, 5 steps, one {rows}x{cols} bf16 matrix ({name})",
            "bound": "mfma", "ms": round(ms, 4), "flops": flops, "achieved": round(tf, 1),
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "torch_addmm_ms": round(tms, 4)}


def time_planner(ve, sizes=(64, 256, 1024)):
    """The structure-aware planner (host) on the models the pages evaluate it
    on, per FSDP size: whole-model padding and planning time with one bucket
    per layer (each distinct bucket planned once), and with the layers
    grouped into buckets by ve_plan_buckets."""
    import numpy as np
    from synth.models import MODELS, PLANNER_GRANULARITIES
    out = {}
    for name, fn in MODELS.items():
        for g in PLANNER_GRANULARITIES:
            buckets = fn(g)
            for m in sizes:
                t0 = time.perf_counter()
                cache, pad, alloc, lb_pad, lb_alloc = {}, 0, 0, 0, 0
                for b in buckets:
                    sh = np.array([[t.rows, t.cols, t.block_rows] for t in b], dtype=np.int64)
                    key = sh.tobytes()
                    if key not in cache:
                        _, S, lb = ve.plan_layout(sh, m)
                        cache[key] = (S, lb)
                    S, lb = cache[key]
                    total = int((sh[:, 0] * sh[:, 1]).sum())
                    pad += m * S - total
                    alloc += m * S
                    lb_pad += m * lb - total
                    lb_alloc += m * lb
                secs = time.perf_counter() - t0
                units = [np.array([[t.rows, t.cols, t.block_rows] for t in b], dtype=np.int64) for b in buckets]
                t1 = time.perf_counter()
                grouped = ve.plan_buckets(units, m)
                gsecs = time.perf_counter() - t1
                total = sum(int((u[:, 0] * u[:, 1]).sum()) for u in units)
                galloc = sum(m * S for *_, S in grouped)
                out[f"{name} rows/unit {g} fsdp {m}"] = {
                    "per_layer_padding_pct": round(100 * pad / alloc, 4),
                    "per_layer_lower_bound_pct": round(100 * lb_pad / lb_alloc, 4),
                    "per_layer_seconds": round(secs, 4),
                    "grouped_padding_pct": round(100 * (galloc - total) / galloc, 4),
                    "grouped_buckets": len(grouped), "layer_buckets": len(buckets),
                    "grouped_seconds": round(gsecs, 4)}
    log(f"[bench] planner: {len(out)} model/granularity/FSDP cases")
    return out


def whole_bucket_grads(torch, cfg, lay, dev):
    """Every tensor's bf16 gradient of bucket 0 (flat int16 views, drawn a
    few hundred million elements per launch)."""
    from synth.workload import whole_bucket_grads as draw
    return draw(cfg, lay, dev)


def time_copy_in_whole(torch, ve, plan, lay, grads, dev, reps=10, warmup=2):
    """Whole-bucket group copy-in (``ve_dbuffer_copy_in`` with rank -1): every
    tensor's bf16 gradient into the m*S bucket that the reduce-scatter reads,
    padding written as 0.  Algorithmic bytes: 4 per tensor element (read +
    write), 2 per padding element.  HIP events on the launch stream."""
    n = lay.fsdp * lay.shard
    elems = sum(t.numel for t in lay.tensors)
    alg = 4 * elems + 2 * (n - elems)
    gt = ve.grad_pointer_table(grads, dev)
    bucket = torch.empty(n, dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        plan.copy_in(-1, gt, bucket, stream)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        plan.copy_in(-1, gt, bucket, stream)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    gbs = alg / (ms / 1e3) / 1e9
    log(f"[bench] whole-bucket copy-in: {ms:.4f} ms, {gbs:.0f} GB/s")
    del bucket
    return {"bound": "hbm", "bucket_elems": n, "tensor_elems": elems, "alg_bytes": alg, "ms": round(ms, 5),
            "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}


def rank_sweep(torch, ve, plan, lay, grads, dev, reps=10):
    """The fused step on one bucket for every rank of the FSDP group in turn
    (one bucket per call, so a call is ~20 us and launch gaps count): each
    rank's time per call, as min / median / max over the ranks."""
    import statistics
    gt = ve.grad_pointer_table(grads, dev)
    S = lay.shard
    from synth import HPARAMS
    hp = dict(HPARAMS)
    stream = torch.cuda.current_stream()
    master = torch.zeros(S, dtype=torch.float32, device=dev)
    rows = []
    for r in range(lay.fsdp):
        valid, nblocks, _ = plan.query(r)
        st = ve.new_state(plan, r, gt, master)
        table = ve.state_table(plan, r, [st])
        plan.step(r, table, hp, 1, stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(reps):
            plan.step(r, table, hp, 2 + i, stream)
        b.record(stream)
        b.synchronize()
        ms = a.elapsed_time(b) / reps
        alg = BYTES_PER_ELEM * valid + BYTES_PER_BLOCK * nblocks + BYTES_PER_PAD * (S - valid)
        rows.append((ms, alg / (ms / 1e3) / 1e9))
        del st, table
    us = sorted(1e3 * ms for ms, _ in rows)
    gb = sorted(g for _, g in rows)
    log(f"[bench] rank sweep: {us[0]:.1f} / {statistics.median(us):.1f} / {us[-1]:.1f} us per call")
    return {"ranks": lay.fsdp, "buckets_per_call": 1, "calls_per_rank": reps,
            "us_per_call": {"min": round(us[0], 2), "median": round(statistics.median(us), 2), "max": round(us[-1], 2)},
            "gbs": {"min": round(gb[0], 1), "median": round(statistics.median(gb), 1), "max": round(gb[-1], 1)}}


def _hip_memcpy_dtod():
    """hipMemcpyDtoDAsync from the HIP runtime (via ctypes), or None."""
    import ctypes as C
    for name in ("libamdhip64.so", "libamdhip64.so.7", "libamdhip64.so.6"):
        try:
            L = C.CDLL(name)
        except OSError:
            continue
        f = L.hipMemcpyDtoDAsync
        f.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
        f.restype = C.c_int
        return f
    return None


def copy_ceiling(torch, ve, dev, gib, reps=10):
    """The streaming reference on ``gib`` GiB: the library's 16-byte
    non-temporal copy kernel (ve_stream_copy) and the runtime's
    hipMemcpyDtoD on the same buffers; read + write bytes over the time,
    HIP events on the launch stream."""
    import ctypes as C
    nbytes = int(gib * (1 << 30)) // 16 * 16
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    ms = timed(lambda: ve.stream_copy(dst, src, stream))
    assert torch.equal(dst, src)
    out = {"bytes": 2 * nbytes, "kernel": "ve_stream_copy (16-byte non-temporal loads and stores)",
           "ms": round(ms, 5), "gbs": round(2 * nbytes / (ms / 1e3) / 1e9, 2)}
    dtod = _hip_memcpy_dtod()
    if dtod is not None:
        h = C.c_void_p(stream.cuda_stream)
        mt = timed(lambda: dtod(C.c_void_p(dst.data_ptr()), C.c_void_p(src.data_ptr()), nbytes, h))
        out["hipMemcpyDtoD"] = {"ms": round(mt, 5), "gbs": round(2 * nbytes / (mt / 1e3) / 1e9, 2)}
    log(f"[bench] copy ceiling {gib} GiB: stream copy {out['gbs']} GB/s"
        + (f", hipMemcpyDtoD {out['hipMemcpyDtoD']['gbs']} GB/s" if "hipMemcpyDtoD" in out else ""))
    del src, dst
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# rocprofv3 summaries (the text and JSON files under profiles/)

def _csv_rows(path):
    import csv
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def _workload_alg(workload, buckets=None, rank=None):
    """(algorithmic bytes of one all-bucket step launch, buckets, valid, blocks, shard)."""
    from synth import CONFIGS, plan_p0
    import ragged_shard_optimizer_amd as ve
    cfg = CONFIGS[workload]
    lay = plan_p0(cfg.tensors, cfg.fsdp)
    rank = lay.largest_rank() if rank is None else rank
    nv, nb, _ = ve.Plan(lay.spec_array(), lay.fsdp, lay.shard, device=-1).query(rank)
    nbk = buckets or cfg.n_buckets
    alg = nbk * (BYTES_PER_ELEM * nv + BYTES_PER_BLOCK * nb + BYTES_PER_PAD * (lay.shard - nv))
    return alg, nbk, nv, nb, lay.shard


def _grid(r):
    """Work-items of a dispatch (counter rows give Grid_Size, trace rows X/Y/Z)."""
    if "Grid_Size" in r:
        return int(r["Grid_Size"])
    return int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])


def _step_dispatches(rows, weight):
    """The step-kernel rows of the launch that covers every bucket: among
    kernels named k_step_*, the one with the largest total `weight` (duration
    or counter value), at its largest grid (a persistent kernel's grid does
    not grow with the work, so the grid alone cannot pick it)."""
    st = [r for r in rows if "k_step" in r["Kernel_Name"]]
    if not st:
        raise SystemExit("no k_step_* kernel in the profile")
    tot = {}
    for r in st:
        tot[r["Kernel_Name"]] = tot.get(r["Kernel_Name"], 0.0) + weight(r)
    name = max(tot, key=tot.get)
    mine = [r for r in st if r["Kernel_Name"] == name]
    big = max(_grid(r) for r in mine)
    return [r for r in mine if _grid(r) == big]


def _duration(r):
    return float(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))


def _counter(r):
    return float(r["Counter_Value"])


def summarize_counters(args):
    """HBM bytes per launch of the step kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each counter scaled by
    what it reads for the streaming copy of known size in the same run."""
    if args.rank is not None:
        raise SystemExit("counters are summarised for the default rank only (bench.py reads them back there)")
    import statistics
    f_rows = [r for r in _csv_rows(os.path.join(args.fetch_dir, "run_counter_collection.csv"))
              if r["Counter_Name"] == "FETCH_SIZE"]
    w_rows = [r for r in _csv_rows(os.path.join(args.write_dir, "run_counter_collection.csv"))
              if r["Counter_Name"] == "WRITE_SIZE"]
    copy_kib = int(args.copy_gib * (1 << 30)) // 16 * 16 / 1024.0

    def calib(rows):
        v = [float(r["Counter_Value"]) for r in rows if "k_stream_copy" in r["Kernel_Name"]]
        if not v:
            raise SystemExit("no streaming-copy dispatch in the counter run (run bench.py with --copy-gib > 0)")
        return copy_kib / statistics.mean(v), statistics.mean(v)

    fx, fc = calib(f_rows)
    wx, wc = calib(w_rows)
    fs = _step_dispatches(f_rows, _counter)
    ws = _step_dispatches(w_rows, _counter)
    kernel = fs[0]["Kernel_Name"]
    fk = statistics.mean(float(r["Counter_Value"]) for r in fs)
    wk = statistics.mean(float(r["Counter_Value"]) for r in ws)
    rb, wb = fk * fx * 1024, wk * wx * 1024
    alg, nbk, nv, nb, S = _workload_alg(args.workload, args.buckets)
    h = kernel_source_hash(STEP_SOURCES)
    txt = [f"# HBM traffic of the fused shard step, {args.workload} workload (rocprofv3 --pmc)",
           f"kernel sources hash: {h}", "",
           "commands (run from the repository root, on the machine with the GPU), one pass per counter:",
           "  " + args.command_fetch, "  " + args.command_write, "",
           f"calibration: the streaming copy (k_stream_copy) reads and writes {copy_kib:.0f} KiB per dispatch;",
           f"  it reads FETCH_SIZE {fc:.1f} KiB and WRITE_SIZE {wc:.1f} KiB -> FETCH_SIZE x {fx:.4f}, WRITE_SIZE x {wx:.4f}",
           "", f"kernel: {kernel} ({len(fs)} / {len(ws)} dispatches of the all-bucket launch)",
           f"  per dispatch FETCH_SIZE {fk:.1f} KiB, WRITE_SIZE {wk:.1f} KiB",
           f"  HBM bytes per launch: read {rb / 1e9:.4f} GB + write {wb / 1e9:.4f} GB = {(rb + wb) / 1e9:.4f} GB",
           f"  algorithmic bytes per launch ({nbk} buckets x ({BYTES_PER_ELEM} B x {nv} elements + "
           f"{BYTES_PER_BLOCK} B x {nb} blocks + {BYTES_PER_PAD} B x {S - nv} padding)) = {alg / 1e9:.4f} GB",
           f"  measured / algorithmic = {(rb + wb) / alg:.4f}"]
    base = os.path.join(args.profiles_dir, f"shard_step_{args.workload}")
    with open(base + "_hbm_counters.txt", "w") as fh:
        fh.write("\n".join(txt) + "\n")
    summarize_group_counters(args, f_rows, w_rows, fx, wx, fc, wc, copy_kib, nbk, nv, S)
    with open(base + "_traffic.json", "w") as fh:
        json.dump({"kernel": kernel, "kernel_source_hash": h, "hbm_bytes_per_launch": rb + wb, "read_bytes": rb,
                   "write_bytes": wb, "alg_bytes_per_launch": float(alg), "fetch_factor": fx, "write_factor": wx,
                   "summary": f"profiles/shard_step_{args.workload}_hbm_counters.txt"}, fh, indent=1)
    print("\n".join(txt))


def summarize_group_counters(args, f_rows, w_rows, fx, wx, fc, wc, copy_kib, nbk, nv, S):
    """The DBuffer group operations' HBM bytes per launch, when the counter
    runs included them (all buckets' rank chunks per launch)."""
    import statistics
    kinds = {"zero": "k_group<0>", "scale": "k_group<1>", "accumulate": "k_group<2>"}
    if not any(kinds["zero"] in r["Kernel_Name"] for r in f_rows):
        return
    h = kernel_source_hash(GROUP_SOURCES)
    out = [f"# HBM traffic of the DBuffer group operations, {args.workload} workload, all buckets' rank chunks "
           "per launch (rocprofv3 --pmc)", f"kernel sources hash: {h}", "",
           "commands (run from the repository root, on the machine with the GPU), one pass per counter:",
           "  " + args.command_fetch, "  " + args.command_write, "",
           f"calibration: FETCH_SIZE x {fx:.4f}, WRITE_SIZE x {wx:.4f} (the streaming copy of {copy_kib:.0f} KiB "
           f"reads {fc:.1f} / {wc:.1f} KiB)", ""]
    names, hb, ab = {}, {}, {}
    for op, key in kinds.items():
        fr = [r for r in f_rows if key in r["Kernel_Name"]]
        wr = [r for r in w_rows if key in r["Kernel_Name"]]
        if not fr or not wr:
            continue
        rb = statistics.mean(float(r["Counter_Value"]) for r in fr) * fx * 1024
        wb = statistics.mean(float(r["Counter_Value"]) for r in wr) * wx * 1024
        per = GROUP_BYTES[op]
        alg = nbk * (S * per if op == "zero" else per * nv + GROUP_PAD_BYTES * (S - nv))
        names[op], hb[op], ab[op] = fr[0]["Kernel_Name"], rb + wb, float(alg)
        out += [f"{op}: {fr[0]['Kernel_Name']} ({len(fr)} / {len(wr)} dispatches)",
                f"  HBM bytes per launch: read {rb / 1e9:.4f} GB + write {wb / 1e9:.4f} GB = {(rb + wb) / 1e9:.4f} GB; "
                f"algorithmic {alg / 1e9:.4f} GB -> measured / algorithmic = {(rb + wb) / alg:.4f}", ""]
    base = os.path.join(args.profiles_dir, f"dbuffer_group_{args.workload}")
    with open(base + "_hbm_counters.txt", "w") as fh:
        fh.write("\n".join(out).rstrip() + "\n")
    with open(base + "_traffic.json", "w") as fh:
        json.dump({"kernels": names, "kernel_source_hash": h, "hbm_bytes_per_launch": hb, "alg_bytes_per_launch": ab,
                   "summary": f"profiles/dbuffer_group_{args.workload}_hbm_counters.txt"}, fh, indent=1)


def summarize_trace(args):
    """Kernel table and the step kernel's average duration (all-bucket
    launches) from a rocprofv3 --kernel-trace --stats run."""
    import statistics
    stats = _csv_rows(os.path.join(args.trace_dir, "run_kernel_stats.csv"))
    trace = _csv_rows(os.path.join(args.trace_dir, "run_kernel_trace.csv"))
    st = sorted(_step_dispatches(trace, _duration), key=lambda r: int(r["Start_Timestamp"]))
    kernel = st[0]["Kernel_Name"]
    if args.skip_first >= len(st):
        raise SystemExit(f"--skip-first {args.skip_first} leaves none of {len(st)} step dispatches")
    skipped, st = len(st[:args.skip_first]), st[args.skip_first:]
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in st]
    avg = statistics.mean(durs)
    alg, nbk, nv, nb, S = _workload_alg(args.workload, args.buckets, args.rank)
    who = args.workload + ("" if args.rank is None else f" rank {args.rank}")
    t = [f"# Kernel trace of bench.py, {who} workload (rocprofv3 --kernel-trace --stats)", "",
         f"kernel sources hash: {kernel_source_hash(STEP_SOURCES)}", "",
         "command (run from the repository root, on the machine with the GPU):", "  " + args.command, "",
         f"{'kernel':72s} {'calls':>6s} {'avg us':>10s} {'min us':>10s} {'max us':>10s}"]
    for r in stats[:args.top]:
        t.append(f"{r['Name'][:72]:72s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.1f} "
                 f"{float(r['MinNs']) / 1e3:10.1f} {float(r['MaxNs']) / 1e3:10.1f}")
    t += ["", f"step: {kernel}",
          f"  all-bucket launches: average {avg:.1f} us over {len(durs)} dispatches"
          + (f" (the first {skipped}, bench.py's warm-up steps, left out)" if skipped else "")
          + f" (min {min(durs):.1f}, "
          f"max {max(durs):.1f}); algorithmic bytes per launch {alg / 1e9:.4f} GB -> {alg / avg / 1e3:.1f} GB/s "
          f"= {alg / avg / 1e3 / HBM_PEAK_GBS * 100:.1f}% of 8 TB/s"]
    if args.bench_log and os.path.exists(args.bench_log):
        with open(args.bench_log) as fh:
            keep = [ln.strip() for ln in fh if ln.startswith("[bench]")]
        t += ["", "bench.py's own HIP-event timing in the same run:"] + ["  " + ln for ln in keep]
    with open(args.out, "w") as fh:
        fh.write("\n".join(t) + "\n")
    print("\n".join(t))


def summarize_muon(args):
    """Per-call kernel times of the Newton-Schulz iterations bench.py times
    (the LLaMA MLP matrix, then the routed-expert matrix) from a rocprofv3
    --kernel-trace run: each call runs from its k_sumsq to the next one; the
    first call of each shape is the warm-up and is left out."""
    import collections
    import re
    import statistics
    trace = sorted(_csv_rows(os.path.join(args.trace_dir, "run_kernel_trace.csv")),
                   key=lambda r: int(r["Start_Timestamp"]))
    muon_kernels = ("k_sumsq", "k_norm_scale", "k_normalize", "k_gemm", "k_split_sum")
    calls, cur = [], None
    for r in trace:
        name = r["Kernel_Name"]
        if "k_sumsq" in name:
            cur = []
            calls.append(cur)
        elif cur is not None and not any(k in name for k in muon_kernels):
            cur = None
            continue
        if cur is not None:
            cur.append(r)
    shapes = collections.OrderedDict()
    for c in calls:
        norm = next(r for r in c if "k_normalize" in r["Kernel_Name"])
        shapes.setdefault(_grid(norm), []).append(c)
    dims = [(8192, 28672, "LLaMA-3-70B MLP"), (2048, 7168, "DeepSeek-V3 routed expert")]
    t = ["# Kernel trace of the Newton-Schulz iterations in bench.py (rocprofv3 --kernel-trace --stats)", "",
         f"kernel sources hash: {kernel_source_hash(MUON_SOURCES)}", "",
         "command (run from the repository root, on the machine with the GPU):", "  " + args.command, ""]
    short = lambda n: re.sub(r"ve::\(anonymous namespace\)::", "", n)
    for (grid, cs), (rows, cols, what) in zip(shapes.items(), dims):
        timed = cs[1:] if len(cs) > 1 else cs
        tot = [sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in c) / 1e3 for c in timed]
        per = collections.OrderedDict()
        for c in timed:
            for r in c:
                k = (short(r["Kernel_Name"])[:96], _grid(r))
                per.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        fl = ns_flops(rows, cols)
        avg = statistics.mean(tot)
        t += [f"{rows} x {cols} ({what}), 5 steps: {len(timed)} timed calls, kernel time per call {avg:.1f} us "
              f"(min {min(tot):.1f}, max {max(tot):.1f}); {fl / 1e12:.2f} TFLOP (minimal count) -> "
              f"{fl / avg / 1e6:.1f} TFLOP/s = {fl / avg / 1e6 / MFMA_BF16_PEAK_TFLOPS * 100:.1f}% of 2.5 PFLOP/s", "",
              f"  {'kernel':96s} {'grid':>9s} {'per call':>8s} {'avg us':>9s} {'us/call':>9s}"]
        for (name, g), d in sorted(per.items(), key=lambda kv: -sum(kv[1])):
            t.append(f"  {name:96s} {g:9d} {len(d) / len(timed):8.0f} {statistics.mean(d):9.1f} "
                     f"{sum(d) / len(timed):9.1f}")
        t.append("")
    if args.bench_log and os.path.exists(args.bench_log):
        with open(args.bench_log) as fh:
            keep = [ln.strip() for ln in fh if ln.startswith("[bench] muon")]
        t += ["bench.py's own HIP-event timing in the same run:"] + ["  " + ln for ln in keep]
    with open(args.out, "w") as fh:
        fh.write("\n".join(t) + "\n")
    print("\n".join(t))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama", choices=["llama", "gptoss", "deepseek", "adversarial"])
    ap.add_argument("--buckets", type=int, default=None, help="override the number of buckets")
    ap.add_argument("--rank", type=int, default=None,
                    help="the rank whose step is timed (default: the one with the most valid elements)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-group-ops", action="store_true", help="skip timing the DBuffer group operations")
    ap.add_argument("--no-muon", action="store_true", help="skip timing Muon's Newton-Schulz iteration")
    ap.add_argument("--no-planner", action="store_true", help="skip the bucket planner's padding / time report")
    ap.add_argument("--no-copy-in", action="store_true", help="skip timing the whole-bucket copy-in")
    ap.add_argument("--no-rank-sweep", action="store_true", help="skip the step over every rank of one bucket")
    ap.add_argument("--copy-gib", type=float, default=1.0,
                    help="size of the streaming-reference copy that measures the copy ceiling (0: skip)")
    sm = ap.add_argument_group("profile summaries (no GPU needed)")
    sm.add_argument("--summarize", choices=["counters", "trace", "muon"], default=None,
                    help="write a profiles/ summary from rocprofv3 output instead of benchmarking")
    sm.add_argument("--fetch-dir", help="counters: output folder of the FETCH_SIZE run")
    sm.add_argument("--write-dir", help="counters: output folder of the WRITE_SIZE run")
    sm.add_argument("--command-fetch", default="", help="counters: the FETCH_SIZE command, for the record")
    sm.add_argument("--command-write", default="", help="counters: the WRITE_SIZE command, for the record")
    sm.add_argument("--trace-dir", help="trace: output folder of the --kernel-trace --stats run")
    sm.add_argument("--command", default="", help="trace: the profiled command, for the record")
    sm.add_argument("--bench-log", default=None, help="trace: bench.py's stderr of the profiled run")
    sm.add_argument("--skip-first", type=int, default=0,
                    help="trace: leave out the first N step dispatches (the profiled run's --warmup)")
    sm.add_argument("--out", default=None, help="trace: summary file to write")
    sm.add_argument("--top", type=int, default=16, help="trace: kernels listed")
    sm.add_argument("--profiles-dir", default=os.path.join(ROOT, "profiles"),
                    help="counters: folder the summaries and traffic files are written to")
    args = ap.parse_args()
    if args.summarize:
        sys.path.insert(0, ROOT)
        {"counters": summarize_counters, "trace": summarize_trace, "muon": summarize_muon}[args.summarize](args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the data-parallel step; --gpus {args.gpus} is not "
              f"supported (the collectives around the step are outside this library)", file=sys.stderr)
        sys.exit(2)

    import torch
    sys.path.insert(0, ROOT)
    import ragged_shard_optimizer_amd as ve
    from synth import CONFIGS, HPARAMS, plan_p0
    from synth.workload import device_buckets

    cfg = CONFIGS[args.workload]
    lay = plan_p0(cfg.tensors, cfg.fsdp)
    rank = lay.largest_rank() if args.rank is None else args.rank
    if not 0 <= rank < lay.fsdp:
        print(f"bench.py: --rank {rank} outside [0, {lay.fsdp}) for the {args.workload} workload", file=sys.stderr)
        sys.exit(2)
    # the committed HBM counters were taken on the default rank
    own_counters = rank == lay.largest_rank()
    nbk = args.buckets or cfg.n_buckets
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    plan = ve.Plan(lay.spec_array(), lay.fsdp, lay.shard, device=0)
    valid, nblocks, nseg = plan.query(rank)
    log(f"[bench] {cfg.name}: rank {rank}, {nbk} buckets, S={lay.shard}, valid={valid}, blocks={nblocks}")
    t0 = time.time()
    buckets = device_buckets(cfg, lay, rank, dev, n_buckets=nbk)
    states = [ve.new_state(plan, rank, ve.grad_pointer_table(g, dev), m) for g, m in buckets]
    table = ve.state_table(plan, rank, states)
    torch.cuda.synchronize()
    log(f"[bench] inputs resident in HBM ({time.time() - t0:.1f} s)")

    hp = dict(HPARAMS)
    stream = torch.cuda.current_stream()
    step = 0
    for _ in range(args.warmup):
        step += 1
        plan.step(rank, table, hp, step, stream)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done")

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i in range(args.steps):
        step += 1
        starts[i].record(stream)
        plan.step(rank, table, hp, step, stream)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]  # ms, on the launch stream
    ms = sum(per) / len(per)
    ms_wall = wall * 1e3 / args.steps
    log(f"[bench] timed {args.steps} steps: event avg {ms:.4f} ms, min {min(per):.4f}, max {max(per):.4f}; "
        f"wall {ms_wall:.4f} ms/step")

    S = lay.shard
    alg_bytes = nbk * (BYTES_PER_ELEM * valid + BYTES_PER_BLOCK * nblocks + BYTES_PER_PAD * (S - valid))
    gbs = alg_bytes / (ms / 1e3) / 1e9
    params_s = nbk * valid / (ms / 1e3)
    traffic = measured_traffic(args.workload) if own_counters else None
    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.description + f"; rank {rank}", "buckets": nbk, "fsdp": lay.fsdp,
                   "shard_elems": S, "valid_elems_per_bucket": valid, "blocks_per_bucket": nblocks,
                   "alg_bytes_per_step": alg_bytes},
        "params_per_s": round(params_s, 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "ms_per_step_wall": round(ms_wall, 5),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     # measured HBM bytes per launch (rocprofv3 counters on these kernel sources)
                     # over the same launch time, comparable with "achieved"
                     "traffic": None if traffic is None else round(traffic / (ms / 1e3) / 1e9, 2),
                     "traffic_bytes_per_launch": None if traffic is None else round(traffic)},
    }
    if not args.no_group_ops:
        out["group_ops"] = time_group_ops(torch, ve, plan, rank, states, lay, valid, 10, 2,
                                          measured_group_traffic(args.workload) if own_counters else None)
    del states, table, buckets
    torch.cuda.empty_cache()
    if not (args.no_copy_in and args.no_rank_sweep):
        grads_all = whole_bucket_grads(torch, cfg, lay, dev)
        if not args.no_copy_in:
            out["copy_in_whole"] = time_copy_in_whole(torch, ve, plan, lay, grads_all, dev)
        if not args.no_rank_sweep:
            out["rank_sweep"] = rank_sweep(torch, ve, plan, lay, grads_all, dev)
        del grads_all
        torch.cuda.empty_cache()
    if not args.no_muon:
        out["muon"] = time_muon(torch, ve, dev)
        # a matrix far below one round of 256 x 256 tiles: a routed expert
        out["muon_expert"] = time_muon(torch, ve, dev, rows=2048, cols=7168, steps=20, warmup=3,
                                       name="DeepSeek-V3 routed expert")
    if not args.no_planner:
        out["planner"] = time_planner(ve)
    if args.copy_gib > 0:
        out["copy_ceiling"] = copy_ceiling(torch, ve, dev, args.copy_gib)
        out["copy_ceiling_frac"] = round(gbs / out["copy_ceiling"]["gbs"], 4)
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on host cores")
        out["cpu_baseline"] = cpu_baseline(cfg, lay, rank)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
