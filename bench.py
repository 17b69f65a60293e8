"""Decode-latency benchmark of split-KV absorbed-MLA decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME|all]

A step is one pass of the whole hot path over one decode batch: the host
partition chooser, the partition kernel and (when the plan splits) the
LSE-weighted reduce. Inputs are synthetic and resident in HBM before timing
starts. To keep the 256 MB Infinity Cache from serving repeated reads, each
step reads a different copy of the KV pool (enough copies that the steps'
working set is several times the cache). The K timed steps are captured into
one HIP graph; after at least W untimed steps (whole replays of that graph)
it is replayed once between two HIP events, so host launch cost does not pad
the figure. More timed replays (--trials in all) give the spread across
trials.

By default every workload of the pages' configurations is timed in one run
(the tiny case, V2-Lite 32K with the chooser's split and single pass, the
two two-request batches, V3 81K and 131K, the mixed batch of eight), each
with its own roofline and CPU baseline under "workloads"; the headline
fields are V3 131K's, the largest single-GPU configuration in the metric's
32K-131K span. --workload NAME times one workload only.

Prints one JSON line on stdout (details on stderr). ``value`` is the decode
latency in microseconds per step (lower is better). ``roofline`` is for the
partition kernel: algorithmic bytes of one launch over its mean duration,
taken with HIP events around back-to-back launches on the launch stream,
against the 8 TB/s peak and against a plain contiguous read of the same
byte count on the same device (``frac_of_stream``).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
KV_BYTES_PER_TOKEN = (512 + 64) * 2
HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "absorbed_mla_paged_amd", "csrc")
# Sources of each partition kernel; their hash keys the counter table below.
KERNEL_SOURCES = {
    16: ["partition.hip", "partition_common.h", "device_common.h", "fused_common.h"],
    64: ["partition_wide.hip", "partition_common.h", "device_common.h"],
}
# HBM traffic per partition launch from rocprofv3 --pmc (FETCH_SIZE and
# WRITE_SIZE in KiB per dispatch, separate runs), keyed by workload and the
# kernel source hash (code only) at the time of measurement; the summaries are in
# profiles/. FETCH_SIZE on this part reads half of what a plain copy of known
# size moves, WRITE_SIZE reads exactly it: the scale factors below.
FETCH_SCALE = 2.0
WRITE_SCALE = 1.0
MEASURED = {
    # profiles/partition_kernel_v2lite_32k.md
    ("v2lite_32k", "cf90aa654a53"): dict(fetch_kib=18630.2, write_kib=8208.0, mfma_busy=0.022),
    ("v2lite_32k@bs16", "cf90aa654a53"): dict(fetch_kib=18635.3, write_kib=8208.0,
                                              mfma_busy=0.022),
    ("two_req_32k_32k", "cf90aa654a53"): dict(fetch_kib=37134.5, write_kib=8208.0,
                                              mfma_busy=0.034),
    # profiles/partition_kernel_v2lite_32k_fp8.md
    ("v2lite_32k@fp8_e4m3", "cf90aa654a53"): dict(fetch_kib=9426.6, write_kib=8208.0,
                                                  mfma_busy=0.024),
    # profiles/wide_kernel_v3_131k.md
    ("v3_131k", "42ccfc983e44"): dict(fetch_kib=74501.3, write_kib=32832.0, mfma_busy=0.286),
    # profiles/wide_kernel_v3_81k.md
    ("v3_81k", "42ccfc983e44"): dict(fetch_kib=46884.2, write_kib=32062.5, mfma_busy=0.230),
    # profiles/wide_kernel_mixed_b8.md
    ("mixed_b8", "42ccfc983e44"): dict(fetch_kib=326796.0, write_kib=32062.5, mfma_busy=0.348),
    # profiles/wide_kernel_v3_131k_fp8.md
    ("v3_131k@fp8_e4m3", "42ccfc983e44"): dict(fetch_kib=37628.3, write_kib=32832.0,
                                               mfma_busy=0.276),
}


def workload_key(name: str, block_size: int, kv_dtype=None) -> str:
    """Key of the recorded counters: the workload, the block size when it is
    not 32, and the cache storage when it is not 16-bit."""
    key = name if block_size == 32 else f"{name}@bs{block_size}"
    return key if kv_dtype is None else f"{key}@{kv_dtype}"


def kernel_hash(hpw: int) -> str:
    """Hash of the kernel's sources with comments and whitespace removed, so
    that recorded counters stay valid across documentation-only edits."""
    import hashlib
    import re
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[hpw]:
        with open(os.path.join(CSRC, name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:12]


def host_chooser_us(case, prm, calls: int = 2000) -> float:
    """Host time of one mla_choose_partitions call (the plan of every step),
    through ctypes with the arguments built once: an upper bound on the C
    call itself."""
    import ctypes
    import absorbed_mla_paged_amd as mla
    lib = mla.load_library()
    B = case.batch
    ctx = (ctypes.c_int32 * B)(*[int(n) for n in case.context_lens])
    P = (ctypes.c_int32 * B)()
    S = (ctypes.c_int32 * B)()
    ind = (ctypes.c_int32 * (B + 1))()
    info = mla._PlanInfo()
    c_prm = prm._c() if prm is not None else None
    pp = ctypes.byref(c_prm) if c_prm is not None else None
    args = (B, case.heads, case.q_len, ctx, case.block_size, pp, P, S, ind, ctypes.byref(info))
    fn = lib.mla_choose_partitions
    if fn(*args) != 0:
        raise RuntimeError(mla.mla_last_error())
    t0 = time.perf_counter()
    for _ in range(calls):
        fn(*args)
    return (time.perf_counter() - t0) / calls * 1e6


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(case):
    """KV rows read + q read + out written + table and context lengths."""
    tokens = int(case.context_lens.astype(np.int64).sum())
    bs = case.block_size
    nblk = int(sum((int(n) + bs - 1) // bs for n in case.context_lens))
    per_token = KV_BYTES_PER_TOKEN // 2 if case.kv_dtype == "fp8_e4m3" else KV_BYTES_PER_TOKEN
    kv = tokens * per_token
    rows = case.batch * case.q_len * case.heads   # query rows: new tokens x heads
    q = rows * (512 + 64) * 2
    out = rows * 512 * 2
    meta = nblk * 4 + case.batch * 4
    # Score and value products: 2 * rows * (576 + 512) flops per visible
    # token (new token j of a window sees n - q_len + 1 + j of them).
    visible = sum(max(0, int(n) - case.q_len + 1 + j) for n in case.context_lens
                  for j in range(case.q_len))
    flops = 2 * case.heads * (576 + 512) * visible
    return dict(kv=kv, q=q, out=out, meta=meta, total=kv + q + out + meta,
                partition=kv + q + meta, tokens=tokens, flops=flops)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def blas_build() -> str:
    try:
        blas = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        return f"{blas.get('name')} {blas.get('version')}"
    except Exception:   # older numpy: no dict mode
        return "unknown"


def cpu_baseline(case, budget_s: float, decompressed: bool = False):
    """Time the f64 oracle on the same workload: one warm-up, then at least
    three timed runs and as many more as fit in ~budget_s; the median. With
    decompressed=True also one run of the pre-absorption oracle in its
    square-orthogonal mode (per-head 512 x 512 orthogonal W_UK, W_UV^T) on
    the same inputs, as context."""
    import oracle
    from oracle import reference
    cores = len(os.sched_getaffinity(0))
    oracle.latent_f64(case)   # warm-up
    times = []
    t0 = time.perf_counter()
    while len(times) < 3 or time.perf_counter() - t0 < budget_s:
        t1 = time.perf_counter()
        oracle.latent_f64(case)
        times.append(time.perf_counter() - t1)
    per = float(np.median(times))
    res = dict(value=round(per * 1e6, 1), unit="us", cores=cores, kind="oracle",
               sample=f"whole workload (every request and head), f64 numpy: median of "
                      f"{len(times)} timed runs after one warm-up",
               cpu_model=cpu_model(), blas=blas_build(), numpy=np.__version__)
    if decompressed and int(getattr(case, "q_len", 1)) == 1:
        W_UK, W_UV_T = oracle.orthogonal_weights(99, case.heads)
        qa = reference.decode16(case.q_absorbed, case.dtype)
        q_nope = np.einsum("bhr,hdr->bhd", qa, W_UK)
        t1 = time.perf_counter()
        oracle.decompressed_f64(case, q_nope, W_UK, W_UV_T)
        res["decompressed_us"] = round((time.perf_counter() - t1) * 1e6, 1)
        res["decompressed_sample"] = ("pre-absorption oracle, square-orthogonal mode (512-wide "
                                      "per-head keys and values), one run")
    return res


def projections(case, args, torch, mla):
    """Fold and unfold for the workload's rows (batch x new tokens) and heads,
    each launch reading its 128 x 512 weights per head from HBM. K launches
    of each in a graph (weights rotated over copies so the cache cannot hold
    them), HIP events on the launch stream."""
    td = torch.float16 if case.dtype == "f16" else torch.bfloat16
    dev = torch.device("cuda", 0)
    rows, H = case.batch * case.q_len, case.heads
    g = torch.Generator(device=dev).manual_seed(1234)
    wbytes = H * 128 * 512 * 2
    ncopy = max(1, min(64, math.ceil(args.cold_bytes / (2 * wbytes))))
    w_uk = [(torch.randn((H, 128, 512), device=dev, generator=g) / 11.3).to(td) for _ in range(ncopy)]
    w_uv = [(torch.randn((H, 512, 128), device=dev, generator=g) / 22.6).to(td) for _ in range(ncopy)]
    qn = torch.randn((rows, H, 128), device=dev, generator=g).to(td)
    lat = torch.randn((rows, H, 512), device=dev, generator=g).to(td)
    qa = torch.empty((rows, H, 512), dtype=td, device=dev)
    o = torch.empty((rows, H, 128), dtype=td, device=dev)
    stream = torch.cuda.Stream(device=dev)
    res = {}
    for name, fn, x, ws, y in (("fold", mla.mla_absorb_query, qn, w_uk, qa),
                               ("unfold", mla.mla_unabsorb_output, lat, w_uv, o)):
        with torch.cuda.stream(stream):
            for j in range(args.warmup):
                fn(x, ws[j % ncopy], y, stream)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=stream):
            for j in range(args.steps):
                fn(x, ws[j % ncopy], y, stream)
        gr.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            gr.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        nbytes = wbytes + x.numel() * 2 + y.numel() * 2
        res[name] = dict(us=round(us, 3), bytes=nbytes, gbs=round(nbytes / (us * 1e-6) / 1e9, 1))
        log(f"[bench] {name}: {us:.2f} us, {nbytes / 1e6:.2f} MB -> {res[name]['gbs']:.0f} GB/s")
    total = res["fold"]["us"] + res["unfold"]["us"]
    big = max(res.values(), key=lambda r: r["us"])
    line = {
        "metric": "per-head fold and unfold latency (us), absorbed-MLA decode",
        "value": round(total, 3), "unit": "us", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(total * 1e-3, 6), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": case.dtype, "data": "synthetic",
        "config": {"workload": args.workload, "rows": rows, "heads": H, "weight_copies": ncopy},
        "kernels": res,
        "roofline": {"bound": "hbm", "achieved": big["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(big["gbs"] / HBM_PEAK_GBS, 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


# The pages' configurations, in order; the label keys each under
# "workloads" in the JSON line.
ALL_WORKLOADS = [
    ("tiny", "tiny", dict(force_partitions=2)),   # 2 partitions of 512 tokens, device-tiled
    ("v2lite_32k", "v2lite_32k", None),
    ("v2lite_32k@single_pass", "v2lite_32k", dict(force_partitions=1, force_splits=1)),
    ("two_req_32k_32k", "two_req_32k_32k", None),
    ("two_req_32k_20k", "two_req_32k_20k", None),
    ("v3_81k", "v3_81k", None),
    ("v3_131k", "v3_131k", None),
    ("mixed_b8", "mixed_b8", dict(workspace_limit_bytes=64 << 20)),
]
HEADLINE = "v3_131k"
# The pre-absorption oracle is timed (as context) on the 16-head workloads.
DECOMPRESSED_CPU = ("tiny", "v2lite_32k", "two_req_32k_32k", "two_req_32k_20k")
METRIC = "decode latency (µs) + achieved HBM GB/s vs peak, absorbed-MLA 32K–131K ctx"


class StreamRef:
    """mla_stream_read over a 2 GiB buffer: a plain contiguous read of a
    given byte count, rotated over the buffer so the Infinity Cache cannot
    serve it; 100 launches in a graph, the median of five replays."""

    def __init__(self, torch, mla, stream):
        self.torch, self.mla, self.stream = torch, mla, stream
        self.buf = torch.ones(2 << 30, dtype=torch.uint8, device="cuda")
        self.sink = torch.zeros(4, dtype=torch.int32, device="cuda")

    def time_us(self, nbytes: int, reps: int = 100) -> float:
        torch = self.torch
        nbytes = max(16, (int(nbytes) // 16) * 16)
        span = self.buf.numel() - nbytes
        offs = [((j * nbytes) % max(1, span)) // 256 * 256 for j in range(reps)]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=self.stream):
            for o in offs:
                self.mla.mla_stream_read(self.buf[o:o + nbytes], self.sink, self.stream)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts = []
        for _ in range(5):
            with torch.cuda.stream(self.stream):
                e0.record(self.stream)
                g.replay()
                e1.record(self.stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / reps)
        return float(np.median(ts))


def measure(label, name, prm_kw, args, torch, mla, stream, sref, cpu_budget):
    """Time one workload: the step graph, the partition kernel alone, the
    reduce alone, the stream reference over the partition's bytes, and the
    CPU oracle. Returns the result record (raises on a replay mismatch)."""
    import mla_synth
    log(f"[bench] === {label}: generating inputs")
    fp8 = dict(kv_dtype="fp8_e4m3", kv_scale=2.0 ** -5) if args.kv_fp8 else {}
    case = mla_synth.make_workload(name, block_size=args.block_size, **fp8)
    alg = algorithmic_bytes(case)
    td = torch.float16 if case.dtype == "f16" else torch.bfloat16
    dev = torch.device("cuda", 0)

    def t16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(td).to(dev)

    if args.kv_fp8:
        ckv = torch.from_numpy(case.ckv_pool).to(dev)
        kpe = torch.from_numpy(case.kpe_pool).to(dev)
    else:
        ckv = t16(case.ckv_pool)
        kpe = t16(case.kpe_pool)
    pool_bytes = ckv.numel() * ckv.element_size() + kpe.numel() * kpe.element_size()
    ncopy = max(1, min(64, math.ceil(args.cold_bytes / max(1, alg["kv"]))))
    copies = [(ckv, kpe)] + [(ckv.clone(), kpe.clone()) for _ in range(ncopy - 1)]
    qa, qp = t16(case.q_absorbed), t16(case.q_pe)
    table = torch.from_numpy(case.block_table).to(dev)
    ctx = torch.from_numpy(case.context_lens).to(dev)
    prm = mla.PlanParams(**prm_kw) if prm_kw else None
    plan = mla.DecodePlan(case.context_lens, case.heads, prm, device=dev, q_len=case.q_len,
                          block_size=case.block_size)
    qrows = case.q_len * case.heads
    info = plan.info
    out = torch.empty((case.batch, qrows, 512), dtype=td, device=dev)
    lse2 = torch.empty((case.batch, qrows), dtype=torch.float32, device=dev)
    log(f"[bench] {label}: plan P={info['P']} S={info['S']} rows={info['total_rows']} "
        f"tile={info['tile_blocks']} reduce={info['needs_reduce']} copies={ncopy} "
        f"pool={pool_bytes / 1e6:.1f} MB")

    def step(j):
        # Host chooser (same contexts every step, so the device plan arrays
        # already hold its answer), then the device work.
        mla.mla_choose_partitions(case.batch, case.heads, case.q_len, case.context_lens, prm,
                                  block_size=case.block_size)
        c, k = copies[j % ncopy]
        mla.decode(plan, qa, qp, c, k, table, ctx, case.scale, out, lse2, fused=args.fused,
                   kv_scale=case.kv_scale)

    torch.cuda.synchronize()
    # Eager reference result, then graph capture of the timed steps.
    with torch.cuda.stream(stream):
        step(0)
    torch.cuda.synchronize()
    eager = out.clone()

    graph = torch.cuda.CUDAGraph()
    # The library counts launches on the host as they are made, so counters
    # reset before the capture show which paths the K timed steps hold.
    mla.mla_reset_counters()
    with torch.cuda.graph(graph, stream=stream):
        for j in range(args.steps):
            step(j)
    torch.cuda.synchronize()
    c = mla.mla_get_counters()
    path_counters = {"single_pass_launches": c[0], "split_launches": c[1],
                     "reduce_launches": c[2], "rows_launched": c[3]}
    # Warm-up: untimed replays of the same K steps, at least W steps in all.
    # Under sustained load the step time keeps falling for tens of ms (at
    # V3 131K from 66 to 54 us per step over the first three replays of 200
    # steps), so the timed run starts in that steady state.
    warm_replays = max(1, math.ceil(args.warmup / max(1, args.steps)))
    with torch.cuda.stream(stream):
        for _ in range(warm_replays):
            graph.replay()
    torch.cuda.synchronize()
    # The output is checked against the eager result only after the timed
    # replays: a check between the warm-up and the timed run (a reduction
    # and a read back to the host) slowed the replays right after it (V3
    # 131K: 67 against 57 us per step).
    warmup_steps = warm_replays * args.steps

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        e0.record(stream)
        graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    device_ms = gpu_ms / args.steps
    # More replays of the same K steps (--trials in all), each timed on its
    # own, so the spread across trials is reported next to the timed run.
    trials_us = [round(device_ms * 1e3, 3)]
    for _ in range(args.trials - 1):
        with torch.cuda.stream(stream):
            e0.record(stream)
            graph.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        trials_us.append(round(e0.elapsed_time(e1) * 1e3 / args.steps, 3))
    if not torch.equal(out, eager):
        raise RuntimeError(f"{label}: timed replay differs from the eager result")
    chooser_us = host_chooser_us(case, prm)
    # The step is the whole path: the host chooser, then the device work.
    ms_per_step = device_ms + chooser_us * 1e-3
    log(f"[bench] {label}: {args.steps} steps: {gpu_ms:.3f} ms GPU ({wall * 1e3:.3f} ms wall) "
        f"-> {device_ms * 1e3:.2f} us/step on the device + {chooser_us:.2f} us host chooser")

    # Partition kernel alone: back-to-back launches (rotating copies) in a
    # graph, HIP events on the launch stream around them; the median of five
    # replays. Then the reduce alone the same way.
    reps = args.kernel_reps

    def kernel_graph(body):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for j in range(reps):
                body(j)
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            with torch.cuda.stream(stream):
                e0.record(stream)
                g.replay()
                e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / reps)
        return ts

    def partition_only(j):
        c, k = copies[j % ncopy]
        if args.kv_fp8:
            mla.mla_decode_partition_fp8(qa, qp, c, k, case.kv_scale, table, ctx, case.scale,
                                         plan.partitions, plan.splits, plan.row_indptr,
                                         plan.total_rows, info["max_rows_per_req"],
                                         info["heads_per_wg"], plan.partial_out,
                                         plan.partial_lse2, out, lse2, q_len=plan.q_len)
            return
        mla.mla_decode_partition(qa, qp, c, k, table, ctx, case.scale, plan.partitions,
                                 plan.splits, plan.row_indptr, plan.total_rows,
                                 info["max_rows_per_req"], info["heads_per_wg"],
                                 plan.partial_out, plan.partial_lse2,
                                 None if info["needs_reduce"] else out,
                                 None if info["needs_reduce"] else lse2, q_len=plan.q_len)

    kernel_trials = kernel_graph(partition_only)
    part_us = float(np.median(kernel_trials))
    reduce_us = None
    if info["needs_reduce"]:
        reduce_us = float(np.median(kernel_graph(
            lambda j: mla.mla_decode_reduce(plan.partial_out, plan.partial_lse2, plan.row_indptr,
                                            plan.batch, qrows, plan.total_rows, out, lse2))))
    achieved = alg["partition"] / (part_us * 1e-6) / 1e9
    stream_us = sref.time_us(alg["partition"]) if sref is not None else None
    stream_gbs = alg["partition"] / (stream_us * 1e-6) / 1e9 if stream_us else None
    split_bytes = info["total_rows"] * qrows * 513 * 4 if info["needs_reduce"] else 0
    part_written = split_bytes if info["needs_reduce"] else alg["out"]
    pair_gbs = alg["total"] / (ms_per_step * 1e-3) / 1e9
    khash = kernel_hash(info["heads_per_wg"])
    wkey = workload_key(name, case.block_size, case.kv_dtype)
    if prm_kw and prm_kw.get("force_partitions") == 1 and prm_kw.get("force_splits") == 1:
        wkey += "@single_pass"
    meas = MEASURED.get((wkey, khash))
    traffic = None
    if meas is not None:
        traffic = int(round((meas["fetch_kib"] * FETCH_SCALE + meas["write_kib"] * WRITE_SCALE) * 1024))
    log(f"[bench] {label}: partition kernel source hash {khash}; counters "
        f"{'on record' if meas else 'not on record for this source'}")
    log(f"[bench] {label}: partition kernel {part_us:.2f} us -> {achieved:.0f} GB/s "
        f"({100 * achieved / HBM_PEAK_GBS:.1f}% of 8 TB/s"
        + (f", {100 * achieved / stream_gbs:.1f}% of a {stream_us:.2f} us stream read"
           if stream_gbs else "") + f"); reduce {reduce_us if reduce_us else 0:.2f} us; "
        f"pair {pair_gbs:.0f} GB/s; split overhead {split_bytes / 1e6:.2f} MB written")

    cpu = None
    if cpu_budget is not None:
        cpu = cpu_baseline(case, cpu_budget, decompressed=name in DECOMPRESSED_CPU)
        log(f"[bench] {label}: cpu oracle {cpu}")

    rec = {
        "value": round(ms_per_step * 1e3, 3),
        "unit": "us",
        "ms_per_step": round(ms_per_step, 6),
        "warmup": warmup_steps,
        "dtype": {"f16": "f16", "bf16": "bf16"}[case.dtype],
        "config": {"workload": name, "batch": case.batch, "heads": case.heads,
                   "q_len": case.q_len,
                   "context_lens": [int(n) for n in case.context_lens],
                   "block_size": case.block_size, "kv_lora_rank": 512, "rope_dim": 64,
                   "kv_dtype": case.kv_dtype or case.dtype,
                   "plan": {"P": info["P"], "S": info["S"], "rows": info["total_rows"],
                            "heads_per_wg": info["heads_per_wg"], "groups": info["groups"],
                            "tile_blocks": info["tile_blocks"],
                            "needs_reduce": bool(info["needs_reduce"]),
                            "params": prm_kw or {}},
                   "single_pass": not bool(info["needs_reduce"]), "kv_copies": ncopy},
        "path_counters": path_counters,
        "device_us": round(device_ms * 1e3, 3),
        "device_us_trials": {"median": float(np.median(trials_us)), "min": min(trials_us),
                             "max": max(trials_us), "trials": trials_us},
        "host_chooser_us": round(chooser_us, 3),
        "partition_us": round(part_us, 3),
        "reduce_us": round(reduce_us, 3) if reduce_us else None,
        "achieved_gbs_pair": round(pair_gbs, 1),
        # the whole step (algorithmic bytes of the call over the step time)
        # against the 8 TB/s peak and against the plain read of the
        # partition's bytes
        "pair_frac": round(pair_gbs / HBM_PEAK_GBS, 4),
        "pair_frac_of_stream": round(pair_gbs / stream_gbs, 4) if stream_gbs else None,
        "split_bytes_written": split_bytes,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "stream_read_us": round(stream_us, 3) if stream_us else None,
                     "stream_read_gbs": round(stream_gbs, 1) if stream_gbs else None,
                     "frac_of_stream": round(achieved / stream_gbs, 4) if stream_gbs else None,
                     "kernel": "partition_kernel" if info["heads_per_wg"] == 16 else "wide_kernel",
                     "kernel_source_hash": khash,
                     "kernel_us": round(part_us, 3),
                     "kernel_us_trials": [round(t, 3) for t in kernel_trials],
                     "algorithmic_bytes": alg["partition"],
                     # traffic against what the launch must move (KV, q and
                     # table read, fp32 partials written); above 1.10 means
                     # re-reads worth chasing
                     "traffic_vs_algorithmic": (round(traffic / (alg["partition"] + part_written), 3)
                                                if traffic else None),
                     # counted HBM traffic over the launch time, and whether
                     # it exceeds the bytes the launch must move by over 10%
                     "traffic_gbs": round(traffic / (part_us * 1e-6) / 1e9, 1) if traffic else None,
                     "traffic_frac": (round(traffic / (part_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                                      if traffic else None),
                     "traffic_frac_of_stream": (round(traffic / (part_us * 1e-6) / 1e9 / stream_gbs, 4)
                                                if traffic and stream_gbs else None),
                     "traffic_excess_flag": (traffic > 1.10 * (alg["partition"] + part_written)
                                             if traffic else None),
                     # FETCH_SIZE and WRITE_SIZE as read (KiB per dispatch),
                     # and the scale factors applied to them (the copy
                     # calibration: FETCH_SIZE reads half of a known copy)
                     "counters_kib": ({"fetch": meas["fetch_kib"], "write": meas["write_kib"],
                                       "fetch_scale": FETCH_SCALE, "write_scale": WRITE_SCALE}
                                      if meas else None),
                     # time floors of one launch: its bytes at 8 TB/s and its
                     # flops on 16-bit MFMA at 2.5 PFLOP/s (dense)
                     "hbm_floor_us": round(alg["partition"] / (HBM_PEAK_GBS * 1e3), 3),
                     "mfma_floor_us": round(alg["flops"] / 2.5e9, 3),
                     "mfma_busy": meas.get("mfma_busy") if meas else None},
        "cpu_baseline": cpu,
    }
    del copies, ckv, kpe, graph, plan
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def copy_probe(args, torch, mla):
    """Copies only (mla_copy_probe): the V3 131K byte count (4096 blocks of
    36 KB) read as 256 rows x 16 blocks by one workgroup each, and as 128
    rows x 32 blocks by two workgroups each (the 64-head layout of 128
    heads), for several copying-wave counts and copies in flight; and a
    plain stream read of the same bytes. Blocks are drawn at random from a
    pool 4x the size, a different draw per launch (the Infinity Cache
    cannot serve them); 20 launches each, the median."""
    dev = torch.device("cuda", 0)
    nblk, pool = 4096, 4 * 4096 * 4
    ckv = torch.ones((pool, 32, 512), dtype=torch.bfloat16, device=dev)
    kpe = torch.ones((pool, 32, 64), dtype=torch.bfloat16, device=dev)
    gen = torch.Generator().manual_seed(5)
    tables = [torch.randperm(pool, generator=gen)[:nblk].to(torch.int32).to(dev)
              for _ in range(8)]
    stream = torch.cuda.Stream(device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nbytes = nblk * 36 * 1024
    res = []
    for groups, rows in ((1, 256), (2, 128)):
        for waves, inflight in ((4, 8), (4, 16), (8, 8), (8, 16)):
            ts = []
            for rep in range(24):
                with torch.cuda.stream(stream):
                    e0.record(stream)
                    mla.mla_copy_probe(ckv, kpe, tables[rep % len(tables)], rows, nblk // rows,
                                       groups, waves, inflight, stream)
                    e1.record(stream)
                torch.cuda.synchronize()
                if rep >= 4:
                    ts.append(e0.elapsed_time(e1) * 1e3)
            us = float(np.median(ts))
            r = dict(groups=groups, rows=rows, blocks_per_row=nblk // rows, waves=waves,
                     inflight_kb_per_cu=waves * inflight, us=round(us, 2),
                     hbm_tbs=round(nbytes / us / 1e6, 3),
                     lds_fill_tbs=round(groups * nbytes / us / 1e6, 3))
            log(f"[bench] copy probe {r}")
            res.append(r)
    sref = StreamRef(torch, mla, stream)
    stream_us = sref.time_us(nbytes)
    log(f"[bench] stream read of {nbytes / 1e6:.1f} MB: {stream_us:.2f} us")
    print(json.dumps({"metric": "copy-only probe (us) at the V3 131K byte count", "unit": "us",
                      "bytes": nbytes, "probe": res, "stream_read_us": round(stream_us, 2)}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=1000,
                    help="untimed steps before the timed ones (run as whole replays of the "
                         "K-step graph)")
    ap.add_argument("--workload", default="all",
                    help="'all' (every configuration; headline V3 131K) or one workload name")
    ap.add_argument("--single-pass", action="store_true", help="force P = S = 1")
    ap.add_argument("--block-size", type=int, default=32, choices=(16, 32),
                    help="tokens per cache block of the paged layout")
    ap.add_argument("--kv-fp8", action="store_true",
                    help="latent cache stored as E4M3 bytes times a scale of 2^-5 "
                         "(mla_decode_partition_fp8)")
    ap.add_argument("--fused", action="store_true",
                    help="partition and merge in one launch (mla_decode_fused)")
    ap.add_argument("--projections", action="store_true",
                    help="instead: time the per-head fold (q_nope W_UK) and unfold "
                         "(out W_UV^T) for the workload's batch and heads")
    ap.add_argument("--cold-bytes", type=float, default=1.5e9,
                    help="bytes of distinct KV copies cycled through (MALL is 256 MB)")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of CPU oracle timing for the headline workload")
    ap.add_argument("--cpu-budget-other", type=float, default=2.0,
                    help="seconds of CPU oracle timing for each other workload")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-stream", action="store_true",
                    help="skip the plain stream-read reference")
    ap.add_argument("--kernel-reps", type=int, default=100)
    ap.add_argument("--trials", type=int, default=5,
                    help="timed replays of the step graph (the first one is `value`)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="instead: time copy-only launches (mla_copy_probe) at the V3 131K "
                         "byte count, one and two workgroups per row")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 device-to-device copies of MIB MiB (for scaling "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "this library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    rank = int(os.environ.get("RANK", "0"))

    import torch
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 5 copies of {n} bytes ({args.copy_calibration} MiB)")
        return
    import absorbed_mla_paged_amd as mla
    import mla_synth

    if args.copy_probe:
        copy_probe(args, torch, mla)
        return
    if args.projections:
        name = HEADLINE if args.workload == "all" else args.workload
        log(f"[bench] projections for {name}")
        projections(mla_synth.make_workload(name, block_size=args.block_size), args, torch, mla)
        return
    log(f"[bench] workload={args.workload} steps={args.steps} warmup={args.warmup}")
    if args.workload == "all":
        todo = [w for w in ALL_WORKLOADS]
        headline = HEADLINE
    else:
        known = {label: p for label, _, p in ALL_WORKLOADS}
        prm = (dict(force_partitions=1, force_splits=1) if args.single_pass
               else known.get(args.workload))
        label = args.workload + ("@single_pass" if args.single_pass else "")
        todo = [(label, args.workload, prm)]
        headline = label
    dev = torch.device("cuda", 0)
    stream = torch.cuda.Stream(device=dev)
    sref = None if args.no_stream else StreamRef(torch, mla, stream)
    results = {}
    for label, name, prm in todo:
        budget = None
        if rank == 0 and not args.no_cpu:
            budget = args.cpu_budget if label == headline else args.cpu_budget_other
        results[label] = measure(label, name, prm, args, torch, mla, stream, sref, budget)

    head = results[headline]
    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": head["warmup"],
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": head["config"],
        "path_counters": head["path_counters"],
        "device_us": head["device_us"],
        "device_us_trials": head["device_us_trials"],
        "host_chooser_us": head["host_chooser_us"],
        "partition_us": head["partition_us"],
        "reduce_us": head["reduce_us"],
        "achieved_gbs_pair": head["achieved_gbs_pair"],
        "pair_frac": head["pair_frac"],
        "pair_frac_of_stream": head["pair_frac_of_stream"],
        "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
        "host": platform.node(),
    }
    if len(results) > 1:
        line["workloads"] = results
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
