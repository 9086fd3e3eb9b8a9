"""Benchmark: one FSDP FULL_SHARD rank's fused optimizer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over the rank's shard: the fp32 mean
of the N incoming gradient slices, AdamW on the shard, and the bf16 cast into
the all-gather slot -- one fsdp_mt_step launch over every local shard.  The
shard layout is planned once, before timing, as FSDP does at wrap time.
Inputs are synthetic and already resident in HBM when timing starts.

Default workload: the 7B model's rank shard at N=8 (291 Shard(0) shards,
842,301,952 local params, 8 bf16 gradient slices, fp32 master/m/v, bf16 out).

Prints ONE JSON line: params/s as ``value``, HBM GB/s, the roofline fraction
of the fused kernel against the 8 TB/s HBM3E peak (kernel time from HIP events
on the launch stream), the other paths on the same state (clipped step, fp8
copy, gradient accumulation, slice tables, the unfused chain), the other
workloads timed the same way (``configs``: the 128 MiB unit, the Llama-7B
block and the 70B shard), and the CPU oracle timed on one full step of the
same workload on this host's cores.
"""

import argparse
import hashlib
import json
import os
import sys
import time

METRIC = "sharded AdamW step params/s + HBM GB/s (% peak), 7B rank shard at N=8"
HBM_PEAK_GBS = 8000.0
# MI355X's Infinity Cache (memory-side, in front of HBM).  A step whose bytes
# are within a few times this size would be served partly from it if the same
# buffers were stepped back to back.  Such workloads rotate through several
# copies of the rank's state, so that at least ROTATE_BYTES of other traffic
# passes between two steps on the same copy.  Steps stay back to back: each
# one pays the write-back of its predecessor's dirty lines, as in a training
# loop, which a step timed alone after a cache flush would not.
INFINITY_CACHE_BYTES = 256 << 20
ROTATE_BYTES = 16 * INFINITY_CACHE_BYTES
MAX_COPIES = 64
# The warm-up runs at least this long (seconds of steps)
SETTLE_S = 0.3
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["rank_step_amd/csrc/rank_step.hip"]
WORKLOAD_BY_NAME = {"llama7b_full_n8": 4, "llama7b_block_n8": 3, "mlp128m_flat_n4": 2,
                    "tiny_mlp_flat_n4": 1, "llama70b_full_n32": 5, "mlp128m_zero1_n4": 6}


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def bytes_per_param(w, bf16_out):
    """Algorithmic HBM bytes per parameter of the fused pass: N slices read,
    fp32 master/m/v read and written, the bf16 copy written.  The reduced
    gradient never leaves registers."""
    slice_b = 2 if w.slice_dtype == "bf16" else 4
    return w.n_slices * slice_b + 12 + 12 + (2 if bf16_out else 0)


def measured_traffic(workload, launches_numel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_source_hash() or d.get("total_numel") != launches_numel:
        return None
    return d.get("bytes_per_launch")


def host_cores():
    """Cores this process may use: the affinity mask, bounded by the cgroup's
    CPU quota where one is set (a host may show more cores than its quota)."""
    n = len(os.sched_getaffinity(0))
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()
        if quota != "max":
            n = min(n, max(1, int(quota) // int(period)))
    except (OSError, ValueError):
        pass
    return max(1, n)


def _cpu_inputs(rng, n, w):
    """One shard's oracle inputs on the host, drawn with the workload's
    distributions: fp32 state (master ~ N(0, 0.02), moments of a running
    optimizer) widened to float64, and N slices as raw bf16 bits (the top
    half of each fp32 draw) or fp32."""
    import numpy as np
    p = (rng.standard_normal(n, dtype=np.float32) * np.float32(0.02)).astype(np.float64)
    m = (rng.standard_normal(n, dtype=np.float32) * np.float32(1e-4)).astype(np.float64)
    v = (rng.standard_normal(n, dtype=np.float32) ** 2 * np.float32(1e-8)).astype(np.float64)
    x = rng.standard_normal((w["n_slices"], n), dtype=np.float32) * np.float32(w["sigma"])
    if w["outlier_frac"] > 0:
        x = np.where(rng.random((w["n_slices"], n), dtype=np.float32) < w["outlier_frac"],
                     x * np.float32(w["outlier_scale"]), x)
    raw = (x.view(np.uint32) >> 16).astype(np.uint16) if w["bf16"] else x
    return p, m, v, raw


def _cpu_oracle_step(inputs, w, t):
    """The oracle as the parity tests call it: the slices widened exactly,
    then oracle.step.rank_step over the shard."""
    from oracle import step as O
    p, m, v, raw = inputs
    sl = O.widen_bf16_bits(raw) if w["bf16"] else O.widen_f32(raw)
    O.rank_step(p, m, v, sl, p.size, t, w["hparams"])
    return p.size


def _cpu_worker(shards, w, t, seed, ready, go, out):
    """One process of the CPU baseline: draws its shards' inputs (untimed),
    says so, waits for the start, then runs the oracle over its shards and
    reports the parameters done."""
    import numpy as np
    rng = np.random.default_rng(seed)
    inputs = [_cpu_inputs(rng, n, w) for n in shards]
    ready.put(1)
    go.wait()
    done = sum(_cpu_oracle_step(x, w, t) for x in inputs)
    out.put(done)


def _collect(q, n, procs, limit_s):
    """n items from q, failing early if a worker process has died."""
    import queue
    got, deadline = [], time.time() + limit_s
    while len(got) < n:
        try:
            got.append(q.get(timeout=2))
        except queue.Empty:
            dead = [p.exitcode for p in procs if p.exitcode not in (None, 0)]
            if dead or time.time() > deadline:
                raise RuntimeError(f"cpu baseline: worker exit codes {dead}" if dead else
                                   "cpu baseline: timed out")
    return got


def _workload_spec(w):
    return {"n_slices": w.n_slices, "bf16": w.slice_dtype == "bf16", "sigma": w.grad_sigma,
            "outlier_frac": w.outlier_frac, "outlier_scale": w.outlier_scale, "hparams": dict(w.hparams)}


def cpu_baseline(w, segments, total, t):
    """The oracle (float64 NumPy), as it stands, timed on this host:
    one full step of the rank's workload, every shard, chunked by shard
    over one spawned process per core (largest shards first, each to the
    least-loaded process), wall time from the moment every process holds its
    inputs to the last one's finish; and one step of the Llama-7B block on a
    single core, for a per-core figure."""
    import multiprocessing as mp

    from rank_step_amd.workloads import WORKLOADS

    cores = host_cores()
    sizes = sorted((length for length, _ in segments), reverse=True)
    share = [[] for _ in range(cores)]
    load = [0] * cores
    for n in sizes:
        i = load.index(min(load))
        share[i].append(n)
        load[i] += n
    spec = _workload_spec(w)
    ctx = mp.get_context("spawn")          # fresh interpreters: nothing of this process's GPU state
    ready, go, out = ctx.Queue(), ctx.Event(), ctx.Queue()
    procs = [ctx.Process(target=_cpu_worker, args=(share[i], spec, t, 1000 + i, ready, go, out))
             for i in range(cores)]
    for p in procs:
        p.start()
    try:
        _collect(ready, cores, procs, 600)     # every process holds its inputs
        t0 = time.perf_counter()
        go.set()
        done = sum(_collect(out, cores, procs, 900))
        wall = time.perf_counter() - t0
    finally:
        for p in procs:
            p.join(timeout=60)
            if p.is_alive():
                p.kill()
    assert done == total, (done, total)
    # one core: the Llama-7B block's step (every dim 0 divides by its N = 8)
    import numpy as np
    wb = WORKLOADS[3]
    rng = np.random.default_rng(7)
    block_shards = [p.numel // wb.world_size for p in wb.params]
    inputs = [_cpu_inputs(rng, n, _workload_spec(wb)) for n in block_shards]
    t1 = time.perf_counter()
    n1 = sum(_cpu_oracle_step(x, _workload_spec(wb), t) for x in inputs)
    one = time.perf_counter() - t1
    return {"value": total / wall, "unit": "params/s", "cores": cores, "kind": "oracle",
            "sample": f"one full step of the {w.name} rank shard: all {len(sizes)} shards, "
                      f"{total:,} params, {w.n_slices} {w.slice_dtype} gradient slices each, "
                      f"chunked by shard over {cores} spawned processes (one per core of this "
                      f"host's {len(os.sched_getaffinity(0))}-core affinity mask); inputs drawn on "
                      f"the host with the workload's distributions; {wall:.1f} s wall",
            "seconds": wall,
            "single_core": {"workload": wb.name, "params": n1, "seconds": one,
                            "params_per_s": n1 / one}}


def clipped_step(st, stream, args, t0):
    """Time the clipped step on the same state: reduce + sum of squares
    (pass 1), the clip coefficient, AdamW + cast from the scaled gradient
    (pass 2).  Bytes per param: 2N+4 in pass 1, 4+24+2 in pass 2."""
    import torch
    from rank_step_amd import binding as B

    w = st.w
    plan = B.MtPlan(st.mt_tensors(with_grad_out=True), w.n_slices, w.slice_dtype, stream)
    sq = torch.zeros(1, dtype=torch.float64, device=st.device)
    coef = torch.zeros(1, dtype=torch.float32, device=st.device)

    def one(t):
        plan.reduce_sqnorm(sq, stream)
        B.fsdp_clip_coef(coef, None, sq, 1, args.clip, stream)
        plan.step_clipped(w.hparams, t, coef, stream)

    t = t0
    for _ in range(args.warmup):
        t += 1
        one(t)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        t += 1
        one(t)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    plan.close()
    slice_b = 2 if w.slice_dtype == "bf16" else 4
    bpp = w.n_slices * slice_b + 4 + 4 + 24 + (2 if w.bf16_out else 0)
    return {"ms_per_step": ms, "params_per_s": st.total / (ms / 1e3), "bytes_per_param": bpp,
            "hbm_gb_s": bpp * st.total / (ms / 1e3) / 1e9, "max_norm": args.clip,
            "coef": float(coef.item()), "launches": 4}


def fp8_step(st, stream, args, t0):
    """Time the step with an fp8 all-gather copy instead of the bf16 one:
    the fused step with per-tensor amax (2N+24 B/param), then the cast with
    per-tensor scales (4+1 B/param); and the one-pass variant with scales
    fixed before the step (delayed scaling)."""
    import torch
    from rank_step_amd import binding as B

    w = st.w
    plan = B.MtPlan(st.mt_tensors(with_grad_out=False, with_bf16=False, with_fp8=True), w.n_slices,
                    w.slice_dtype, stream)
    n = len(st.segments)
    amax = torch.zeros(n, dtype=torch.float32, device=st.device)
    scale = torch.zeros(n, dtype=torch.float32, device=st.device)

    def one(t):
        plan.step_amax(w.hparams, t, amax, stream)
        plan.cast_fp8(amax, 1, scale, stream)

    t = t0
    for _ in range(args.warmup):
        t += 1
        one(t)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        t += 1
        one(t)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    # delayed scaling: the codes use the scales the previous step derived, in
    # the one pass of the step (2N+24+1 B/param), and the step's amax feeds
    # the next scales
    def delayed(t):
        plan.step_fp8(w.hparams, t, scale, amax, stream)

    for _ in range(args.warmup):
        t += 1
        delayed(t)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        t += 1
        delayed(t)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_d = e0.elapsed_time(e1) / args.steps
    plan.close()
    slice_b = 2 if w.slice_dtype == "bf16" else 4
    bpp = w.n_slices * slice_b + 24 + 4 + 1
    bpp_d = w.n_slices * slice_b + 24 + 1
    return {"ms_per_step": ms, "params_per_s": st.total / (ms / 1e3), "bytes_per_param": bpp,
            "hbm_gb_s": bpp * st.total / (ms / 1e3) / 1e9, "launches": 3,
            "all_gather_bytes_per_param": 1,
            "delayed_scaling": {"ms_per_step": ms_d, "params_per_s": st.total / (ms_d / 1e3),
                                "bytes_per_param": bpp_d,
                                "hbm_gb_s": bpp_d * st.total / (ms_d / 1e3) / 1e9, "launches": 2}}


def accumulation(st, stream, args):
    """Time one micro-batch of gradient accumulation at the rank shard's size:
    synchronised (reduce the N slices and add into the fp32 gradient shard,
    2N+8 B/param) and no_sync (add one bf16 micro-batch into an fp32 gradient
    buffer, 10 B/param; a rank's real unsharded buffer is N times longer)."""
    import torch
    from rank_step_amd import binding as B

    w = st.w
    plan = B.MtPlan(st.mt_tensors(with_grad_out=True), w.n_slices, w.slice_dtype, stream)
    acc = torch.zeros(st.total, dtype=torch.float32, device=st.device)
    micro = st.slices[0]

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_sync = timed(lambda: plan.reduce_accumulate(1, None, stream))
    ms_nos = timed(lambda: B.fsdp_grad_accumulate(acc, micro, w.slice_dtype, st.total, 1, stream))
    plan.close()
    slice_b = 2 if w.slice_dtype == "bf16" else 4
    b_sync = w.n_slices * slice_b + 8
    b_nos = slice_b + 8
    return {"synchronised": {"ms_per_micro_batch": ms_sync, "bytes_per_param": b_sync,
                             "hbm_gb_s": b_sync * st.total / ms_sync / 1e6},
            "no_sync": {"ms_per_micro_batch_per_shard_size": ms_nos, "bytes_per_param": b_nos,
                        "hbm_gb_s": b_nos * st.total / ms_nos / 1e6}}


def slice_table_step(st, stream, args, t0):
    """Time the fused step with every shard reading its N slices through a
    table of slice pointers (the form for N receive buffers that do not share
    an allocation).  The entries point at the rows of the same slice buffer,
    so the bytes and addresses equal the stride form's."""
    import torch
    from rank_step_amd import binding as B

    w = st.w
    es = st.slices.element_size()
    base = st.slices.data_ptr()
    recs = []
    for d, (off, length, held, _) in zip(st.mt_tensors(with_grad_out=False, with_fp8=False),
                                         st.segments):
        d = dict(d)
        d.pop("grad_slices")
        d.pop("slice_stride")
        d["grad_slice_ptrs"] = [base + es * (q * st.slice_stride + off) for q in range(w.n_slices)]
        recs.append(d)
    plan = B.MtPlan(recs, w.n_slices, w.slice_dtype, stream)
    t = t0
    for _ in range(args.warmup):
        t += 1
        plan.step(w.hparams, t, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        t += 1
        plan.step(w.hparams, t, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    plan.close()
    bpp = bytes_per_param(w, w.bf16_out)
    return {"ms_per_step": ms, "params_per_s": st.total / (ms / 1e3),
            "hbm_gb_s": bpp * st.total / ms / 1e6, "bytes_per_param": bpp}


def unfused_chain(st, stream, args, t0):
    """Time the same step as three separate calls per shard (reduce -> AdamW
    -> cast, 3 launches x shards), which moves 2N+4 + 28 + 6 B/param, beside
    the fused one-pass launch."""
    import torch
    from rank_step_amd import binding as B

    w = st.w
    g = torch.empty(st.total, dtype=torch.float32, device=st.device)
    tens = st.mt_tensors(with_grad_out=False, with_fp8=False)
    gp = g.data_ptr()
    steps = max(1, min(args.steps, 10))

    def one(t, s=stream):
        for d, (off, length, held, _) in zip(tens, st.segments):
            B.fsdp_reduce_grad_shard(gp + 4 * off, d["grad_slices"], w.slice_dtype, d["slice_stride"],
                                     w.n_slices, length, held, s)
            B.fsdp_adamw_shard_step(d["param_fp32"], d["exp_avg"], d["exp_avg_sq"], gp + 4 * off,
                                    length, held, w.hparams, t, s)
            if d["unshard_bf16_out"] is not None:
                B.fsdp_cast_unshard_bf16(d["unshard_bf16_out"], d["param_fp32"], length, held, s)

    t = t0
    one(t + 1)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for k in range(steps):
        one(t + 2 + k)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps

    # the same chain captured once in a HIP graph and replayed: no host launch
    # cost per kernel, so what remains beside the fused pass is the extra
    # bytes and the gaps between dependent kernels
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one(t + 2 + steps, s=None)          # the capture stream is torch's current one
    graph.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_graph = e0.elapsed_time(e1) / steps
    del graph

    # the same three calls once each over the rank's whole buffer (its shards
    # are packed back to back, so one call covers them all): 3 launches, the
    # unfused bytes without the per-shard launches
    d0 = tens[0]
    n_all = st.total

    def whole(t):
        B.fsdp_reduce_grad_shard(gp, d0["grad_slices"], w.slice_dtype, st.slice_stride, w.n_slices,
                                 n_all, n_all, stream)
        B.fsdp_adamw_shard_step(d0["param_fp32"], d0["exp_avg"], d0["exp_avg_sq"], gp, n_all, n_all,
                                w.hparams, t, stream)
        if d0["unshard_bf16_out"] is not None:
            B.fsdp_cast_unshard_bf16(d0["unshard_bf16_out"], d0["param_fp32"], n_all, n_all, stream)

    whole(t + 3 + steps)
    torch.cuda.synchronize()
    e0.record(stream)
    for k in range(steps):
        whole(t + 4 + steps + k)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_whole = e0.elapsed_time(e1) / steps
    slice_b = 2 if w.slice_dtype == "bf16" else 4
    bpp = w.n_slices * slice_b + 4 + 28 + (6 if w.bf16_out else 0)
    return {"ms_per_step": ms, "bytes_per_param": bpp, "hbm_gb_s": bpp * st.total / ms / 1e6,
            "launches": 3 * len(tens), "steps": steps,
            "hip_graph": {"ms_per_step": ms_graph, "hbm_gb_s": bpp * st.total / ms_graph / 1e6},
            "whole_buffer_3_launches": {"ms_per_step": ms_whole,
                                        "hbm_gb_s": bpp * st.total / ms_whole / 1e6}}


def launch_info(info):
    """The fused step's launch, from the plan's info: one range (workgroup b
    on tile b of the whole) or through the chunk table (8 per entry)."""
    if info["step_one_range"]:
        return {"workgroups": -(-info["total_numel"] // 256), "form": "one range",
                "chunks": info["n_chunks"], "chunk_numel": info["chunk_numel"]}
    return {"workgroups": info["n_blocks"], "form": "chunk table", "chunks": info["n_chunks"],
            "chunk_numel": info["chunk_numel"]}


def time_fused(w, dev, stream, args, keep=False, **state_kw):
    """Plan the rank's shards of workload ``w`` and time K fused steps
    (``fsdp_mt_step``, one launch each) back to back between two events on
    the launch stream, after W warm-up steps; then K more with an event
    between consecutive steps for the spread.  Workloads whose step moves
    less than ROTATE_BYTES rotate through copies of the rank's state.  With
    ``keep`` the first copy stays open for the other legs."""
    import torch

    from rank_step_amd.state import RankState

    st = RankState(w, 0, dev, bf16_out=w.bf16_out, **state_kw)
    st.load_grads(1)
    # plan creation: once per wrap, on the host (layout of the chunk and
    # descriptor tables, argument and alias checks, one upload)
    torch.cuda.synchronize()
    p0 = time.perf_counter()
    st.make_plan(stream, with_grad_out=False, with_fp8=False)
    plan_s = time.perf_counter() - p0
    total = st.total
    bpp = bytes_per_param(w, w.bf16_out)
    # copies of the state to rotate through (1: the workload is large enough)
    n_copies = min(MAX_COPIES, max(1, -(-ROTATE_BYTES // (bpp * total)) + 1)) \
        if bpp * total < ROTATE_BYTES else 1
    copies = [st]
    for _ in range(n_copies - 1):
        c = RankState(w, 0, dev, bf16_out=w.bf16_out)
        c.load_grads(1)
        c.make_plan(stream, with_grad_out=False, with_fp8=False)
        copies.append(c)
    torch.cuda.synchronize()
    t = 0
    # warm-up: W steps, at least one on every copy, and at least SETTLE_S of
    # steps, so that a GPU that was idle has reached its working clocks (a
    # GPU's first few hundred milliseconds of work can run several % slower)
    n_warm = max(args.warmup, n_copies) if n_copies > 1 else args.warmup
    w0 = time.perf_counter()
    i = 0
    while i < n_warm or time.perf_counter() - w0 < SETTLE_S:
        t += 1
        copies[i % n_copies].step(t, stream)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()         # the elapsed time is the GPU's
    torch.cuda.synchronize()
    warm_steps = i
    # the timed region: K steps between two events on the launch stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        t += 1
        copies[i % n_copies].step(t, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = e0.elapsed_time(e1) / args.steps
    # the per-step spread, from K more steps with an event between
    # consecutive ones (kept out of the timed region: an event between two
    # launches adds a few microseconds, which shows on the short steps of the
    # small workloads)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record(stream)
    for i in range(args.steps):
        t += 1
        copies[i % n_copies].step(t, stream)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    info = st.plan.info()
    for c in copies[0 if not keep else 1:]:
        c.close()
    gbs = bpp * total / (ms / 1e3) / 1e9
    return {
        "state": st if keep else None,
        "t": t,
        "ms_per_step": ms,
        "params_per_s": total / (ms / 1e3),
        "hbm_gb_s": gbs,
        "frac": gbs / HBM_PEAK_GBS,
        "bytes_per_param": bpp,
        "local_params": total,
        "shards": info["n_tensors"],
        "launch": launch_info(info),
        "per_step_ms": {"median": per_step[len(per_step) // 2],
                        "p95": per_step[min(len(per_step) - 1, (95 * len(per_step)) // 100)],
                        "min": per_step[0], "max": per_step[-1],
                        "from": "a second pass of K steps with an event between consecutive steps"},
        "host_wall_s_timed": wall,
        "plan_create_ms": plan_s * 1e3,
        "warmup_steps_run": warm_steps,
        "timing": ("steps back to back" if n_copies == 1 else
                   f"steps back to back, rotating through {n_copies} copies of the rank's "
                   f"state ({n_copies * bpp * total / 1e9:.2f} GB) so that none finds its "
                   f"data in the {INFINITY_CACHE_BYTES >> 20} MB Infinity Cache"),
    }


# the other workloads timed in the same run (their own plans, one after
# another once the headline's buffers are freed)
OTHER_CONFIGS = ("mlp128m_flat_n4", "llama7b_block_n8", "llama70b_full_n32")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama7b_full_n8", choices=sorted(WORKLOAD_BY_NAME))
    ap.add_argument("--configs", default=",".join(OTHER_CONFIGS),
                    help="comma-separated other workloads to time after the headline ('' for none)")
    ap.add_argument("--stream", choices=("default", "own"), default="default",
                    help="launch on torch's default stream or on a stream of its own")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle timing (e.g. under a profiler)")
    ap.add_argument("--clip", type=float, default=1.0, metavar="MAX_NORM",
                    help="also time the clipped step (global grad-norm clipping) with this max_norm")
    ap.add_argument("--no-clip", dest="clip", action="store_const", const=None,
                    help="do not time the clipped step")
    ap.add_argument("--no-chain", action="store_true",
                    help="do not time the unfused three-call chain")
    ap.add_argument("--no-table", action="store_true",
                    help="do not time the step with slices read through tables of pointers")
    ap.add_argument("--no-fp8", action="store_true",
                    help="do not time the step with the fp8 all-gather copy")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the step, run torch copies of MIB MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: measures one GPU; --gpus {args.gpus} is not supported "
              "(each rank's step is independent of the others; one GPU shows one rank's share)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.stream == "own":
        torch.cuda.set_stream(torch.cuda.Stream(dev))
    stream = torch.cuda.current_stream(dev)

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(args.warmup):
            b.copy_(a)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            b.copy_(a)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        print(json.dumps({"calibrate_copy_bytes_read": 4 * n, "calibrate_copy_bytes_written": 4 * n,
                          "ms_per_copy": ms, "gb_s": 8 * n / ms / 1e6}), flush=True)
        return

    from rank_step_amd.workloads import WORKLOADS

    w = WORKLOADS[WORKLOAD_BY_NAME[args.workload]]
    r = time_fused(w, dev, stream, args, keep=True, grad_out=args.clip is not None,
                   fp8_out=not args.no_fp8)
    st = r.pop("state")
    t = r["t"]
    traffic = measured_traffic(w.name, st.total)
    out = {
        "metric": METRIC,
        "value": r["params_per_s"],
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "layout": w.mode,
            "world_size": w.world_size,
            "rank": 0,
            "local_params": st.total,
            "shards": r["shards"],
            "grad_slices": f"{w.n_slices} x {w.slice_dtype}",
            "state": "fp32 master + exp_avg + exp_avg_sq" if w.has_master else "fp32 param + exp_avg + exp_avg_sq",
            "bf16_out": w.bf16_out,
            "bytes_per_param": r["bytes_per_param"],
            "launch": r["launch"],
            "stream": "torch's default stream" if args.stream == "default" else "a stream of its own",
            "timing": r["timing"],
        },
        "hbm_gb_s": r["hbm_gb_s"],
        "hbm_frac_of_peak": r["frac"],
        "per_step_ms": r["per_step_ms"],
        "host_wall_s_timed": r["host_wall_s_timed"],
        "plan_create_ms": r["plan_create_ms"],
        "warmup_steps_run": r["warmup_steps_run"],
        "roofline": {
            "bound": "hbm",
            "achieved": r["hbm_gb_s"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": r["frac"],
            "traffic": traffic,
        },
    }
    if args.clip is not None:
        out["clipped_step"] = clipped_step(st, stream, args, t)
    if not args.no_fp8:
        out["fp8_step"] = fp8_step(st, stream, args, t)
    if args.clip is not None:
        out["grad_accumulation"] = accumulation(st, stream, args)
    if not args.no_table:
        out["slice_table_step"] = slice_table_step(st, stream, args, t)
    if not args.no_chain:
        out["unfused_chain"] = unfused_chain(st, stream, args, t)
    segments = [(length, held) for _, length, held, _ in st.segments]
    total = st.total
    st.close()
    del st
    torch.cuda.empty_cache()
    others = [c for c in args.configs.split(",") if c and c != w.name]
    if others:
        out["configs"] = {}
        for name in others:
            if name not in WORKLOAD_BY_NAME:
                raise SystemExit(f"bench.py: unknown workload {name!r} in --configs")
            rc = time_fused(WORKLOADS[WORKLOAD_BY_NAME[name]], dev, stream, args)
            rc.pop("state")
            rc.pop("t")
            out["configs"][name] = rc
            torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, segments, total, t + 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
