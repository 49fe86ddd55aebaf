#!/usr/bin/env python3
"""Benchmark of the paged KV-cache decode step on one MI355X.

Workload (the headline batch-256 decode): 256 sequences with context lengths
U[100, 1024] at step 0, 16 query / 8 KV heads, head_dim 128, block size 256, bf16,
30 % of the sequences sharing the same first 1-2 physical (ref-counted) blocks, and
50 successive decode steps that each append one token per sequence (a new block is
taken when a token opens one).  One benchmark step = one decode step of that
sequence: the store of the 256 new K/V rows and the decode, fused in one
nv_paged_decode_store launch.  Steps cycle through the 50 steps; the timed region
starts at step 0.  All inputs (pool, tables, slots, schedule, q, new rows) are
resident in HBM before timing starts; the host builds no metadata in the timed loop.

Warm-up: at least --warmup steps AND at least WARMUP_FLOOR_S seconds of back-to-back
steps, in whole passes over the 50 steps (the chip runs its first ~10 ms of work after
the host-side set-up several per cent slower).  The line records the steps and the time
the warm-up actually took, and the first pass's per-launch time is kept in "extra".

Prints ONE JSON line.  Extra measurements (other workloads, cold-cache kernel time)
go into the same line under "extra"; a failing extra leg records "<leg>_error" there
instead of ending the run.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
import traceback

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
WARMUP_FLOOR_S = 0.1           # least wall time of warm-up steps before the timed region
MAX_CPU_WORKERS = 16           # host cores a one-GPU share of the machine provides
DECODE_KERNEL = "paged_decode_kernel<BF16,128,2,4,fast,store,2>"


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50,
                    help="least number of untimed steps first (the warm-up also lasts at "
                         f"least {WARMUP_FLOOR_S * 1e3:.0f} ms, in whole passes of the "
                         "50-step workload)")
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", choices=["c3", "c4", "c5", "copy", "sampler", "small", "sweep"],
                    default=None,
                    help="run one leg only (for profiler runs); c3 = the headline alone")
    args = ap.parse_args(argv)
    if args.steps < 1:
        ap.error("--steps must be >= 1")
    if args.warmup < 0:
        ap.error("--warmup must be >= 0")
    return args


# ---------------------------------------------------------------------------
# byte / flop accounting
# ---------------------------------------------------------------------------

def decode_bytes(step, shape):
    """Algorithmic bytes of one decode launch: every distinct physical K/V row it must
    read (shared blocks once) + q + out + lengths + the block-table entries used."""
    bs, nb = shape.block_size, shape.num_blocks
    row = shape.num_kv_heads * shape.head_dim * shape.elem_bytes
    seen = np.zeros(nb * bs, dtype=bool)
    logical = 0
    tbl = 0
    for b, L in enumerate(step.context_lens):
        L = int(L)
        nblk = -(-L // bs)
        blocks = step.block_tables[b, :nblk].astype(np.int64)
        offs = np.arange(L)
        seen[blocks[offs // bs] * bs + offs % bs] = True
        logical += L
        tbl += nblk
    B = len(step.context_lens)
    qo = 2 * B * shape.num_q_heads * shape.head_dim * shape.elem_bytes
    unique = int(seen.sum())
    return (2 * unique * row + qo + 4 * B + 4 * tbl), 2 * logical * row


def decode_flops(step, shape):
    return 4.0 * shape.num_q_heads * shape.head_dim * float(np.sum(step.context_lens))


def store_bytes(shape, rows):
    """K and V rows read and written, plus the slots."""
    return 2 * 2 * rows * shape.num_kv_heads * shape.head_dim * shape.elem_bytes + 4 * rows


# ---------------------------------------------------------------------------
# step order, warm-up and timing helpers (no GPU specifics: the tests drive them with
# a stand-in device)
# ---------------------------------------------------------------------------

def cycle(nsteps, n, start=0):
    """n step indices cycling over the workload's nsteps steps from ``start``."""
    return [(start + i) % nsteps for i in range(n)]


def warm_up(launch, nsteps, min_steps, floor_s, sync, clock=time.perf_counter):
    """Launch whole passes over steps 0 .. nsteps-1 until at least ``min_steps`` steps
    and ``floor_s`` seconds have gone by; returns (steps launched, seconds).  Ending on a
    pass boundary means the next step is step 0 and every earlier row is stored."""
    t0 = clock()
    done = 0
    while True:
        for t in range(nsteps):
            launch(t)
        done += nsteps
        sync()
        if done >= min_steps and clock() - t0 >= floor_s:
            return done, clock() - t0


def time_region(fn, reps, torch):
    """Mean ms of one launch: `reps` back-to-back calls bracketed by one HIP event pair on
    the stream they are launched on (per-launch event pairs would add their own overhead)."""
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def time_each(launches, torch, flush=None):
    """Per-launch ms from an event pair around each launch (each pair adds its own
    overhead), optionally with ``flush()`` before each pair, outside the events."""
    stream = torch.cuda.current_stream()
    ev = []
    for fn in launches:
        if flush is not None:
            flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        ev.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def warm(fn, torch, seconds=0.05):
    """Run fn back to back for `seconds` of wall time before an extra leg is timed."""
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()


def guarded(extra, name, fn, *a, **kw):
    """Run one extra leg; merge its dict into ``extra`` or record ``<name>_error``."""
    try:
        res = fn(*a, **kw)
        if res:
            extra.update(res)
    except Exception as e:  # an extra leg never discards the headline
        extra[f"{name}_error"] = f"{type(e).__name__}: {e}"
        traceback.print_exc(file=sys.stderr)


# ---------------------------------------------------------------------------
# the headline: fused store + decode of the batch-256 workload
# ---------------------------------------------------------------------------

def headline(args, torch, extra, case, dev):
    """Warm-up, then exactly args.steps back-to-back fused steps from step 0."""
    sh = case.shape
    nsteps = len(case.steps)
    B = case.batch
    acct = [decode_bytes(st, sh) for st in case.steps]
    flops = [decode_flops(st, sh) for st in case.steps]
    sbytes = store_bytes(sh, B)
    # One prepared call per step: arguments validated and marshalled once, so the host
    # spends a few microseconds per launch (the kernel takes ~80).
    launches = [dev.prepare_fused(t) for t in range(nsteps)]

    # The first pass after set-up, an event pair around each launch (the first launch
    # also carries the one-time load of the kernel code), then the rest of the warm-up.
    t_first = time.perf_counter()
    first = np.array(time_each([launches[t] for t in range(nsteps)], torch))
    first_s = time.perf_counter() - t_first
    w_steps, w_s = warm_up(lambda t: launches[t](), nsteps, max(0, args.warmup - nsteps),
                           WARMUP_FLOOR_S, torch.cuda.synchronize)
    warm_steps = nsteps + w_steps
    warm_ms = (first_s + w_s) * 1e3

    # Timed region: exactly K steps, back to back on the stream.  One HIP event pair on
    # that stream brackets the K launches, so event time / K is the kernel's average
    # launch duration; the host clock around the same region (synchronised on both
    # sides) gives the value.
    order = cycle(nsteps, args.steps)
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for t in order:
        launches[t]()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = ev0.elapsed_time(ev1) / args.steps
    alg_bytes = np.array([acct[t][0] for t in order], dtype=np.float64) + sbytes
    log_bytes = np.array([acct[t][1] for t in order], dtype=np.float64)
    fl = np.array([flops[t] for t in order])
    span_s = launch_ms * 1e-3 * args.steps
    gbs = alg_bytes.sum() / span_s / 1e9
    # Spread of single launches: the same steps with an event pair around each launch.
    step_ms = np.array(time_each([launches[t] for t in order], torch))
    extra.update({
        "c3_first_launch_us": float(first[0] * 1e3),
        "c3_first_pass_us_median": float(np.median(first) * 1e3),
        "c3_first_pass_us_max": float(first.max() * 1e3),
        "kernel_us_mean": float(launch_ms * 1e3),
        "per_launch_event_us_p10": float(np.percentile(step_ms, 10) * 1e3),
        "per_launch_event_us_p50": float(np.percentile(step_ms, 50) * 1e3),
        "per_launch_event_us_p90": float(np.percentile(step_ms, 90) * 1e3),
        "alg_bytes_per_launch": float(alg_bytes.mean()),
        "effective_kv_gbs": float(log_bytes.sum() / span_s / 1e9),
        "tflops": float(fl.sum() / span_s / 1e12),
        "kernel_tokens_per_s": float(B / (launch_ms * 1e-3)),
    })
    return dict(value=B * args.steps / wall, wall=wall, ms_per_step=wall * 1e3 / args.steps,
                gbs=gbs, warmup_steps=warm_steps, warmup_ms=warm_ms)


def time_region_seq(launches, torch):
    """Mean ms of one launch over a list of different launches, back to back, one event
    pair around all of them."""
    it = iter(launches)
    return time_region(lambda: next(it)(), len(launches), torch)


def extra_c3(torch, case, dev, reps=50):
    """The headline steps in other forms, each over `reps` steps cycling from step 0:
    replays of per-step HIP graphs, one graph holding all steps, the store and the
    decode as separate launches, and fused launches with a cold cache."""
    sh = case.shape
    nsteps = len(case.steps)
    order = cycle(nsteps, reps)
    out = {}
    dev.capture_graphs()
    out["c3_fused_graph_replay_us"] = float(
        time_region_seq([lambda t=t: dev.replay(t) for t in order], torch) * 1e3)
    # all steps in one graph: one replay runs them back to back
    dev.capture_sequence(range(nsteps))
    dev.seq_graph.replay()
    out["c3_fused_graph_seq_us"] = float(
        time_region(lambda: dev.seq_graph.replay(), 2, torch) / nsteps * 1e3)
    del dev.seq_graph, dev.seq_outs
    stores = {t: dev.prepare_store(t) for t in set(order)}
    st_ms = time_region_seq([stores[t] for t in order], torch)
    de_ms = time_region_seq([lambda t=t: dev.decode(t) for t in order], torch)
    db = np.array([decode_bytes(case.steps[t], sh)[0] for t in order])
    sb = store_bytes(sh, case.batch)
    out["c3_separate_store_us"] = float(st_ms * 1e3)
    out["c3_separate_decode_us"] = float(de_ms * 1e3)
    out["c3_separate_decode_gbs"] = float(db.mean() / (de_ms * 1e-3) / 1e9)
    out["c3_separate_store_gbs"] = float(sb / (st_ms * 1e-3) / 1e9)
    # Cold-cache kernel times: reading a 1 GiB buffer between steps (outside the
    # events) leaves L2 and the 256 MB MALL holding only clean lines of that buffer.
    scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    cold_order = cycle(nsteps, 20)
    cold = np.array(time_each([lambda t=t: dev.step_fused(t) for t in cold_order], torch,
                              flush=lambda: scratch.sum()))
    cb = np.array([decode_bytes(case.steps[t], sh)[0] for t in cold_order]) + sb
    out["c3_fused_cold_us_mean"] = float(cold.mean() * 1e3)
    out["c3_fused_cold_gbs"] = float(cb.sum() / (cold.sum() * 1e-3) / 1e9)
    del scratch
    return out


# ---------------------------------------------------------------------------
# other workloads (extras)
# ---------------------------------------------------------------------------

def extra_decode(name, torch, reps=50, tp=1):
    """Decode alone on a fresh pool, timed after 50 ms of warm launches.  ``tp`` > 1 runs
    one GPU's head shard of the workload (heads / tp, same lengths and tables)."""
    from workloads import decode_config
    from paged_kv_cache_319_amd.harness import DeviceDecode
    case = decode_config(name, tp=tp)
    dev = DeviceDecode(case, poison=True)
    b, _ = decode_bytes(case.steps[0], case.shape)
    dev.store(0)
    warm(lambda: dev.decode(0), torch)
    ms = time_region(lambda: dev.decode(0), reps, torch)
    tag = name.lower() if tp == 1 else f"{name.lower()}_tp{tp}_shard"
    out = {f"{tag}_decode_us": float(ms * 1e3),
           f"{tag}_decode_gbs": float(b / (ms * 1e-3) / 1e9),
           f"{tag}_decode_hbm_frac": float(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS)}
    del dev
    torch.cuda.empty_cache()
    return out


def extra_block_size(bs, torch, tp=1):
    """The batch-256 workload redrawn with block size `bs` (same lengths, pool bytes and
    shared 256-token prefixes), or as one GPU's head shard under `tp`-way head
    parallelism: fused store + decode cycling over the 50 steps for 50 ms untimed, then
    one timed pass from step 0, back to back."""
    from workloads import decode_config
    from paged_kv_cache_319_amd.harness import DeviceDecode
    case = decode_config("C3", block_size=bs, tp=tp)
    dev = DeviceDecode(case, poison=False)
    nst = len(case.steps)
    sh = case.shape
    alg = np.array([decode_bytes(st, sh)[0] for st in case.steps]) + store_bytes(sh, case.batch)
    for t in range(nst):
        dev.step_fused(t)
    state = {"t": 0}

    def one():
        dev.step_fused(state["t"] % nst)
        state["t"] += 1
    warm(one, torch)
    state["t"] = 0
    ms = time_region(one, nst, torch)
    tag = f"c3_bs{bs}" if tp == 1 else f"c3_tp{tp}_shard"
    out = {f"{tag}_fused_us": float(ms * 1e3),
           f"{tag}_fused_gbs": float(alg.mean() / (ms * 1e-3) / 1e9)}
    del dev
    torch.cuda.empty_cache()
    return out


def extra_small_step(torch, reps=200):
    """The tiny fp32 decode step (4 sequences, lengths 1-200, block size 16): the fused
    store + decode as eager launches, as replays of its captured HIP graph and as a
    prepared call (arguments marshalled once), back to back.  At this size launch
    overhead, not bandwidth, sets the step time."""
    from workloads import decode_config
    from paged_kv_cache_319_amd.harness import DeviceDecode
    case = decode_config("C1")
    dev = DeviceDecode(case)
    dev.capture_graphs([0])
    warm(lambda: dev.step_fused(0), torch)
    eager = time_region(lambda: dev.step_fused(0), reps, torch)
    warm(lambda: dev.replay(0), torch)
    graph = time_region(lambda: dev.replay(0), reps, torch)
    t0 = time.perf_counter()
    for _ in range(reps):
        dev.step_fused(0)
    torch.cuda.synchronize()
    host_eager = (time.perf_counter() - t0) / reps
    t0 = time.perf_counter()
    for _ in range(reps):
        dev.replay(0)
    torch.cuda.synchronize()
    host_graph = (time.perf_counter() - t0) / reps
    launch = dev.prepare_fused(0)
    warm(launch, torch)
    prepared = time_region(launch, reps, torch)
    del dev, launch
    torch.cuda.empty_cache()
    return {"c1_fused_eager_us": float(eager * 1e3), "c1_fused_graph_us": float(graph * 1e3),
            "c1_fused_prepared_us": float(prepared * 1e3),
            "c1_fused_eager_wall_us": float(host_eager * 1e6),
            "c1_fused_graph_wall_us": float(host_graph * 1e6)}


def extra_block_manager():
    """Host cost of the C++ block manager on the batch-256 shape: 256 prompts of
    U[100, 1024] tokens (30 % sharing a 512-token stem) allocated in one prefill step,
    then 50 decode steps, each appending one token per sequence and writing the step's
    block tables, lengths and slots (block size 256, 2048 blocks)."""
    from paged_kv_cache_319_amd import BlockManager, _native
    rng = np.random.default_rng(1003)
    stem = rng.integers(0, 32000, size=512)
    lens = rng.integers(100, 1024, endpoint=True, size=256)
    prompts = []
    for i, n in enumerate(lens):
        p = rng.integers(0, 32000, size=int(n))
        if i % 10 < 3 and n > 512:
            p[:512] = stem
        prompts.append(p)
    bm = BlockManager(2048, 256)
    t0 = time.perf_counter()
    _, cached = bm.prefill_step(list(range(256)), prompts, 6)
    t1 = time.perf_counter()
    lib = _native.load()
    ids = np.arange(256, dtype=np.int64)
    toks = rng.integers(0, 32000, size=(50, 256)).astype(np.int32)
    tables = np.zeros((256, 6), dtype=np.int32)
    ctx = np.zeros(256, dtype=np.int32)
    slots = np.zeros(256, dtype=np.int32)
    ptrs = [a.ctypes.data_as(_native.c_i32p) for a in (tables, ctx, slots)]
    t2 = time.perf_counter()
    for step in range(50):
        st = lib.nv_bm_decode_step(bm._h, ids.ctypes.data_as(_native.c_i64p),
                                   toks[step].ctypes.data_as(_native.c_i32p), 256, ptrs[0], 6,
                                   ptrs[1], ptrs[2])
        if st != 0:
            raise RuntimeError(f"nv_bm_decode_step failed ({st})")
    t3 = time.perf_counter()
    return {"block_manager_prefill_step_ms": float((t1 - t0) * 1e3),
            "block_manager_cached_tokens": int(cached.sum()),
            "block_manager_decode_step_us": float((t3 - t2) / 50 * 1e6)}


def prefill_flops(case):
    sh = case.shape
    n = case.num_new.astype(np.float64)
    p = case.num_cached.astype(np.float64)
    return 4.0 * sh.head_dim * sh.num_q_heads * float(np.sum(n * p + n * (n + 1) / 2))


def extra_prefill(torch, reps=20, bs=None):
    from workloads import prefill_config
    from paged_kv_cache_319_amd.harness import DevicePrefill
    case = prefill_config(block_size=bs)
    tag = "c5" if bs is None else f"c5_bs{bs}"
    dev = DevicePrefill(case, poison=True)
    dev.store()
    dev.attend()
    sh = case.shape
    flops = prefill_flops(case)
    warm(dev.attend, torch)
    store = dev.prepare_store()                 # arguments marshalled once: kernel-bound
    st = time_region(store, reps, torch)        # the store is idempotent
    at = time_region(dev.attend, reps, torch)
    # the real rows are moved; every row, padding included, has a slot to read
    sbytes = 2 * 2 * int(case.num_new.sum()) * sh.num_kv_heads * sh.head_dim * sh.elem_bytes \
        + 4 * int(case.k_new.shape[0])
    out = {f"{tag}_prefill_us": float(at * 1e3),
           f"{tag}_prefill_tflops": float(flops / (at * 1e-3) / 1e12),
           f"{tag}_prefill_mfma_frac": float(flops / (at * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS),
           f"{tag}_store_us": float(st * 1e3),
           f"{tag}_store_gbs": float(sbytes / (st * 1e-3) / 1e9),
           f"{tag}_store_hbm_frac": float(sbytes / (st * 1e-3) / 1e9 / HBM_PEAK_GBS)}
    del dev
    torch.cuda.empty_cache()
    return out


def sampler_bytes(case):
    """Algorithmic bytes of one sampler call: every logit, the noise of the rows with
    T > 0 (greedy rows read none), the temperatures and the tokens."""
    es = 2 if case.dtype == "bf16" else 4
    sampled = int(np.count_nonzero(case.temperatures))
    return case.batch * case.vocab * es + sampled * case.vocab * 4 + 8 * case.batch


def extra_sampler(torch, reps=50, dtype="bf16"):
    """Temperature + Gumbel-max sampler over batch 256 x vocabulary 151,936 (1/8 of the
    rows greedy), timed after 50 ms of warm launches."""
    from workloads import sampler_case
    from paged_kv_cache_319_amd.harness import DeviceSampler
    case = sampler_case(dtype=dtype)
    dev = DeviceSampler(case)
    warm(dev.sample, torch)
    ms = time_region(dev.sample, reps, torch)
    b = sampler_bytes(case)
    # The inputs (233 MB for bf16) fit in the 256 MB MALL, so back-to-back launches
    # partly read cached lines.  Cold: a 1 GiB read between launches (outside the
    # events); the HBM fraction is taken from this median.
    scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    cold = float(np.median(time_each([dev.sample] * 30, torch, flush=lambda: scratch.sum())))
    del scratch
    tag = "sampler" if dtype == "bf16" else f"sampler_{dtype}"
    out = {f"{tag}_us": float(ms * 1e3), f"{tag}_gbs": float(b / (ms * 1e-3) / 1e9),
           f"{tag}_cold_us": float(cold * 1e3),
           f"{tag}_cold_gbs": float(b / (cold * 1e-3) / 1e9),
           f"{tag}_cold_hbm_frac": float(b / (cold * 1e-3) / 1e9 / HBM_PEAK_GBS),
           f"{tag}_alg_bytes": int(b)}
    del dev
    torch.cuda.empty_cache()
    return out


def sweep(torch):
    """Where the kernels sit across sizes: the fused decode step at batch 1 .. 1024 (the
    batch-256 recipe: lengths U[100, 1024], 16 q / 8 kv heads, head_dim 128, block 256,
    bf16; prepared call, back to back after 50 ms warm) and causal prefill over 2-32
    sequences of 128 .. 8192 new tokens (32 q / 8 kv heads, no prefix) beside the
    varlen workload with cached prefixes."""
    from workloads import build_decode, build_prefill, prefill_config, Shape
    from paged_kv_cache_319_amd.harness import DeviceDecode, DevicePrefill
    out = {"decode": [], "prefill": []}
    rng = np.random.default_rng(1234)
    for batch in (1, 4, 16, 64, 256, 1024):
        sh = Shape("bf16", 16, 8, 128, 256, max(64, 5 * batch), 0.5)
        lens = rng.integers(100, 1024, endpoint=True, size=batch)
        case = build_decode("sweep", sh, lens, seed=batch)
        dev = DeviceDecode(case, poison=False)
        launch = dev.prepare_fused(0)
        warm(launch, torch)
        ms = time_region(launch, 100, torch)
        b = decode_bytes(case.steps[0], sh)[0] + store_bytes(sh, batch)
        out["decode"].append({"batch": batch, "us": ms * 1e3, "gbs": b / (ms * 1e-3) / 1e9,
                              "hbm_frac": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                              "tokens_per_s": batch / (ms * 1e-3)})
        del dev, launch
        torch.cuda.empty_cache()
    shapes = [(32, 128), (16, 512), (8, 1024), (4, 2048), (2, 4096), (2, 8192)]
    for seqs, n in shapes:
        sh = Shape("bf16", 32, 8, 128, 256, seqs * (-(-n // 256)) + 8, 0.5)
        case = build_prefill("sweep", sh, [n] * seqs, [0] * seqs, seed=n, pad_to=128)
        out["prefill"].append(_time_prefill(torch, case, f"{seqs} x {n}"))
    out["prefill"].append(_time_prefill(torch, prefill_config(), "varlen with cached prefixes"))
    return {"sweep": out}


def _time_prefill(torch, case, name):
    from paged_kv_cache_319_amd.harness import DevicePrefill
    dev = DevicePrefill(case, poison=False)
    dev.store()
    warm(dev.attend, torch)
    ms = time_region(dev.attend, 20, torch)
    fl = prefill_flops(case)
    res = {"case": name, "us": ms * 1e3, "tflops": fl / (ms * 1e-3) / 1e12,
           "mfma_frac": fl / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}
    del dev
    torch.cuda.empty_cache()
    return res


def copy_calibration(torch, reps=5):
    """A plain 1 GiB device copy: known bytes for scaling the HBM traffic counters."""
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4}


# ---------------------------------------------------------------------------
# HBM traffic recorded by the counter runs
# ---------------------------------------------------------------------------

ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "paged_decode_c3_hbm_traffic.md")
# the kernel and the host code that orders its work (the order shapes the cache hits)
DECODE_SOURCES = [os.path.join(ROOT, "paged_kv_cache_319_amd", "csrc", f)
                  for f in ("paged_decode.hip", "common.h", "prepare.cpp")]


def decode_source_digest():
    import hashlib
    h = hashlib.sha256()
    for path in DECODE_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per decode launch (FETCH_SIZE + WRITE_SIZE, scaled by the copy
    calibration) from the committed counter summary, or None when that summary was
    taken on different decode kernel sources than the ones built now."""
    try:
        text = open(TRAFFIC_RECORD).read()
    except OSError:
        return None
    rec = {}
    for line in text.splitlines():
        if line.startswith("record:"):
            k, _, v = line[len("record:"):].strip().partition("=")
            rec[k.strip()] = v.strip()
    if rec.get("decode_sources_sha256") != decode_source_digest():
        return None
    try:
        return float(rec["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle on the same workload, over the host's cores
# ---------------------------------------------------------------------------

_CPU = {}   # state the forked workers inherit: the workload and the oracle's pools


def _oracle_decode_share(pairs):
    """Worker: the oracle's decode of each (step, sequence) pair, BLAS on one thread."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover
        limit = None
    case, kc, vc = _CPU["case"], _CPU["kc"], _CPU["vc"]
    scale = case.shape.scale
    t0 = time.perf_counter()
    for t, b in pairs:
        st = case.steps[t]
        oracle.paged_decode(st.q[b:b + 1], kc, vc, st.block_tables[b:b + 1],
                            st.context_lens[b:b + 1], scale)
    el = time.perf_counter() - t0
    if limit is not None:
        limit.restore_original_limits()
    return len(pairs), el


def cpu_worker_count():
    return max(1, min(len(os.sched_getaffinity(0)), MAX_CPU_WORKERS))


def cpu_baseline(case, workers=None, steps=None):
    """The float64 oracle, unchanged, on the headline workload: the stores of the steps'
    new rows (one process), then every (step, sequence) decode fanned out over a pool of
    forked worker processes, one per available host core (BLAS limited to one thread
    each).  Decoding step t reads positions below its own length only, so storing every
    step's rows first leaves each decode's inputs as they are at its step.  Must run
    before this process touches the GPU (the workers are forked)."""
    import multiprocessing as mp
    import oracle
    from workloads import np_storage_dtype, poison_bits
    sh = case.shape
    nsteps = len(case.steps) if steps is None else min(steps, len(case.steps))
    workers = cpu_worker_count() if workers is None else workers
    kc = oracle.new_pool(sh.num_blocks, sh.block_size, sh.num_kv_heads, sh.head_dim,
                         np_storage_dtype(sh.dtype), poison_bits(sh.dtype))
    vc = kc.copy()
    f = case.fill
    oracle.store_kvcache(kc, vc, f.k, f.v,
                         oracle.fill_slot_mapping(f.block_tables, f.start, f.end, sh.block_size))
    t0 = time.perf_counter()
    for st in case.steps[:nsteps]:
        slots, _ = oracle.decode_slot_mapping(st.block_tables, st.context_lens, sh.block_size)
        oracle.store_kvcache(kc, vc, st.k_new, st.v_new, slots)
    t_store = time.perf_counter() - t0
    pairs = [(t, b) for t in range(nsteps) for b in range(case.batch)]
    nchunks = workers * 8
    chunks = [pairs[i::nchunks] for i in range(nchunks) if pairs[i::nchunks]]
    _CPU.update(case=case, kc=kc, vc=vc)
    try:
        with mp.get_context("fork").Pool(workers) as pool:
            pool.map(int, range(workers))          # workers started before the clock
            t1 = time.perf_counter()
            res = pool.map(_oracle_decode_share, chunks, chunksize=1)
            t_decode = time.perf_counter() - t1
    finally:
        _CPU.clear()
    done = sum(n for n, _ in res)
    cpu_s = sum(e for _, e in res) + t_store
    el = t_store + t_decode
    alg = sum(decode_bytes(st, sh)[0] for st in case.steps[:nsteps]) \
        + nsteps * store_bytes(sh, case.batch)
    return {"value": done / el, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"store + decode of all {nsteps} steps of the batch-256 workload "
                      f"({done} decoded tokens), numpy float64, decodes spread over "
                      f"{workers} worker processes with one BLAS thread each; "
                      f"{el:.2f} s wall, {cpu_s:.1f} s of CPU work",
            "gbs": alg / el / 1e9,
            "wall_s": el, "cpu_s": cpu_s,
            "cpu_model": cpu_model(),
            "host_cores_available": len(os.sched_getaffinity(0))}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ---------------------------------------------------------------------------
# main
# ---------------------------------------------------------------------------

def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "nvpaged runs on one GPU (sharding across GPUs is a "
                                   "design note only); --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    # The path only (importing the package would import torch before the oracle's
    # workers are forked); the library itself is loaded after the CPU leg.
    lib_path = os.path.join(ROOT, "paged_kv_cache_319_amd", "libnvpaged.so")
    if not os.path.exists(lib_path):
        raise RuntimeError(f"{lib_path} is missing: build the HIP library first")
    headline_run = args.only in (None, "c3")
    case = None
    cpu = None
    if headline_run:
        from workloads import decode_config
        log("building the batch-256 workload")
        case = decode_config("C3")
        if not args.no_cpu and args.only is None:
            # Before the GPU is touched: the oracle's workers are forked from this process.
            log(f"cpu baseline (oracle) on {cpu_worker_count()} worker processes")
            cpu = cpu_baseline(case)
    import torch
    from paged_kv_cache_319_amd import load_library
    load_library()                                    # fails loudly if not built
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(3)
    single = {"copy": lambda: copy_calibration(torch), "c5": lambda: extra_prefill(torch),
              "sampler": lambda: extra_sampler(torch), "c4": lambda: extra_decode("C4", torch),
              "small": lambda: extra_small_step(torch), "sweep": lambda: sweep(torch)}
    if args.only in single:
        print(json.dumps(single[args.only]()), flush=True)
        return

    from paged_kv_cache_319_amd.harness import DeviceDecode
    extra = {}
    dev = DeviceDecode(case, poison=True)
    log(f"headline: >= {args.warmup} warm-up steps and >= {WARMUP_FLOOR_S * 1e3:.0f} ms, "
        f"then {args.steps} timed steps")
    res = headline(args, torch, extra, case, dev)
    if not args.no_extra and args.only is None:
        log("extra: batch-256 step as graph replays, separate launches, cold cache")
        guarded(extra, "c3_forms", extra_c3, torch, case, dev)
    del dev
    torch.cuda.empty_cache()
    if not args.no_extra and args.only is None:
        legs = [("c2", extra_decode, ("C2", torch)), ("c4", extra_decode, ("C4", torch)),
                ("c5", extra_prefill, (torch,)),
                ("c3_bs16", extra_block_size, (16, torch)),
                ("c3_bs64", extra_block_size, (64, torch)),
                ("c5_bs16", lambda t: extra_prefill(t, bs=16), (torch,)),
                ("c3_tp2", lambda t: extra_block_size(None, t, tp=2), (torch,)),
                ("c4_tp2", lambda t: extra_decode("C4", t, tp=2), (torch,)),
                ("c1_small", extra_small_step, (torch,)),
                ("sampler", extra_sampler, (torch,)),
                ("sampler_f32", lambda t: extra_sampler(t, dtype="f32"), (torch,)),
                ("block_manager", extra_block_manager, ())]
        for name, fn, a in legs:
            log(f"extra: {name}")
            guarded(extra, name, fn, *a)
    sh = case.shape
    line = {
        "metric": "paged-decode KV-read GB/s + decode tokens/s at batch 256; % of HBM peak",
        "value": res["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps": res["warmup_steps"],
        "warmup_ms": res["warmup_ms"],
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)*0.5 q/k/v, random block placement)",
        "config": {"workload": "batch-256 paged decode with 30% shared prefix blocks, "
                               "50 successive steps (fused store + decode per step)",
                   "batch": case.batch, "q_heads": sh.num_q_heads, "kv_heads": sh.num_kv_heads,
                   "head_dim": sh.head_dim, "block_size": sh.block_size,
                   "num_blocks": sh.num_blocks, "context_len": "U[100,1024] + step",
                   "parallelism": "single GPU"},
        "decode_kv_read_gbs": res["gbs"],
        "pct_hbm_peak": res["gbs"] / HBM_PEAK_GBS,
        "roofline": {"bound": "hbm", "achieved": res["gbs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": res["gbs"] / HBM_PEAK_GBS,
                     "traffic": recorded_traffic(), "kernel": DECODE_KERNEL},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
