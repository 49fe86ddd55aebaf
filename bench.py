#!/usr/bin/env python3
"""Benchmark of the paged KV-cache decode step on one MI355X.

Workload (the headline batch-256 decode): 256 sequences with context lengths
U[100, 1024] at step 0, 16 query / 8 KV heads, head_dim 128, block size 256, bf16,
30 % of the sequences sharing the same first 1-2 physical (ref-counted) blocks, and
50 successive decode steps that each append one token per sequence (a new block is
taken when a token opens one).  One benchmark step = one decode step of that
sequence: the store of the 256 new K/V rows and the decode, fused in one
nv_paged_decode_store launch.  Steps cycle through the 50 steps.  All inputs (pool, tables, slots, schedule, q, new rows) are
resident in HBM before timing starts; the host builds no metadata in the timed loop.

Prints ONE JSON line.  Extra measurements (other workloads, cold-cache kernel time)
go into the same line under "extra".
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=500,
                    help="untimed steps first (default: ten passes over the 50-step workload, "
                         "~45 ms of GPU work: the first ~10 ms after the host-side set-up run "
                         "~6 %% slower)")
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", choices=["c3", "c4", "c5", "copy", "sampler", "small"],
                    default=None,
                    help="run one leg only (for profiler runs)")
    return ap.parse_args()


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


# ---------------------------------------------------------------------------
# GPU legs
# ---------------------------------------------------------------------------

def time_fused_steps(dev, steps_idx, torch, flush=None, graphs=True):
    """Fused store + decode (nv_paged_decode_store), one launch per step, replayed from the
    step's captured HIP graph (or called eagerly); per-step ms from HIP events recorded on
    the stream the graph is launched on."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in steps_idx]
    for (a, b), t in zip(ev, steps_idx):
        if flush is not None:
            flush()
        a.record(stream)
        if graphs:
            dev.replay(t)
        else:
            dev.step_fused(t)
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def headline(args, torch, extra):
    from workloads import decode_config
    from paged_kv_cache_319_amd.harness import DeviceDecode
    case = decode_config("C3")
    sh = case.shape
    nsteps = len(case.steps)
    dev = DeviceDecode(case, poison=True)
    acct = [decode_bytes(st, sh) for st in case.steps]
    flops = [decode_flops(st, sh) for st in case.steps]
    B = case.batch
    row = sh.num_kv_heads * sh.head_dim * sh.elem_bytes
    store_bytes = 2 * 2 * B * row + 4 * B          # K and V rows read + written, slots

    # warmup
    for i in range(args.warmup):
        dev.step_fused(i % nsteps)
    torch.cuda.synchronize()

    # Timed region: exactly K steps, each the fused store + decode of one step, back to
    # back on the stream.  One HIP event pair on that stream brackets the K launches (an
    # event pair per launch would add several microseconds of stream time to each), so
    # event time / K is the kernel's average launch duration; the host clock around the
    # same region (synchronised on both sides) gives the value.
    order = [(args.warmup + i) % nsteps for i in range(args.steps)]
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for t in order:
        dev.step_fused(t)
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    launch_ms = ev0.elapsed_time(ev1) / args.steps
    alg_bytes = np.array([acct[t][0] for t in order], dtype=np.float64) + store_bytes
    log_bytes = np.array([acct[t][1] for t in order], dtype=np.float64)
    fl = np.array([flops[t] for t in order])
    span_s = launch_ms * 1e-3 * args.steps
    gbs = alg_bytes.sum() / span_s / 1e9
    # Spread of single launches: the same steps with an event pair around each launch
    # (these durations include the event overhead).
    step_ms = np.array(time_fused_steps(dev, order, torch, graphs=False))
    res = dict(
        value=B * args.steps / wall, wall=wall,
        ms_per_step=wall * 1e3 / args.steps,
        kernel_us_mean=launch_ms * 1e3,
        per_launch_event_us_p10=float(np.percentile(step_ms, 10) * 1e3),
        per_launch_event_us_p50=float(np.percentile(step_ms, 50) * 1e3),
        per_launch_event_us_p90=float(np.percentile(step_ms, 90) * 1e3),
        alg_bytes_per_launch=float(alg_bytes.mean()),
        gbs=gbs,
        effective_kv_gbs=float(log_bytes.sum() / span_s / 1e9),
        tflops=float(fl.sum() / span_s / 1e12),
        kernel_tokens_per_s=float(B / (launch_ms * 1e-3)),
    )

    if not args.no_extra:
        # The same fused steps replayed from per-step HIP graphs.
        dev.capture_graphs()
        it = iter(order[:50])
        extra["c3_fused_graph_replay_us"] = float(
            time_region(lambda: dev.replay(next(it)), 50, torch) * 1e3)
        # The same steps as two launches (nv_store_kvcache, then nv_paged_decode), each
        # kind timed over back-to-back launches of the 50 steps.
        stores = {t: dev.prepare_store(t) for t in set(order[:50])}
        it = iter(order[:50] * 2)
        st_ms = time_region(lambda: stores[next(it)](), 50, torch)
        it = iter(order[:50])
        de_ms = time_region(lambda: dev.decode(next(it)), 50, torch)
        db = np.array([acct[t][0] for t in order[:50]])
        extra["c3_separate_store_us"] = float(st_ms * 1e3)
        extra["c3_separate_decode_us"] = float(de_ms * 1e3)
        extra["c3_separate_decode_gbs"] = float(db.mean() / (de_ms * 1e-3) / 1e9)
        extra["c3_separate_store_gbs"] = float(store_bytes / (st_ms * 1e-3) / 1e9)
        # Cold-cache kernel times: reading a 1 GiB buffer between steps (outside the
        # events) leaves L2 and the 256 MB MALL holding only clean lines of that buffer.
        scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        cold = np.array(time_fused_steps(dev, order[:20], torch, graphs=False,
                                         flush=lambda: scratch.sum()))
        cb = np.array([acct[t][0] for t in order[:20]]) + store_bytes
        extra["c3_fused_cold_us_mean"] = float(cold.mean() * 1e3)
        extra["c3_fused_cold_gbs"] = float(cb.sum() / (cold.sum() * 1e-3) / 1e9)
        del scratch
    del dev
    torch.cuda.empty_cache()
    return case, res


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


def warm(fn, torch, seconds=0.05):
    """Run fn back to back for `seconds` of wall time: after the host-side set-up of a
    workload the GPU runs its first ~10 ms of work up to 10 % slower."""
    import time
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()


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
    store_bytes = 2 * 2 * case.batch * sh.num_kv_heads * sh.head_dim * sh.elem_bytes + 4 * case.batch
    alg = np.array([decode_bytes(st, sh)[0] for st in case.steps]) + store_bytes
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
    import time
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


def extra_prefill(torch, reps=20, bs=None):
    from workloads import prefill_config
    from paged_kv_cache_319_amd.harness import DevicePrefill
    case = prefill_config(block_size=bs)
    tag = "c5" if bs is None else f"c5_bs{bs}"
    try:
        dev = DevicePrefill(case, poison=True)
        dev.store()
        dev.attend()
    except Exception as e:  # prefill not available: report, do not fail the bench
        return {f"{tag}_prefill_error": str(e)}
    sh = case.shape
    n = case.num_new.astype(np.float64)
    p = case.num_cached.astype(np.float64)
    flops = 4.0 * sh.head_dim * sh.num_q_heads * float(np.sum(n * p + n * (n + 1) / 2))
    dev.store()
    warm(dev.attend, torch)
    store = dev.prepare_store()                 # arguments marshalled once: kernel-bound
    st = time_region(store, reps, torch)        # the store is idempotent
    at = time_region(dev.attend, reps, torch)
    rows = int(case.k_new.shape[0])
    sbytes = 2 * 2 * int(n.sum()) * sh.num_kv_heads * sh.head_dim * sh.elem_bytes + 4 * rows
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
    stream = torch.cuda.current_stream()
    ev = []
    for _ in range(30):
        scratch.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dev.sample()
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    cold = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))
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
DECODE_SOURCES = [os.path.join(ROOT, "paged_kv_cache_319_amd", "csrc", f)
                  for f in ("paged_decode.hip", "common.h")]


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
# CPU baseline: the float64 oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------

def cpu_baseline(case, budget_s=12.0):
    import contextlib
    import oracle
    from workloads import np_storage_dtype, poison_bits
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover
        limit = contextlib.nullcontext()
    sh = case.shape
    with limit:
        kc = oracle.new_pool(sh.num_blocks, sh.block_size, sh.num_kv_heads, sh.head_dim,
                             np_storage_dtype(sh.dtype), poison_bits(sh.dtype))
        vc = kc.copy()
        f = case.fill
        oracle.store_kvcache(kc, vc, f.k, f.v,
                             oracle.fill_slot_mapping(f.block_tables, f.start, f.end,
                                                      sh.block_size))
        # time store + decode of the workload's steps in order, sequence by sequence,
        # until the budget is spent
        t0 = time.perf_counter()
        done = 0
        steps_done = 0
        for st in case.steps:
            slots, _ = oracle.decode_slot_mapping(st.block_tables, st.context_lens,
                                                  sh.block_size)
            oracle.store_kvcache(kc, vc, st.k_new, st.v_new, slots)
            for b in range(case.batch):
                oracle.paged_decode(st.q[b:b + 1], kc, vc, st.block_tables[b:b + 1],
                                    st.context_lens[b:b + 1], sh.scale)
                done += 1
            steps_done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        el = time.perf_counter() - t0
    alg = sum(decode_bytes(st, sh)[0] for st in case.steps[:steps_done])
    return {"value": done / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"store + decode of the first {steps_done} of {len(case.steps)} steps "
                      f"of the batch-256 workload ({done} decoded tokens), numpy float64, "
                      f"BLAS limited to 1 thread, {el:.1f} s",
            "gbs": alg / el / 1e9,
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


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "nvpaged runs on one GPU (sharding across GPUs is a "
                                   "design note only); --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    import torch
    from paged_kv_cache_319_amd import load_library
    load_library()                                    # fails loudly if not built
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(3)
    if args.only == "copy":
        print(json.dumps(copy_calibration(torch)), flush=True)
        return
    if args.only == "c5":
        print(json.dumps(extra_prefill(torch)), flush=True)
        return
    if args.only == "sampler":
        print(json.dumps(extra_sampler(torch)), flush=True)
        return
    if args.only == "c4":
        print(json.dumps(extra_decode("C4", torch)), flush=True)
        return
    if args.only == "small":
        print(json.dumps(extra_small_step(torch)), flush=True)
        return
    extra = {}
    print(f"[bench] headline workload: {args.warmup} warmup + {args.steps} timed steps",
          file=sys.stderr, flush=True)
    case, res = headline(args, torch, extra)
    if not args.no_extra and args.only is None:
        for name in ("C2", "C4"):
            print(f"[bench] extra decode {name}", file=sys.stderr, flush=True)
            extra.update(extra_decode(name, torch))
        print("[bench] extra prefill C5", file=sys.stderr, flush=True)
        extra.update(extra_prefill(torch))
        for bs in (16, 64):
            print(f"[bench] extra block size {bs}", file=sys.stderr, flush=True)
            extra.update(extra_block_size(bs, torch))
        extra.update(extra_prefill(torch, bs=16))
        print("[bench] extra head shards", file=sys.stderr, flush=True)
        extra.update(extra_block_size(None, torch, tp=2))
        extra.update(extra_decode("C4", torch, tp=2))
        print("[bench] extra small step", file=sys.stderr, flush=True)
        extra.update(extra_small_step(torch))
        print("[bench] extra sampler", file=sys.stderr, flush=True)
        extra.update(extra_sampler(torch))
        extra.update(extra_sampler(torch, dtype="f32"))
        extra.update(extra_block_manager())
    extra.update({k: res[k] for k in ("kernel_us_mean", "per_launch_event_us_p10",
                                      "per_launch_event_us_p50", "per_launch_event_us_p90",
                                      "effective_kv_gbs", "tflops", "kernel_tokens_per_s",
                                      "alg_bytes_per_launch")})
    cpu = None
    if not args.no_cpu and args.only is None:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(case)
    sh = case.shape
    line = {
        "metric": "paged-decode KV-read GB/s + decode tokens/s at batch 256; % of HBM peak",
        "value": res["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
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
                     "traffic": recorded_traffic(),
                     "kernel": "paged_decode_kernel<BF16,128,2,4,fast,store,2>"},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
