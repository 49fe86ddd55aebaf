"""The benchmark's contract pieces that need no GPU: the one-GPU refusal and the
algorithmic byte count its throughput and roofline figures divide by."""
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    line = json.loads(res.stdout.strip().splitlines()[-1])
    assert "error" in line and line["n_gpus"] == 2


def test_decode_bytes_counts_shared_rows_once():
    """Two sequences share block 0 (16 rows); worked by hand:
    seq 0: L = 20 -> block 0 rows 0-15, block 1 rows 0-3; seq 1: L = 17 -> block 0 rows
    0-15 (shared), block 2 row 0.  Distinct rows 16 + 4 + 1 = 21, logical rows 37."""
    import bench
    shape = SimpleNamespace(block_size=16, num_blocks=4, num_kv_heads=2, head_dim=8,
                            elem_bytes=2, num_q_heads=4)
    step = SimpleNamespace(context_lens=np.array([20, 17]),
                           block_tables=np.array([[0, 1, -1], [0, 2, -1]], dtype=np.int32))
    alg, logical = bench.decode_bytes(step, shape)
    row = 2 * 8 * 2                                   # Hkv * D * bytes per element
    q_and_out = 2 * 2 * 4 * 8 * 2                     # B * Hq * D * bytes, read + written
    assert alg == 2 * 21 * row + q_and_out + 4 * 2 + 4 * (2 + 2)
    assert logical == 2 * 37 * row


# ---------------------------------------------------------------------------
# The headline flow and the batch-256 extra legs, driven with a stand-in device and a
# stand-in torch (no GPU): every --steps value a caller may pass runs to the end,
# times exactly that many launches from step 0 and loses no leg.
# ---------------------------------------------------------------------------

class _Event:
    clock = [0.0]

    def __init__(self, enable_timing=True):
        self.t = None

    def record(self, stream=None):
        self.t = _Event.clock[0]

    def elapsed_time(self, other):
        return other.t - self.t


class _Cuda:
    Event = _Event

    @staticmethod
    def synchronize():
        pass

    @staticmethod
    def current_stream(device=None):
        return None

    @staticmethod
    def empty_cache():
        pass


class _Tensor:
    def sum(self):
        return 0.0


class _Torch:
    cuda = _Cuda
    float32 = "float32"

    @staticmethod
    def ones(*a, **kw):
        return _Tensor()


class _Device:
    """Records every launch; each takes 0.08 ms of stand-in stream time."""

    def __init__(self, nsteps):
        self.nsteps = nsteps
        self.log = []
        self.graphs = None

    def _launch(self, kind, t):
        if not 0 <= t < self.nsteps:
            raise IndexError(f"step {t} out of range")
        self.log.append((kind, t))
        _Event.clock[0] += 0.08

    def prepare_fused(self, t):
        return lambda: self._launch("fused", t)

    def step_fused(self, t):
        self._launch("fused", t)

    def prepare_store(self, t):
        return lambda: self._launch("store", t)

    def decode(self, t):
        self._launch("decode", t)

    def capture_graphs(self, steps=None):
        self.graphs = set(range(self.nsteps))

    def replay(self, t):
        assert t in self.graphs
        self._launch("graph", t)

    def capture_sequence(self, steps):
        steps = list(steps)
        dev = self

        class _SeqGraph:
            def replay(self):
                for t in steps:
                    dev._launch("graph_seq", t)
        self.seq_graph, self.seq_outs = _SeqGraph(), {t: None for t in steps}
        return self.seq_graph


def _tiny_case(nsteps=50, batch=3):
    shape = SimpleNamespace(block_size=16, num_blocks=8, num_kv_heads=2, head_dim=8,
                            elem_bytes=2, num_q_heads=4, scale=0.35)
    tables = np.array([[0, 1], [2, 3], [4, 5]], dtype=np.int32)[:batch]
    steps = [SimpleNamespace(context_lens=np.full(batch, 10 + t % 20, dtype=np.int32),
                             block_tables=tables) for t in range(nsteps)]
    return SimpleNamespace(shape=shape, steps=steps, batch=batch)


import pytest  # noqa: E402


@pytest.mark.parametrize("steps", [1, 5, 20, 49, 50, 100])
@pytest.mark.parametrize("warmup", [0, 5, 500])
def test_headline_and_extra_legs_run_for_any_step_count(steps, warmup):
    import bench
    case = _tiny_case()
    dev = _Device(len(case.steps))
    args = bench.parse(["--steps", str(steps), "--warmup", str(warmup)])
    extra = {}
    res = bench.headline(args, _Torch, extra, case, dev)
    fused = [t for kind, t in dev.log if kind == "fused"]
    # first timed pass + warm-up (whole passes, >= --warmup), K timed, K spaced launches
    w = res["warmup_steps"]
    assert w % 50 == 0 and w >= max(warmup, 100)
    assert len(fused) == w + 2 * steps
    timed = fused[w:w + steps]
    assert timed == [i % 50 for i in range(steps)]          # from step 0, cycling
    assert res["ms_per_step"] > 0 and res["value"] > 0 and res["gbs"] > 0
    assert res["warmup_ms"] >= bench.WARMUP_FLOOR_S * 1e3 * 0.99 or w > 100
    assert abs(extra["kernel_us_mean"] - 80.0) < 1e-6      # event time / K
    bench.guarded(extra, "c3_forms", bench.extra_c3, _Torch, case, dev)
    assert not [k for k in extra if k.endswith("_error")], extra
    for key in ("c3_fused_graph_replay_us", "c3_fused_graph_seq_us", "c3_separate_store_us",
                "c3_separate_decode_us", "c3_fused_cold_us_mean"):
        assert key in extra


def test_guarded_leg_records_the_error_and_keeps_going():
    import bench
    extra = {"kept": 1}

    def boom():
        raise StopIteration("ran out")
    bench.guarded(extra, "leg", boom)
    bench.guarded(extra, "ok", lambda: {"ok_value": 2})
    assert extra["kept"] == 1 and extra["ok_value"] == 2
    assert extra["leg_error"].startswith("StopIteration")


def test_cycle_and_warm_up_helpers():
    import bench
    assert bench.cycle(50, 3) == [0, 1, 2]
    assert bench.cycle(50, 52) == list(range(50)) + [0, 1]
    assert bench.cycle(4, 6, start=3) == [3, 0, 1, 2, 3, 0]
    launched = []
    now = [0.0]

    def launch(t):
        launched.append(t)
        now[0] += 0.001
    n, s = bench.warm_up(launch, 50, 0, 0.12, lambda: None, clock=lambda: now[0])
    assert n == 150 and len(launched) == 150 and s >= 0.12     # 50 ms per pass
    launched.clear()
    n, _ = bench.warm_up(launch, 50, 120, 0.0, lambda: None, clock=lambda: now[0])
    assert n == 150                                              # rounded up to passes


def test_cpu_baseline_fans_out_over_worker_processes():
    """The oracle leg on a shrunken batch-256 recipe (8 sequences, 3 steps) with two
    forked workers: every (step, sequence) decode is done once, and the reported core
    count is the worker count."""
    import bench
    from workloads import decode_config
    case = decode_config("C3", batch=8, steps=3, num_blocks=64)
    res = bench.cpu_baseline(case, workers=2)
    assert res["cores"] == 2 and res["kind"] == "oracle" and res["unit"] == "tokens/s"
    assert "24 decoded tokens" in res["sample"]
    assert res["value"] > 0 and res["gbs"] > 0
    assert res["host_cores_available"] == len(os.sched_getaffinity(0))
    assert not bench._CPU                                    # worker state released
