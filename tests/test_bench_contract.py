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
