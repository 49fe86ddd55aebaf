"""Shared helpers for the GPU parity tests."""
import sys

import numpy as np

# Tolerances of the method's accuracy target: attention outputs within 1e-2 (max-abs
# and max-abs relative to the largest reference magnitude) for bf16 inputs with fp32
# accumulation, and within 1e-5 for fp32 inputs.
TOL = {"f32": 1e-5, "bf16": 1e-2}


def banner(msg: str):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def assert_close(got: np.ndarray, want: np.ndarray, tol: float, what: str = ""):
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output (a poisoned row leaked?)"
    err = np.abs(got - want)
    max_abs = float(err.max()) if err.size else 0.0
    scale = float(np.abs(want).max()) if want.size else 1.0
    rel = max_abs / scale if scale > 0 else max_abs
    assert max_abs <= tol and rel <= tol, f"{what}: max-abs {max_abs:.3e} rel {rel:.3e} > {tol}"
    return max_abs, rel
