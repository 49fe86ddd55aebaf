"""Pins of the token sampler oracle (CPU only), and planted mistakes they must catch.

The sampler (walkthrough section 六: divide the logits by the temperature, add Gumbel
noise, take the argmax; temperature 0 = greedy) is pinned against facts that do not
come from the oracle itself:

* the Gumbel-max theorem: over many independent noise draws the token frequencies
  approach softmax(logits / T), here within 5 standard errors;
* a pure-Python brute force that emulates binary32 rounding (double rounding is exact
  for one division or addition, 53 >= 2 * 24 + 2 bits);
* the greedy rule (temperature 0 reads no noise), the small-temperature limit, ties to
  the lowest index, invariance under a constant shift of a row's logits, and exact
  widening of bfloat16 logits.

Each mutant at the end is a plausible slip; at least one pin must fail on it.
"""
import math
import struct

import numpy as np
import pytest

import oracle.sampler as osm
from workloads import bf16_bits_from_f32

LOGITS = np.array([1.0, 0.5, 0.0, -0.5, 2.0, 1.5, -1.0, 0.25], dtype=np.float32)


def _softmax(z, t):
    """softmax(z / t) written out from its definition."""
    e = [math.exp((float(x) - float(max(z))) / t) for x in z]
    s = sum(e)
    return np.array([x / s for x in e])


def _f32(x: float) -> float:
    return struct.unpack("f", struct.pack("f", x))[0]


def _brute(logits, temps, gumbel, emulate_f32):
    out = []
    for b in range(len(temps)):
        t = float(temps[b])
        best, best_i = None, None
        for i in range(len(logits[b])):
            z = float(logits[b][i])
            if t == 0.0:
                s = z
            elif emulate_f32:
                s = _f32(_f32(z / t) + float(gumbel[b][i]))
            else:
                s = z / t + float(gumbel[b][i])
            if best is None or s > best:
                best, best_i = s, i
        out.append(best_i)
    return np.array(out)


# ---- pins ---------------------------------------------------------------------

@pytest.mark.parametrize("t", [0.5, 1.0, 2.0])
def pin_frequencies_follow_softmax(t):
    n = 30000
    rng = np.random.default_rng(7)
    logits = np.tile(LOGITS, (n, 1))
    g = rng.gumbel(size=logits.shape).astype(np.float32)
    tok = osm.sample(logits, np.full(n, t, np.float32), g, score_dtype=np.float64)
    freq = np.bincount(tok, minlength=LOGITS.size) / n
    p = _softmax(LOGITS, t)
    se = np.sqrt(p * (1 - p) / n)
    assert np.all(np.abs(freq - p) <= 5 * se), (freq, p)


def pin_brute_force():
    rng = np.random.default_rng(11)
    for emulate_f32, dt in ((True, np.float32), (False, np.float64)):
        logits = rng.standard_normal((9, 13)).astype(np.float32) * 2
        temps = np.array([0, 0.5, 0.7, 1.0, 1.3, 0, 2.0, 0.25, 0.9], np.float32)
        g = rng.gumbel(size=logits.shape).astype(np.float32)
        got = osm.sample(logits, temps, g, score_dtype=dt)
        assert np.array_equal(got, _brute(logits, temps, g, emulate_f32))


def pin_greedy_reads_no_noise():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((5, 40)).astype(np.float32)
    g = np.full(logits.shape, np.nan, np.float32)           # must never be read
    got = osm.sample(logits, np.zeros(5, np.float32), g)
    assert np.array_equal(got, np.argmax(logits, axis=1))


def pin_small_temperature_is_greedy():
    rng = np.random.default_rng(5)
    logits = np.round(rng.standard_normal((20, 30)) * 4, 1).astype(np.float32)
    logits += np.arange(30, dtype=np.float32) * 1e-3         # no exact ties
    g = np.clip(rng.gumbel(size=logits.shape), -5, 5).astype(np.float32)
    got = osm.sample(logits, np.full(20, 1e-3, np.float32), g)
    assert np.array_equal(got, np.argmax(logits, axis=1))


def pin_ties_go_to_lowest_index():
    logits = np.zeros((3, 6), np.float32)
    logits[1, [2, 4]] = 1.0
    logits[2, [1, 5]] = 3.0
    g = np.zeros((3, 6), np.float32)
    for temps in (np.zeros(3, np.float32), np.full(3, 0.8, np.float32)):
        assert list(osm.sample(logits, temps, g)) == [0, 2, 1]


def pin_shift_invariance():
    rng = np.random.default_rng(9)
    logits = rng.standard_normal((40, 50)) * 2
    temps = rng.uniform(0.5, 1.5, 40).astype(np.float32)
    g = rng.gumbel(size=logits.shape).astype(np.float32)
    a = osm.sample(logits.astype(np.float32), temps, g, score_dtype=np.float64)
    b = osm.sample((logits + 3.0).astype(np.float32), temps, g, score_dtype=np.float64)
    # rounding of the shifted float32 logits can only move near-ties
    assert np.mean(a == b) >= 0.95


def pin_bf16_logits_widen_exactly():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((6, 64)).astype(np.float32)
    bits = bf16_bits_from_f32(x)
    as_f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    temps = np.array([0, 0.6, 0.8, 1.0, 0, 1.2], np.float32)
    g = rng.gumbel(size=x.shape).astype(np.float32)
    assert np.array_equal(osm.sample(bits, temps, g), osm.sample(as_f32, temps, g))


def pin_float32_scores_match_exact_except_near_ties():
    rng = np.random.default_rng(17)
    logits = (rng.standard_normal((200, 500)) * 2).astype(np.float32)
    temps = rng.uniform(0.5, 1.0, 200).astype(np.float32)
    g = rng.gumbel(size=logits.shape).astype(np.float32)
    a = osm.sample(logits, temps, g, score_dtype=np.float32)
    b = osm.sample(logits, temps, g, score_dtype=np.float64)
    for r in np.flatnonzero(a != b):
        s = logits[r].astype(np.float64) / float(temps[r]) + g[r]
        assert s[b[r]] - s[a[r]] <= 1e-5 * (1 + abs(s[b[r]])), r


PINS = [(name, fn) for name, fn in sorted(globals().items()) if name.startswith("pin_")]


@pytest.mark.parametrize("name", [n for n, _ in PINS])
def test_pin(name):
    fn = dict(PINS)[name]
    marks = getattr(fn, "pytestmark", [])
    if marks:
        for args in marks[0].args[1]:
            fn(args)
    else:
        fn()


# ---- planted mistakes ---------------------------------------------------------

def _mutant(kind):
    def sample(logits, temperatures, gumbel, score_dtype=np.float32):
        z = osm.to_f64(logits)
        temps = np.asarray(temperatures, np.float32)
        out = np.empty(z.shape[0], np.int64)
        for b in range(z.shape[0]):
            t = score_dtype(temps[b])
            zz = z[b].astype(score_dtype)
            gg = np.asarray(gumbel[b]).astype(score_dtype)
            if temps[b] == 0 and kind != "greedy_adds_noise":
                s = zz
            elif kind == "greedy_adds_noise" and temps[b] == 0:
                s = zz + gg
            elif kind == "times_t":
                s = zz * t + gg
            elif kind == "noise_subtracted":
                s = zz / t - gg
            elif kind == "noise_scaled_too":
                s = (zz + gg) / t
            elif kind == "no_temperature":
                s = zz + gg
            else:
                s = zz / t + gg
            if kind == "last_tie":
                out[b] = len(s) - 1 - int(np.argmax(s[::-1]))
            else:
                out[b] = int(np.argmax(s))
        return out
    return sample


@pytest.mark.parametrize("kind", ["times_t", "noise_subtracted", "noise_scaled_too",
                                  "no_temperature", "last_tie", "greedy_adds_noise"])
def test_mutant_is_caught(kind, monkeypatch):
    monkeypatch.setattr(osm, "sample", _mutant(kind))
    failed = []
    for name, fn in PINS:
        try:
            test_pin(name)
        except AssertionError:
            failed.append(name)
    assert failed, f"mutant {kind} passed every pin"
