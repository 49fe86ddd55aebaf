"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant below is a plausible slip in the float64 oracle.  It is patched into
the oracle module for the duration of one check, the pin tests of
test_oracle_pins.py are run against it, and at least one of them must fail.  The
brute-force twin is never patched, so it stays an independent reference.
"""
import inspect

import numpy as np
import pytest

import oracle
import oracle.paged_oracle as po
import test_oracle_pins as pins


def _all_pins():
    out = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        params = inspect.signature(fn).parameters
        if "causal" in params:
            out.append((name + "[causal]", lambda fn=fn: fn(True)))
            out.append((name + "[full]", lambda fn=fn: fn(False)))
        elif "rng" in params:
            out.append((name, lambda fn=fn: fn(np.random.default_rng(12345))))
        else:
            out.append((name, fn))
    return out


# ---- mutants ----------------------------------------------------------------

def m_no_scale(q, K, V, scale, last_key):
    return _orig_attend(q, K, V, 1.0, last_key)


def m_pv_uses_k(q, K, V, scale, last_key):
    return _orig_attend(q, K, K, scale, last_key)


def m_causal_excludes_self(q, K, V, scale, last_key):
    return _orig_attend(q, K, V, scale, np.asarray(last_key) - 1)


def m_causal_sees_next(q, K, V, scale, last_key):
    return _orig_attend(q, K, V, scale, np.minimum(np.asarray(last_key) + 1, K.shape[0] - 1))


def m_slot_transposed(block_table_row, pos, block_size):
    return int(block_table_row[pos // block_size]) + (pos % block_size) * block_size


def m_slot_logical_block(block_table_row, pos, block_size):
    return (pos // block_size) * block_size + pos % block_size


def m_gather_drops_last(cache, block_table_row, length):
    return _orig_gather(cache, block_table_row, max(0, length - 1)) if length > 1 else \
        _orig_gather(cache, block_table_row, length)


def m_store_ignores_skip(k_cache, v_cache, k, v, slot_mapping):
    nb, bs = k_cache.shape[:2]
    for i, s in enumerate(np.asarray(slot_mapping)):
        blk, off = divmod(int(s) % (nb * bs), bs)
        k_cache[blk, off] = k[i]
        v_cache[blk, off] = v[i]


def _decode_gqa_modulo(q, k_cache, v_cache, block_tables, context_lens, scale):
    q64 = po.to_f64(q)
    B, Hq, D = q64.shape
    Hkv = k_cache.shape[2]
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(context_lens[b])
        K = po.gather(k_cache, block_tables[b], L)
        V = po.gather(v_cache, block_tables[b], L)
        for h in range(Hq):
            j = h % Hkv
            out[b, h] = po.attend(q64[b, h][None, :], K[:, j], V[:, j], scale, np.array([L - 1]))[0]
    return out


_orig_attend = po.attend
_orig_gather = po.gather

MUTANTS = {
    "no_scale": {"attend": m_no_scale},
    "pv_uses_k": {"attend": m_pv_uses_k},
    "causal_excludes_self": {"attend": m_causal_excludes_self},
    "causal_sees_next": {"attend": m_causal_sees_next},
    "slot_transposed": {"slot_of": m_slot_transposed},
    "slot_ignores_table": {"slot_of": m_slot_logical_block},
    "gather_drops_last": {"gather": m_gather_drops_last},
    "store_ignores_skip": {"store_kvcache": m_store_ignores_skip},
    "gqa_modulo": {"paged_decode": _decode_gqa_modulo},
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_mutant_is_caught(mutant, monkeypatch):
    for attr, fn in MUTANTS[mutant].items():
        monkeypatch.setattr(po, attr, fn)
        monkeypatch.setattr(oracle, attr, fn)
    failed = []
    for name, run in _all_pins():
        try:
            run()
        except Exception:  # an assertion or an indexing error both count as caught
            failed.append(name)
    assert failed, f"mutant {mutant} passed every pin"
