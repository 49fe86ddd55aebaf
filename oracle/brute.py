"""Brute-force twin of the oracle for tiny inputs (test infrastructure).

Pure Python scalars and loops over lists, ``math.exp`` and no numpy arithmetic: it
walks the pool row by row exactly as the paging article's section 4.1 describes
(token t lives in logical block t // B at offset t % B of that block) and evaluates
softmax(q K^T * scale) V term by term, without the max-subtraction the vectorised
oracle uses.  It exists to catch vectorisation slips (a transposed operand, a wrong
axis, a dropped head) in the numpy oracle.
"""
from __future__ import annotations

import math
from typing import List

import numpy as np

from .paged_oracle import to_f64


def _row(pool: List, table_row, t: int, block_size: int, head: int) -> List[float]:
    return pool[int(table_row[t // block_size])][t % block_size][head]


def _softmax_weighted(qv: List[float], keys: List[List[float]], vals: List[List[float]],
                      scale: float) -> List[float]:
    D = len(vals[0])
    w = []
    for kv in keys:
        dot = 0.0
        for a, b in zip(qv, kv):
            dot += a * b
        w.append(math.exp(dot * scale))
    total = sum(w)
    out = [0.0] * D
    for wi, vv in zip(w, vals):
        for d in range(D):
            out[d] += wi * vv[d]
    return [x / total for x in out]


def decode_brute(q, k_cache, v_cache, block_tables, context_lens, scale: float):
    qq = to_f64(q).tolist()
    K = to_f64(k_cache).tolist()
    V = to_f64(v_cache).tolist()
    bs = len(K[0])
    hq = len(qq[0])
    hkv = len(K[0][0])
    out = []
    for b, L in enumerate(context_lens):
        heads = []
        for h in range(hq):
            j = (h * hkv) // hq
            keys = [_row(K, block_tables[b], t, bs, j) for t in range(int(L))]
            vals = [_row(V, block_tables[b], t, bs, j) for t in range(int(L))]
            heads.append(_softmax_weighted(qq[b][h], keys, vals, scale))
        out.append(heads)
    return np.array(out, dtype=np.float64)


def prefill_brute(q, k_cache, v_cache, cu_q, cu_k, block_tables, scale: float, causal: bool):
    qq = to_f64(q).tolist()
    K = to_f64(k_cache).tolist()
    V = to_f64(v_cache).tolist()
    bs = len(K[0])
    hq = len(qq[0]) if qq else 1
    hkv = len(K[0][0])
    out = [None] * len(qq)
    for s in range(len(cu_q) - 1):
        n = int(cu_q[s + 1]) - int(cu_q[s])
        k = int(cu_k[s + 1]) - int(cu_k[s])
        for i in range(n):
            pos = k - n + i
            visible = pos + 1 if causal else k
            heads = []
            for h in range(hq):
                j = (h * hkv) // hq
                keys = [_row(K, block_tables[s], t, bs, j) for t in range(visible)]
                vals = [_row(V, block_tables[s], t, bs, j) for t in range(visible)]
                heads.append(_softmax_weighted(qq[int(cu_q[s]) + i][h], keys, vals, scale))
            out[int(cu_q[s]) + i] = heads
    return np.array(out, dtype=np.float64)
