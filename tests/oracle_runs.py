"""Drive the float64 oracle over generated workloads (test-side glue, CPU only)."""
from __future__ import annotations

import numpy as np

import oracle
from workloads import DecodeCase, PrefillCase, np_storage_dtype, poison_bits


def oracle_pools(shape, fill):
    """Fresh poisoned pools with the fill rows stored through the oracle's own slots."""
    sd = np_storage_dtype(shape.dtype)
    kc = oracle.new_pool(shape.num_blocks, shape.block_size, shape.num_kv_heads,
                         shape.head_dim, sd, poison_bits(shape.dtype))
    vc = kc.copy()
    slots = oracle.fill_slot_mapping(fill.block_tables, fill.start, fill.end, shape.block_size)
    oracle.store_kvcache(kc, vc, fill.k, fill.v, slots)
    return kc, vc


class OracleDecode:
    """Replays a decode workload step by step on oracle pools."""

    def __init__(self, case: DecodeCase):
        self.case = case
        self.kc, self.vc = oracle_pools(case.shape, case.fill)
        self.next_step = 0

    def store_step(self, t: int):
        st = self.case.steps[t]
        slots, _ = oracle.decode_slot_mapping(st.block_tables, st.context_lens,
                                              self.case.shape.block_size)
        oracle.store_kvcache(self.kc, self.vc, st.k_new, st.v_new, slots)

    def run_to(self, t: int, seqs=None, scale=None):
        """Store steps up to and including t, then decode step t (optionally only
        the sequences in ``seqs``).  Returns float64 [B or len(seqs), Hq, D]."""
        while self.next_step <= t:
            self.store_step(self.next_step)
            self.next_step += 1
        st = self.case.steps[t]
        idx = np.arange(len(st.context_lens)) if seqs is None else np.asarray(seqs)
        return oracle.paged_decode(st.q[idx], self.kc, self.vc, st.block_tables[idx],
                                   st.context_lens[idx],
                                   self.case.shape.scale if scale is None else scale)


def oracle_prefill(case: PrefillCase, seqs=None, scale=None):
    """Store the prefix and the new rows through the oracle, then run its prefill (with
    the shape's 1/sqrt(head_dim) scale unless ``scale`` is given).

    Returns (out float64 [sum(num_new), Hq, D], kc, vc, metadata tuple)."""
    sh = case.shape
    kc, vc = oracle_pools(sh, case.fill)
    meta = oracle.prefill_metadata(case.block_tables, case.num_cached, case.num_new,
                                   sh.block_size, case.pad_to)
    cu_q, cu_k, _, _, slots = meta
    oracle.store_kvcache(kc, vc, case.k_new, case.v_new, slots)
    out = oracle.paged_prefill(case.q, kc, vc, cu_q, cu_k, case.block_tables,
                               sh.scale if scale is None else scale, case.causal)
    return out, kc, vc, meta
