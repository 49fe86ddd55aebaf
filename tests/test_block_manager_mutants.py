"""Planted mistakes in the block-manager oracle must be caught by its pins (CPU only).

Each mutant edits one statement of the oracle's BlockManager source (a plausible slip:
a dropped rule, a reversed order, a wrong index), builds the edited class, and runs
every pin of test_block_manager_oracle.py against it; at least one must fail.
"""
import inspect
import textwrap

import numpy as np
import pytest

import oracle.block_manager as obm
import test_block_manager_oracle as pins

MUTANTS = {
    "hits_after_a_miss": ("and i < nblk - 1 and not missed", "and i < nblk - 1"),
    "last_prompt_block_may_hit": ("and i < nblk - 1 and not missed", "and not missed"),
    "freed_blocks_never_reclaimed": (
        "if cand is not None and self.blocks[cand].token_ids == toks:",
        "if cand is not None and self.blocks[cand].token_ids == toks "
        "and cand in self.used_block_ids:"),
    "index_first_wins": ("self.hash_to_block_id[blk.hash] = blk.block_id",
                         "self.hash_to_block_id.setdefault(blk.hash, blk.block_id)"),
    "seal_without_prefix": ("self._seal(last, seq.token_ids[n - bs:n], prefix)",
                            "self._seal(last, seq.token_ids[n - bs:n], None)"),
    "seal_off_by_one_block": ("self._seal(last, seq.token_ids[n - bs:n], prefix)",
                              "self._seal(last, seq.token_ids[n - bs - 1:n - 1], prefix)"),
    "free_pool_lifo": ("blk = self._take(self.free_block_ids[0])",
                       "blk = self._take(self.free_block_ids[-1])"),
    "release_first_to_last": ("for block_id in reversed(seq.block_table):",
                              "for block_id in seq.block_table:"),
    "new_block_one_token_late": ("if (n - 1) % bs == 0:", "if n % bs == 0 and n > bs:"),
    "decode_slot_of_next_position": ("slots[b] = self.slot(s, lens[b] - 1)",
                                     "slots[b] = self.slot(s, lens[b] % (len(seq.block_table) * self.block_size))"),
    "cached_counts_partial_blocks": ("seq.num_cached_tokens += bs",
                                     "seq.num_cached_tokens += len(toks) + (1 if i == 0 else 0)"),
}


def _mutant_class(old: str, new: str):
    src = textwrap.dedent(inspect.getsource(obm.BlockManager))
    assert src.count(old) == 1, old
    ns = dict(vars(obm))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns["BlockManager"]


def _pins():
    out = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        params = inspect.signature(fn).parameters
        if "nb" in params:
            for nb, bs, seed in ((12, 2, 0), (20, 4, 1), (40, 3, 2)):
                out.append(lambda fn=fn, a=(nb, bs, seed): fn(*a))
        else:
            out.append(fn)
    return out


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    cls = _mutant_class(*MUTANTS[name])
    monkeypatch.setattr(pins, "BlockManager", cls)
    failures = 0
    for pin in _pins():
        try:
            pin()
        except (AssertionError, ValueError, MemoryError, IndexError, KeyError):
            failures += 1
    assert failures > 0, f"mutant {name} passed every pin"


def test_unmutated_oracle_passes_every_pin():
    for pin in _pins():
        pin()
