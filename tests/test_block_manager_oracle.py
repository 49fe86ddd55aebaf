"""Pins of the block-manager oracle (CPU): a published XXH64 digest, two traces worked
by hand from the walkthrough's section 五 rules (expected values are literals derived
on paper, not outputs of the oracle), and brute-force invariants over random traces.
"""
import numpy as np
import pytest

from oracle.block_manager import BlockManager, compute_hash


def test_xxh64_published_digest_and_chaining():
    # XXH64 of the empty input with seed 0 is the value the xxHash documentation lists.
    assert compute_hash([], None) == 0xEF46DB3751D8E999
    h0 = compute_hash([1, 2, 3, 4], None)
    assert compute_hash([5, 6, 7, 8], h0) != compute_hash([5, 6, 7, 8], None)
    assert compute_hash([5, 6, 7, 8], h0) == compute_hash([5, 6, 7, 8], h0)


def _state(bm):
    return {s: (list(q.block_table), q.num_cached_tokens) for s, q in bm.seqs.items()}


def test_hand_trace_hits_reclaim_and_latest_index():
    """NB = 7, BS = 4.  Prompt hits, a seal on decode, reclaiming a freed block whose
    content is intact, the forced miss of the last prompt block and latest-wins index."""
    bm = BlockManager(7, 4)
    assert bm.allocate(1, range(1, 11)) == 0                      # A: 10 tokens
    assert bm.seqs[1].block_table == [0, 1, 2]
    assert bm.allocate(2, [1, 2, 3, 4, 5, 6, 7, 8, 99]) == 8        # B: two hits
    assert bm.seqs[2].block_table == [0, 1, 3]
    assert [bm.blocks[i].ref_count for i in range(4)] == [2, 2, 1, 1]
    for tok in (11, 12, 13):                                       # A: seal, then a new block
        bm.append_token(1, tok)
    assert bm.blocks[2].hash == compute_hash([9, 10, 11, 12], compute_hash(
        [5, 6, 7, 8], compute_hash([1, 2, 3, 4], None)))
    assert bm.seqs[1].block_table == [0, 1, 2, 4]
    assert bm.free_block_ids == [5, 6]
    assert not bm.can_allocate(9)
    bm.deallocate(1)
    assert bm.free_block_ids == [5, 6, 4, 2]
    assert bm.allocate(3, list(range(1, 13)) + [50]) == 12         # C: block 2 reclaimed
    assert bm.seqs[3].block_table == [0, 1, 2, 5]
    assert bm.free_block_ids == [6, 4]
    bm.deallocate(2)
    assert bm.free_block_ids == [6, 4, 3]
    assert bm.allocate(4, range(1, 9)) == 4                        # D: last block forced miss
    assert bm.seqs[4].block_table == [0, 6]
    assert not bm.can_allocate(9)
    bm.deallocate(3)
    assert bm.free_block_ids == [4, 3, 5, 2, 1]
    assert bm.allocate(5, [1, 2, 3, 4, 5, 6, 7, 8, 7]) == 8        # E: hits D's block 6
    assert bm.seqs[5].block_table == [0, 6, 4]
    tables, lens, slots = bm.decode_step([4, 5], [20, 21], 3)
    assert tables.tolist() == [[0, 6, 3], [0, 6, 4]]
    assert lens.tolist() == [9, 10]
    assert slots.tolist() == [3 * 4 + 0, 4 * 4 + 1]
    assert bm.free_block_ids == [5, 2, 1]
    assert [bm.blocks[i].ref_count for i in range(7)] == [2, 0, 0, 1, 1, 0, 2]


def test_hand_trace_cached_tokens_are_a_prefix():
    """NB = 10, BS = 2.  The index loses the first block's hash while the second block's
    entry survives; a prompt with both blocks must still cache nothing."""
    bm = BlockManager(10, 2)
    assert bm.allocate(1, [1, 2]) == 0                 # single block: forced miss
    assert bm.allocate(2, [1, 2, 3, 4, 5]) == 2        # hits block 0
    assert bm.seqs[2].block_table == [0, 1, 2]
    assert bm.allocate(3, [1, 2]) == 0                 # forced miss; index H0 -> block 3
    assert bm.seqs[3].block_table == [3]
    bm.deallocate(3)
    bm.deallocate(2)
    assert bm.free_block_ids == [4, 5, 6, 7, 8, 9, 3, 2, 1]
    assert bm.allocate(4, [7] * 14) == 0               # takes 4..9 and 3 (drops H0)
    assert bm.seqs[4].block_table == [4, 5, 6, 7, 8, 9, 3]
    bm.deallocate(1)
    assert bm.free_block_ids == [2, 1, 0]
    # [1, 2] misses (H0 no longer indexed); [3, 4] is indexed in free block 1 with equal
    # tokens, but it follows a miss, so it misses too.
    assert bm.allocate(5, [1, 2, 3, 4, 9]) == 0
    assert bm.seqs[5].block_table == [2, 1, 0]
    assert bm.free_block_ids == []


def _chain_hashes(tokens, bs):
    out, prev = [], None
    for i in range(len(tokens) // bs):
        prev = compute_hash(tokens[i * bs:(i + 1) * bs], prev)
        out.append(prev)
    return out


def check_invariants(bm):
    bs = bm.block_size
    refs = np.zeros(len(bm.blocks), dtype=np.int64)
    for q in bm.seqs.values():
        n = len(q.token_ids)
        assert len(q.block_table) == -(-n // bs)
        assert q.num_cached_tokens % bs == 0 and q.num_cached_tokens <= n - 1 or n == 0
        for b in q.block_table:
            refs[b] += 1
        # every full block of a live sequence holds its tokens and its chain hash
        for i, h in enumerate(_chain_hashes(q.token_ids, bs)):
            blk = bm.blocks[q.block_table[i]]
            assert blk.hash == h
            assert blk.token_ids == q.token_ids[i * bs:(i + 1) * bs]
        if n % bs:
            assert bm.blocks[q.block_table[-1]].ref_count == 1   # partial blocks are private
    assert [b.ref_count for b in bm.blocks] == refs.tolist()
    used = {i for i, r in enumerate(refs) if r > 0}
    assert bm.used_block_ids == used
    assert sorted(bm.free_block_ids) == sorted(set(range(len(bm.blocks))) - used)
    # two tokens share a slot only at the same position after the same tokens
    owner = {}
    for s, q in bm.seqs.items():
        for p in range(len(q.token_ids)):
            slot = bm.slot(s, p)
            end = (p // bs + 1) * bs
            if slot in owner:
                s2, p2 = owner[slot]
                q2 = bm.seqs[s2]
                assert p2 == p and q2.token_ids[:end] == q.token_ids[:end]
            else:
                owner[slot] = (s, p)


def random_trace(bm, rng, n_ops, vocab=3, check=None):
    """Seeded mix of prompts (from a few shared stems), decode appends and releases."""
    bs = bm.block_size
    stems = [list(rng.integers(0, vocab, size=int(rng.integers(1, 4 * bs)))) for _ in range(4)]
    next_id = 0
    for _ in range(n_ops):
        op = rng.random()
        live = sorted(bm.seqs)
        if op < 0.35 or not live:
            stem = stems[int(rng.integers(len(stems)))]
            cut = int(rng.integers(0, len(stem) + 1))
            prompt = stem[:cut] + list(rng.integers(0, vocab, size=int(rng.integers(1, 2 * bs))))
            if bm.can_allocate(len(prompt)):
                bm.allocate(next_id, prompt)
                next_id += 1
        elif op < 0.8:
            s = live[int(rng.integers(len(live)))]
            if bm.can_append(s):
                bm.append_token(s, int(rng.integers(0, vocab)))
        else:
            bm.deallocate(live[int(rng.integers(len(live)))])
        if check is not None:
            check(bm)


@pytest.mark.parametrize("nb,bs,seed", [(12, 2, 0), (20, 4, 1), (40, 3, 2), (64, 16, 3)])
def test_random_traces_keep_invariants(nb, bs, seed):
    bm = BlockManager(nb, bs)
    random_trace(bm, np.random.default_rng(seed), 400, check=check_invariants)


def test_prefix_reuse_happens_in_random_traces():
    """The random traces do exercise hits (otherwise the invariants above prove little)."""
    bm = BlockManager(40, 2)
    rng = np.random.default_rng(5)
    hits = 0
    orig = bm.allocate

    def counting(seq_id, tokens):
        nonlocal hits
        c = orig(seq_id, tokens)
        hits += c
        return c
    bm.allocate = counting
    random_trace(bm, rng, 400)
    assert hits > 20
