"""Structure of the seeded workloads (CPU only)."""
import numpy as np
import pytest

from workloads import decode_config, prefill_config, build_decode, Shape, poison_bits


def _check_tables(tables, lengths, bs, shared):
    B, W = tables.shape
    owners = {}
    for b in range(B):
        n = -(-int(lengths[b]) // bs)
        assert np.all(tables[b, :n] >= 0)
        assert np.all(tables[b, n:] == -1)
        for i, blk in enumerate(tables[b, :n]):
            blk = int(blk)
            if blk in shared:
                assert i == shared.index(blk), "a shared block keeps its logical index"
            else:
                assert blk not in owners, "private blocks are never handed out twice"
                owners[blk] = b


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4"])
def test_decode_structure(name):
    kw = {} if name == "C1" else {"batch": 12, "num_blocks": 300 if name != "C4" else 1600,
                                   "steps": 4 if name == "C3" else None}
    if name == "C4":
        kw["batch"] = 2
    case = decode_config(name, **kw)
    bs = case.shape.block_size
    for st in case.steps:
        _check_tables(st.block_tables, st.context_lens, bs, case.shared_blocks)
        for b, L in enumerate(st.context_lens):
            # the new row never lands in a shared block
            assert int(st.block_tables[b][(L - 1) // bs]) not in case.shared_blocks
    assert case.fill.k.shape[0] == case.fill.num_rows


def test_c1_is_the_stated_workload():
    case = decode_config("C1")
    st = case.steps[0]
    assert st.context_lens.tolist() == [1, 17, 64, 200]
    assert case.shape.block_size == 16 and case.shape.num_blocks == 64
    used = set(int(x) for x in st.block_tables.ravel() if x >= 0)
    assert len(used) == 1 + 2 + 4 + 13
    assert case.shape.scale == 1 / 8
    assert st.q.dtype == np.float32 and st.q.shape == (4, 2, 64)


def test_c3_sharing_and_growth():
    case = decode_config("C3", batch=40, steps=50, num_blocks=400)
    assert len(case.shared_blocks) in (1, 2)
    first = case.steps[0]
    sharers = [b for b in range(40) if int(first.block_tables[b][0]) == case.shared_blocks[0]]
    assert len(sharers) == round(0.3 * 40)
    last = case.steps[-1]
    assert np.all(last.context_lens == first.context_lens + 49)
    grown = np.sum(last.block_tables >= 0) - np.sum(first.block_tables >= 0)
    expect = sum(-(-int(L + 49) // 256) - -(-int(L) // 256) for L in first.context_lens)
    assert grown == expect


def test_prefill_structure():
    case = prefill_config(num_seqs=6, max_new=300)
    assert np.all(case.num_cached % 256 == 0) and np.all(case.num_cached <= 1024)
    n = int(case.num_new.sum())
    assert case.q.shape[0] == n
    assert case.k_new.shape[0] % 128 == 0 and case.k_new.shape[0] >= n
    assert np.all(case.k_new[n:] == poison_bits("bf16"))
    _check_tables(case.block_tables, case.num_new + case.num_cached, 256, [])


def test_seeded_determinism():
    a = decode_config("C3", batch=10, steps=2, num_blocks=100)
    b = decode_config("C3", batch=10, steps=2, num_blocks=100)
    assert np.array_equal(a.fill.k, b.fill.k)
    assert np.array_equal(a.steps[1].q, b.steps[1].q)
    assert np.array_equal(a.steps[1].block_tables, b.steps[1].block_tables)


def test_pool_exhaustion_raises():
    with pytest.raises(MemoryError):
        build_decode("t", Shape("f32", 1, 1, 4, 4, 3, 1.0), [5, 9], seed=1)


@pytest.mark.parametrize("name,tp", [("C3", 2), ("C3", 4), ("C4", 2), ("C2", 8)])
def test_head_shard_keeps_structure(name, tp):
    """One GPU's head shard: num_q_heads / tp and num_kv_heads / tp, with the lengths,
    block tables and shared blocks of the unsharded workload."""
    kw = {"batch": 12, "num_blocks": 300, "steps": 3} if name == "C3" else \
         {"batch": 2, "num_blocks": 300} if name == "C4" else {"batch": 12, "num_blocks": 300}
    full = decode_config(name, **kw)
    shard = decode_config(name, tp=tp, **kw)
    assert shard.shape.num_q_heads * tp == full.shape.num_q_heads
    assert shard.shape.num_kv_heads * tp == full.shape.num_kv_heads
    assert shard.shape.num_q_heads // shard.shape.num_kv_heads == full.shape.group
    for a, b in zip(full.steps, shard.steps):
        assert np.array_equal(a.context_lens, b.context_lens)
        assert np.array_equal(a.block_tables, b.block_tables)
        assert b.q.shape[1] == shard.shape.num_q_heads and b.k_new.shape[1] == shard.shape.num_kv_heads


def test_head_shard_rejects_uneven_split():
    with pytest.raises(ValueError):
        decode_config("C1", tp=2)       # one KV head
    with pytest.raises(ValueError):
        decode_config("C3", tp=3, batch=4, steps=1)
