"""Pins of the float64 oracle to facts other than itself (CPU only).

Each pin is chosen so that a plausible slip in the oracle (a dropped scale, a
transposed operand, a wrong block/offset split, a wrong GQA head, an off-by-one
causal edge) fails at least one of them; test_oracle_mutants.py plants such slips
and checks that they are caught.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.brute import decode_brute, prefill_brute
from workloads import Shape, build_decode, build_prefill, decode_config, bf16_bits_from_f32
from oracle_runs import OracleDecode, oracle_pools, oracle_prefill

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32_shape(bs=16, nb=64, hq=2, hkv=1, d=64):
    return Shape("f32", hq, hkv, d, bs, nb, 1.0)


# ---------------------------------------------------------------------------
# golden fixtures from the pages' own worked examples
# ---------------------------------------------------------------------------

def _read_golden(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split("=", 1)
            rows[key.strip()] = [int(x) for x in val.split(",")]
    return rows


def test_golden_block_ids_example():
    g = _read_golden("paging_block_ids.txt")
    table = np.array(g["block_ids"], dtype=np.int32)
    bs = g["block_size"][0]
    for t, want in zip(g["positions"], g["slots"]):
        assert oracle.slot_of(table, t, bs) == want


def test_golden_fragmentation_example():
    """Paging article 6.2: block size 16 with 17-token sequences needs 2 blocks and
    leaves 15 slots of the second block unused.  The oracle's slots for positions
    0..16 must span exactly two physical blocks, the second holding one row."""
    g = _read_golden("paging_fragmentation.txt")
    bs, L = g["block_size"][0], g["length"][0]
    table = np.array([5, 9, -1], dtype=np.int32)
    slots = oracle.fill_slot_mapping(table[None, :], np.array([0]), np.array([L]), bs)
    blocks = sorted(set(int(s) // bs for s in slots))
    assert len(blocks) == g["blocks_needed"][0]
    used_in_last = sum(1 for s in slots if int(s) // bs == 9)
    assert bs - used_in_last == g["wasted_slots"][0]


# ---------------------------------------------------------------------------
# store
# ---------------------------------------------------------------------------

def test_store_roundtrip_and_untouched_rows():
    sh = Shape("bf16", 4, 2, 16, 16, 12, 0.5)
    case = build_decode("t", sh, [1, 16, 17, 40], seed=3, steps=1)
    kc, vc = oracle_pools(sh, case.fill)
    before_k = kc.copy()
    st = case.steps[0]
    slots, _ = oracle.decode_slot_mapping(st.block_tables, st.context_lens, sh.block_size)
    oracle.store_kvcache(kc, vc, st.k_new, st.v_new, slots)
    # the new rows read back bit for bit through gather at position L-1
    for b, L in enumerate(st.context_lens):
        row = kc[st.block_tables[b][(L - 1) // sh.block_size], (L - 1) % sh.block_size]
        assert row.tobytes() == st.k_new[b].tobytes()
    # every other pool row is bit-identical to before
    changed = np.any(kc.reshape(-1, 2 * 16) != before_k.reshape(-1, 2 * 16), axis=1)
    assert set(np.nonzero(changed)[0].tolist()) <= set(int(s) for s in slots)


def test_store_skip_minus_one_and_nan_payload():
    sh = Shape("f32", 2, 2, 8, 4, 3, 1.0)
    kc = np.zeros((3, 4, 2, 8), np.float32)
    vc = np.zeros_like(kc)
    k = np.arange(3 * 16, dtype=np.float32).reshape(3, 2, 8)
    payload = np.array([0x7FC01234], dtype=np.uint32).view(np.float32)[0]
    k[2, 1, 3] = payload
    v = -k
    oracle.store_kvcache(kc, vc, k, v, np.array([5, -1, 2], dtype=np.int32))
    assert kc[1, 1].tobytes() == k[0].tobytes()
    assert kc[0, 2].tobytes() == k[2].tobytes()          # NaN payload kept bit for bit
    assert np.count_nonzero(kc.view(np.uint32)) == np.count_nonzero(k[[0, 2]].view(np.uint32))


def test_gather_inverts_fill_store():
    sh = Shape("bf16", 2, 2, 8, 16, 40, 1.0)
    case = build_decode("t", sh, [5, 33, 64, 100], seed=9, steps=1)
    kc, _ = oracle_pools(sh, case.fill)
    off = 0
    for i in range(len(case.fill.start)):
        s, e = int(case.fill.start[i]), int(case.fill.end[i])
        got = kc[[int(case.fill.block_tables[i][t // 16]) for t in range(s, e)],
                 [t % 16 for t in range(s, e)]]
        assert got.tobytes() == case.fill.k[off:off + e - s].tobytes()
        full = oracle.gather(kc, case.fill.block_tables[i], e)
        assert np.array_equal(full[s:e], oracle.to_f64(case.fill.k[off:off + e - s]))
        off += e - s


# ---------------------------------------------------------------------------
# brute force twins
# ---------------------------------------------------------------------------

def test_decode_matches_brute_force_c1():
    case = decode_config("C1")
    run = OracleDecode(case)
    out = run.run_to(0)
    st = case.steps[0]
    ref = decode_brute(st.q, run.kc, run.vc, st.block_tables, st.context_lens, case.shape.scale)
    assert np.max(np.abs(out - ref)) < 1e-12


def test_decode_matches_brute_force_gqa_bf16():
    sh = Shape("bf16", 6, 2, 16, 4, 40, 0.7)
    case = build_decode("t", sh, [1, 3, 4, 5, 9, 23], seed=11, steps=1)
    run = OracleDecode(case)
    out = run.run_to(0)
    st = case.steps[0]
    ref = decode_brute(st.q, run.kc, run.vc, st.block_tables, st.context_lens, sh.scale)
    assert np.max(np.abs(out - ref)) < 1e-12


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_matches_brute_force(causal):
    sh = Shape("f32", 4, 2, 16, 16, 24, 1.0)
    case = build_prefill("t", sh, [5, 1, 20, 0], [16, 0, 32, 16], seed=5, pad_to=8, causal=causal)
    out, kc, vc, meta = oracle_prefill(case)
    cu_q, cu_k = meta[0], meta[1]
    ref = prefill_brute(case.q, kc, vc, cu_q, cu_k, case.block_tables, sh.scale, causal)
    assert out.shape == ref.shape
    assert np.max(np.abs(out - ref)) < 1e-12


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def test_single_key_returns_v_exactly():
    case = decode_config("C1")
    run = OracleDecode(case)
    out = run.run_to(0)
    st = case.steps[0]
    assert st.context_lens[0] == 1
    v_row = oracle.to_f64(st.v_new[0])            # [Hkv=1, D]
    for h in range(case.shape.num_q_heads):
        assert np.array_equal(out[0, h], v_row[0])


def test_two_key_closed_form():
    """q = (1, 0), K = [(2, 0), (0, 5)], V = [(1, 2), (3, 4)], scale 1/2:
    scores (1, 0) -> weights e/(e+1), 1/(e+1)."""
    kc = np.full((4, 2, 1, 2), np.nan, np.float32)
    vc = kc.copy()
    table = np.array([[3, 1]], np.int32)
    kc[3, 0, 0] = [2, 0]
    kc[3, 1, 0] = [0, 5]
    vc[3, 0, 0] = [1, 2]
    vc[3, 1, 0] = [3, 4]
    q = np.array([[[1, 0]]], np.float32)
    out = oracle.paged_decode(q, kc, vc, table, np.array([2]), 0.5)
    e = math.e
    want = np.array([(e * 1 + 3) / (e + 1), (e * 2 + 4) / (e + 1)])
    assert np.allclose(out[0, 0], want, rtol=0, atol=1e-15)


def test_uniform_keys_give_mean_and_running_mean():
    sh = Shape("f32", 2, 1, 8, 4, 16, 1.0)
    case = build_prefill("t", sh, [7], [5], seed=2, pad_to=1)
    # make every key row identical (prefix and new)
    case.fill.k[:] = case.fill.k[0]
    case.k_new[:] = case.fill.k[0]
    out, kc, vc, meta = oracle_prefill(case)
    V = oracle.gather(vc, case.block_tables[0], 12)[:, 0]
    for i in range(7):
        want = V[:5 + i + 1].mean(axis=0)
        assert np.max(np.abs(out[i, 0] - want)) < 1e-13


def test_scale_zero_gives_mean():
    case = decode_config("C1")
    run = OracleDecode(case)
    run.run_to(0)
    st = case.steps[0]
    out = oracle.paged_decode(st.q, run.kc, run.vc, st.block_tables, st.context_lens, 0.0)
    for b, L in enumerate(st.context_lens):
        V = oracle.gather(run.vc, st.block_tables[b], int(L))[:, 0]
        assert np.max(np.abs(out[b, 0] - V.mean(axis=0))) < 1e-12


def test_dominant_key_selects_its_value():
    """A key whose score exceeds every other by a margin gap pulls the output to its
    value row: |out - V_j| <= (L - 1) e^-gap * 2 max|V|."""
    sh = Shape("f32", 1, 1, 4, 4, 8, 1.0)
    case = build_decode("t", sh, [11], seed=4, steps=1)
    run = OracleDecode(case)
    run.run_to(0)
    st = case.steps[0]
    u = np.array([0.5, -0.5, 0.5, 0.5], np.float32)
    blk, off = st.block_tables[0][6 // 4], 6 % 4
    run.kc[blk, off, 0] = 12 * u
    q = (3 * u)[None, None, :]
    out = oracle.paged_decode(q, run.kc, run.vc, st.block_tables, st.context_lens, 1.0)
    V = oracle.gather(run.vc, st.block_tables[0], 11)[:, 0]
    K = oracle.gather(run.kc, st.block_tables[0], 11)[:, 0]
    s = K @ q[0, 0].astype(np.float64)
    gap = s[6] - np.max(np.delete(s, 6))
    assert gap > 20
    assert np.max(np.abs(out[0, 0] - V[6])) <= 10 * math.exp(-gap) * 2 * np.max(np.abs(V))


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def _permute_blocks(kc, vc, tables, rng):
    nb = kc.shape[0]
    perm = rng.permutation(nb)           # new id of old block b is perm[b]
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    t2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1).astype(np.int32)
    return kc2, vc2, t2


def test_block_permutation_invariance_bit_identical(rng):
    case = decode_config("C2", batch=6, num_blocks=100)
    run = OracleDecode(case)
    out = run.run_to(0)
    st = case.steps[0]
    kc2, vc2, t2 = _permute_blocks(run.kc, run.vc, st.block_tables, rng)
    out2 = oracle.paged_decode(st.q, kc2, vc2, t2, st.context_lens, case.shape.scale)
    assert np.array_equal(out, out2)


def test_prefill_block_permutation_invariance(rng):
    sh = Shape("bf16", 4, 2, 16, 16, 30, 0.5)
    case = build_prefill("t", sh, [9, 30], [32, 16], seed=8, pad_to=16)
    out, kc, vc, meta = oracle_prefill(case)
    kc2, vc2, t2 = _permute_blocks(kc, vc, case.block_tables, rng)
    out2 = oracle.paged_prefill(case.q, kc2, vc2, meta[0], meta[1], t2, sh.scale, True)
    assert np.array_equal(out, out2)


def test_shared_prefix_equals_private_copies():
    case = decode_config("C3", batch=20, steps=3, num_blocks=120)
    assert case.shared_blocks, "the reduced C3 still shares prefix blocks"
    run = OracleDecode(case)
    out = run.run_to(2)
    st = case.steps[2]
    # un-share: copy each shared block to a fresh block per extra referencing sequence
    kc, vc, tables = run.kc.copy(), run.vc.copy(), st.block_tables.copy()
    used = set(int(x) for x in tables.ravel() if x >= 0)
    free = [b for b in range(kc.shape[0]) if b not in used]
    n_unshared = 0
    for blk in case.shared_blocks:
        users = [b for b in range(tables.shape[0]) if blk in tables[b]]
        n_unshared += len(users) - 1
        for b in users[1:]:
            nb = free.pop()
            kc[nb], vc[nb] = kc[blk], vc[blk]
            tables[b][tables[b] == blk] = nb
    assert n_unshared >= 2
    out2 = oracle.paged_decode(st.q, kc, vc, tables, st.context_lens, case.shape.scale)
    assert np.array_equal(out, out2)


def test_decode_equals_last_prefill_row():
    sh = Shape("bf16", 4, 2, 32, 16, 64, 0.5)
    L = np.array([1, 16, 17, 45, 64])
    case = build_decode("t", sh, L, seed=21, steps=1)
    run = OracleDecode(case)
    dec = run.run_to(0)
    st = case.steps[0]
    cu_q = np.arange(len(L) + 1, dtype=np.int32)           # one query row: the last token
    cu_k = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    pre = oracle.paged_prefill(st.q, run.kc, run.vc, cu_q, cu_k, st.block_tables, sh.scale, True)
    assert np.max(np.abs(pre - dec)) < 1e-12


def test_gqa_equals_expanded_kv_heads():
    sh = Shape("f32", 8, 2, 16, 8, 30, 1.0)
    case = build_decode("t", sh, [3, 8, 29, 40], seed=13, steps=1)
    run = OracleDecode(case)
    out = run.run_to(0)
    st = case.steps[0]
    g = sh.group
    kx = np.repeat(run.kc, g, axis=2)          # KV head j -> query heads j*g .. j*g+g-1
    vx = np.repeat(run.vc, g, axis=2)
    out2 = oracle.paged_decode(st.q, kx, vx, st.block_tables, st.context_lens, sh.scale)
    assert np.max(np.abs(out - out2)) == 0.0


def test_batch_order_invariance():
    case = decode_config("C1")
    run = OracleDecode(case)
    out = run.run_to(0)
    st = case.steps[0]
    order = np.array([3, 1, 0, 2])
    out2 = oracle.paged_decode(st.q[order], run.kc, run.vc, st.block_tables[order],
                               st.context_lens[order], case.shape.scale)
    assert np.array_equal(out[order], out2)


# ---------------------------------------------------------------------------
# library special case: contiguous K/V through an identity block table
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [True, False])
def test_identity_table_matches_torch_sdpa(causal):
    rng = np.random.default_rng(77)
    bs, hq, hkv, d = 8, 4, 2, 16
    n, p = 13, 11
    k_len = n + p
    nb = -(-k_len // bs)
    k = rng.standard_normal((nb * bs, hkv, d)).astype(np.float32)
    v = rng.standard_normal((nb * bs, hkv, d)).astype(np.float32)
    q = rng.standard_normal((n, hq, d)).astype(np.float32)
    kc = k.reshape(nb, bs, hkv, d)
    vc = v.reshape(nb, bs, hkv, d)
    table = np.arange(nb, dtype=np.int32)[None, :]
    scale = 0.37
    out = oracle.paged_prefill(q, kc, vc, np.array([0, n]), np.array([0, k_len]), table,
                               scale, causal)
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)           # [Hq, n, D]
    kt = torch.from_numpy(k[:k_len].astype(np.float64)).permute(1, 0, 2)   # [Hkv, k, D]
    vt = torch.from_numpy(v[:k_len].astype(np.float64)).permute(1, 0, 2)
    kt = kt.repeat_interleave(hq // hkv, dim=0)
    vt = vt.repeat_interleave(hq // hkv, dim=0)
    rows = torch.arange(n)[:, None] + p
    cols = torch.arange(k_len)[None, :]
    mask = cols <= rows if causal else torch.ones(n, k_len, dtype=torch.bool)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                                           scale=scale)
    assert np.max(np.abs(out - ref.permute(1, 0, 2).numpy())) < 1e-12


# ---------------------------------------------------------------------------
# input representation
# ---------------------------------------------------------------------------

def test_bf16_decoding_is_exact_and_matches_torch():
    x = np.random.default_rng(1).standard_normal(4096).astype(np.float32) * 3
    bits = bf16_bits_from_f32(x)
    via_torch = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, via_torch)             # round-to-nearest-even agrees
    dec = oracle.to_f64(bits)
    assert np.array_equal(dec, torch.from_numpy(x).to(torch.bfloat16).double().numpy())
