"""GPU parity: store_kvcache (bit-exact) and paged decode (tolerance) vs the oracle."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from workloads import decode_config, build_decode, Shape
from oracle_runs import OracleDecode
from gpu_common import TOL, assert_close, banner


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from paged_kv_cache_319_amd import load_library
    load_library()
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"


def _run_decode(case, t_list, seqs=None):
    """Replay the workload on both sides; return [(t, gpu_f64, oracle_f64)]."""
    from paged_kv_cache_319_amd.harness import DeviceDecode, to_host_f64
    dev = DeviceDecode(case)
    orc = OracleDecode(case)
    res = []
    last = max(t_list)
    for t in range(last + 1):
        dev.store(t)
        if t in t_list:
            out = to_host_f64(dev.decode(t))
            want = orc.run_to(t, seqs)
            got = out if seqs is None else out[np.asarray(seqs)]
            res.append((t, got, want))
    torch.cuda.synchronize()
    return dev, orc, res


# ---------------------------------------------------------------------------
# store
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4"])
def test_store_bit_exact_full_pool(name):
    from paged_kv_cache_319_amd.harness import DeviceDecode, to_host_bits
    banner(f"store bit-exact {name}")
    case = decode_config(name)
    dev = DeviceDecode(case)
    orc = OracleDecode(case)
    for t in range(len(case.steps)):
        dev.store(t)
        orc.store_step(t)
    torch.cuda.synchronize()
    for gpu, ref in ((dev.kc, orc.kc), (dev.vc, orc.vc)):
        got = to_host_bits(gpu)
        assert got.dtype == ref.dtype
        assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), "pool bits differ"


def test_store_strided_rows_and_skips():
    """k / v as views into a fused [N, 3, Hkv, D] buffer; -1 slots leave rows untouched."""
    from paged_kv_cache_319_amd import nv_store_kvcache
    from paged_kv_cache_319_amd.harness import to_host_bits
    import oracle
    banner("store strided")
    rng = np.random.default_rng(5)
    nb, bs, hkv, d, n = 6, 16, 2, 64, 40
    fused = rng.standard_normal((n, 3, hkv, d)).astype(np.float32)
    slots = rng.permutation(nb * bs)[:n].astype(np.int32)
    slots[::7] = -1
    kc = np.full((nb, bs, hkv, d), np.nan, np.float32)
    vc = kc.copy()
    oracle.store_kvcache(kc, vc, fused[:, 1], fused[:, 2], slots)
    f = torch.from_numpy(fused).cuda()
    gk = torch.full((nb, bs, hkv, d), float("nan"), device="cuda")
    gv = gk.clone()
    nv_store_kvcache(f[:, 1], f[:, 2], gk, gv, torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(gk).view(np.uint32), kc.view(np.uint32))
    assert np.array_equal(to_host_bits(gv).view(np.uint32), vc.view(np.uint32))


# ---------------------------------------------------------------------------
# decode: the four decode workloads
# ---------------------------------------------------------------------------

def test_decode_c1_fp32():
    banner("decode C1")
    case = decode_config("C1")
    _, _, res = _run_decode(case, [0])
    for t, got, want in res:
        assert_close(got, want, TOL["f32"], "C1")
    # single-key sequence: output equals its V row exactly
    v0 = case.steps[0].v_new[0, 0].astype(np.float64)
    for h in range(case.shape.num_q_heads):
        assert np.array_equal(res[0][1][0, h], v0)


def test_decode_c2_bf16():
    banner("decode C2")
    case = decode_config("C2")
    _, _, res = _run_decode(case, [0])
    for t, got, want in res:
        assert_close(got, want, TOL["bf16"], "C2")


def test_decode_c3_fifty_steps():
    banner("decode C3")
    case = decode_config("C3")
    _, _, res = _run_decode(case, [0, 1, 17, 31, 49])
    for t, got, want in res:
        assert_close(got, want, TOL["bf16"], f"C3 step {t}")


def test_decode_c4_long_context_split():
    banner("decode C4")
    case = decode_config("C4")
    _, _, res = _run_decode(case, [0])
    for t, got, want in res:
        assert_close(got, want, TOL["bf16"], "C4")


# ---------------------------------------------------------------------------
# decode: edge cases
# ---------------------------------------------------------------------------

EDGE_LENGTHS = [1, 2, 63, 64, 65, 255, 256, 257, 511, 512, 513, 767, 1024, 1025, 2047]


@pytest.mark.parametrize("dtype,d,hq,hkv,bs", [
    ("bf16", 128, 16, 8, 256), ("bf16", 128, 8, 8, 16), ("bf16", 128, 32, 8, 16),
    ("bf16", 64, 16, 2, 32), ("bf16", 128, 64, 8, 256), ("f32", 64, 2, 1, 16),
    ("f32", 128, 8, 2, 64), ("f32", 64, 8, 1, 256), ("bf16", 128, 16, 8, 48),
    ("bf16", 128, 16, 8, 1024), ("f32", 64, 4, 2, 272),
])
def test_decode_shapes_and_chunk_edges(dtype, d, hq, hkv, bs):
    banner(f"decode edges {dtype} d{d} hq{hq} hkv{hkv} bs{bs}")
    lengths = EDGE_LENGTHS
    nb = sum(-(-L // bs) for L in lengths) + 3
    sh = Shape(dtype, hq, hkv, d, bs, nb, 0.5 if dtype == "bf16" else 1.0)
    case = build_decode("edge", sh, lengths, seed=hq * 31 + d + bs)
    _, _, res = _run_decode(case, [0])
    for t, got, want in res:
        assert_close(got, want, TOL[dtype], f"edges {dtype} d{d} g{hq // hkv} bs{bs}")


def test_decode_repeat_is_bit_identical_and_workspace_reuse():
    """Two identical calls give identical bits, and a following call with a different
    batch on the same (dirty) workspace still matches the oracle."""
    from paged_kv_cache_319_amd.harness import DeviceDecode, to_host_bits, to_host_f64
    banner("decode repeat")
    case = decode_config("C2", batch=24)
    dev = DeviceDecode(case)
    dev.store(0)
    a = to_host_bits(dev.decode(0)).copy()
    b = to_host_bits(dev.decode(0)).copy()
    assert np.array_equal(a, b)
    small = decode_config("C2", batch=5, seed=99)
    dev2 = DeviceDecode(small)
    dev2.workspace = dev.workspace          # reuse the same (already used) workspace
    dev2.store(0)
    got = to_host_f64(dev2.decode(0))
    want = OracleDecode(small).run_to(0)
    assert_close(got, want, TOL["bf16"], "reused workspace")


def test_decode_block_permutation_and_sharing_bit_identical():
    """The schedule depends only on logical structure: permuting physical block ids, or
    replacing shared prefix blocks by private copies, leaves the GPU output bit-identical."""
    from paged_kv_cache_319_amd import nv_paged_decode
    from paged_kv_cache_319_amd.harness import DeviceDecode, to_host_bits, i32
    banner("decode permutation/sharing")
    case = decode_config("C3", batch=64, steps=1)
    dev = DeviceDecode(case)
    dev.store(0)
    base = to_host_bits(dev.decode(0)).copy()
    st = case.steps[0]
    nb = case.shape.num_blocks
    perm = torch.from_numpy(np.random.default_rng(3).permutation(nb)).cuda()
    kc2 = torch.empty_like(dev.kc)
    vc2 = torch.empty_like(dev.vc)
    kc2[perm] = dev.kc
    vc2[perm] = dev.vc
    bt = st.block_tables
    pm = perm.cpu().numpy()
    bt2 = np.where(bt >= 0, pm[np.maximum(bt, 0)], -1).astype(np.int32)
    out2 = torch.empty_like(dev.out)
    s = dev.steps[0]
    nv_paged_decode(out2, s["q"], kc2, vc2, i32(bt2, "cuda"), s["lens"], s["max_len"],
                    case.shape.scale, workspace=dev.workspace)
    assert np.array_equal(to_host_bits(out2), base)
    # un-share the prefix blocks
    used = set(int(x) for x in bt.ravel() if x >= 0)
    free = [b for b in range(nb) if b not in used]
    bt3 = bt.copy()
    for blk in case.shared_blocks:
        users = [b for b in range(bt.shape[0]) if blk in bt[b]]
        for b in users[1:]:
            nbk = free.pop()
            dev.kc[nbk] = dev.kc[blk]
            dev.vc[nbk] = dev.vc[blk]
            bt3[b][bt3[b] == blk] = nbk
    assert not np.array_equal(bt3, bt)
    out3 = torch.empty_like(dev.out)
    nv_paged_decode(out3, s["q"], dev.kc, dev.vc, i32(bt3, "cuda"), s["lens"], s["max_len"],
                    case.shape.scale, workspace=dev.workspace)
    assert np.array_equal(to_host_bits(out3), base)


def test_decode_empty_batch_is_noop():
    from paged_kv_cache_319_amd import nv_paged_decode
    banner("decode empty batch")
    kc = torch.zeros((4, 16, 1, 64), device="cuda")
    q = torch.zeros((0, 2, 64), device="cuda")
    out = torch.zeros((0, 2, 64), device="cuda")
    nv_paged_decode(out, q, kc, kc, torch.zeros((0, 4), dtype=torch.int32, device="cuda"),
                    torch.zeros((0,), dtype=torch.int32, device="cuda"), 1, 0.125)
    torch.cuda.synchronize()


def test_decode_schedule_changes_nothing():
    """The host schedule only reorders work: outputs with and without it are bit-identical."""
    from paged_kv_cache_319_amd.harness import DeviceDecode, to_host_bits
    banner("decode schedule")
    for name, kw in (("C3", dict(batch=96, steps=1)), ("C2", dict(batch=12))):
        case = decode_config(name, **kw)
        a = DeviceDecode(case, scheduled=True)
        b = DeviceDecode(case, scheduled=False)
        a.store(0)
        b.store(0)
        assert np.array_equal(to_host_bits(a.decode(0)), to_host_bits(b.decode(0)))


@pytest.mark.parametrize("name,kw", [("C1", {}), ("C2", {"batch": 16}), ("C3", {}),
                                     ("C4", {"batch": 2})])
def test_fused_store_decode_matches_separate_and_oracle(name, kw):
    """nv_paged_decode_store against nv_store_kvcache + nv_paged_decode, step after step:
    identical pool bits; outputs within the tolerance of the separate path's (the fused
    kernel adds the decoded token to the softmax state after the cached ones, so its fp32
    sums round in another order) and of the oracle on sampled steps.  C3 runs all 50
    steps of the batch-256 workload: the launch configuration the benchmark times."""
    from paged_kv_cache_319_amd.harness import DeviceDecode, to_host_bits, to_host_f64
    banner(f"fused store+decode {name}")
    case = decode_config(name, **kw)
    tol = TOL[case.shape.dtype]
    a = DeviceDecode(case)
    b = DeviceDecode(case)
    orc = OracleDecode(case)
    n = len(case.steps)
    for t in range(n):
        oa = to_host_f64(a.step(t))
        ob = to_host_f64(b.step_fused(t))
        assert_close(ob, oa, tol, f"{name} fused vs separate, step {t}")
        if t in (0, n // 3, n - 1):
            assert_close(ob, orc.run_to(t), tol, f"{name} fused vs oracle, step {t}")
    torch.cuda.synchronize()
    for x, y in ((a.kc, b.kc), (a.vc, b.vc)):
        assert np.array_equal(to_host_bits(x).view(np.uint8), to_host_bits(y).view(np.uint8))


@pytest.mark.parametrize("name,tp,steps", [("C3", 2, 8), ("C3", 4, 8), ("C4", 2, 1)])
def test_fused_decode_head_shard(name, tp, steps):
    """One GPU's share of a head-parallel decode (num_q_heads / tp and num_kv_heads / tp,
    same lengths and tables): fused store + decode against the oracle."""
    from paged_kv_cache_319_amd.harness import DeviceDecode, to_host_f64
    banner(f"fused decode {name} head shard tp={tp}")
    case = decode_config(name, steps=steps, tp=tp)
    dev = DeviceDecode(case)
    orc = OracleDecode(case)
    for t in range(steps):
        got = to_host_f64(dev.step_fused(t))
        if t in (0, steps - 1):
            assert_close(got, orc.run_to(t), TOL["bf16"], f"{name} tp{tp} step {t}")


@pytest.mark.parametrize("bs", [16, 32, 64])
def test_fused_decode_block_size_variants(bs):
    """The batch-256 workload redrawn with block size bs (same lengths, pool bytes and
    shared 256-token prefixes; power-of-two sizes down to the tokens of one wave-pass take
    one table entry per pass): fused store + decode over 8 steps, against the oracle at the
    first and the last."""
    from paged_kv_cache_319_amd.harness import DeviceDecode, to_host_f64
    banner(f"fused decode C3 bs{bs}")
    case = decode_config("C3", steps=8, block_size=bs)
    dev = DeviceDecode(case)
    orc = OracleDecode(case)
    for t in range(8):
        got = to_host_f64(dev.step_fused(t))
        if t in (0, 7):
            assert_close(got, orc.run_to(t), TOL["bf16"], f"C3 bs{bs} step {t}")


@pytest.mark.parametrize("dtype,d,hq,hkv,batch", [("bf16", 64, 16, 2, 768), ("f32", 128, 8, 4, 400),
                                                  ("bf16", 128, 8, 1, 1600), ("bf16", 128, 32, 8, 200)])
def test_decode_whole_sequence_plans(dtype, d, hq, hkv, batch):
    """Batches with batch x KV heads >= 1536 run every sequence as one work item: two KV
    heads per workgroup when the KV-head count is even, one otherwise.  Two fused steps
    and one plain decode against the oracle, for other head dims, group sizes and dtypes
    than the batch-256 workload's."""
    from paged_kv_cache_319_amd.harness import DeviceDecode, to_host_f64
    banner(f"whole-sequence decode {dtype} d{d} hq{hq} hkv{hkv} batch{batch}")
    rng = np.random.default_rng(hq * 13 + d + batch)
    lengths = rng.integers(1, 300, endpoint=True, size=batch)
    bs = 16
    nb = int(sum(-(-(int(L) + 1) // bs) for L in lengths)) + 4
    sh = Shape(dtype, hq, hkv, d, bs, nb, 0.5 if dtype == "bf16" else 1.0)
    case = build_decode("whole", sh, lengths, seed=batch + d, steps=2)
    dev = DeviceDecode(case)
    orc = OracleDecode(case)
    assert dev.steps[0]["schedule"] is not None
    got0 = to_host_f64(dev.step_fused(0))
    assert_close(got0, orc.run_to(0), TOL[dtype], "whole-sequence fused step 0")
    dev.store(1)
    got1 = to_host_f64(dev.decode(1))
    assert_close(got1, orc.run_to(1), TOL[dtype], "whole-sequence decode step 1")


@pytest.mark.parametrize("dtype,d,hq,hkv,bs", [("bf16", 128, 32, 8, 16), ("f32", 64, 2, 1, 16),
                                               ("bf16", 64, 16, 2, 32)])
def test_fused_store_decode_edges(dtype, d, hq, hkv, bs):
    from paged_kv_cache_319_amd.harness import DeviceDecode, to_host_f64
    banner(f"fused edges {dtype} d{d} hq{hq} hkv{hkv} bs{bs}")
    nb = sum(-(-L // bs) for L in EDGE_LENGTHS) + 3
    sh = Shape(dtype, hq, hkv, d, bs, nb, 0.5 if dtype == "bf16" else 1.0)
    case = build_decode("edge", sh, EDGE_LENGTHS, seed=hq * 7 + d + bs)
    dev = DeviceDecode(case)
    got = to_host_f64(dev.step_fused(0))
    want = OracleDecode(case).run_to(0)
    assert_close(got, want, TOL[dtype], "fused edges")


@pytest.mark.parametrize("dtype,d,hq,hkv,bs", [("bf16", 128, 16, 8, 16), ("f32", 64, 2, 1, 256)])
def test_fused_store_skipped_slots(dtype, d, hq, hkv, bs):
    """slot_mapping[b] = -1 in the fused call: nothing is written for b and its decoded
    token is read from the cache, where the caller stored it beforehand.  Pool bits equal
    the separate store + decode's; outputs agree within the tolerance."""
    from paged_kv_cache_319_amd import nv_store_kvcache, nv_paged_decode_store
    from paged_kv_cache_319_amd.harness import DeviceDecode, to_host_bits, to_host_f64
    banner(f"fused store with skipped slots {dtype} d{d} bs{bs}")
    nb = sum(-(-L // bs) for L in EDGE_LENGTHS) + 3
    sh = Shape(dtype, hq, hkv, d, bs, nb, 0.5 if dtype == "bf16" else 1.0)
    case = build_decode("skip", sh, EDGE_LENGTHS, seed=hq + d + bs + 5)
    a, b = DeviceDecode(case), DeviceDecode(case)
    want = to_host_f64(a.step(0))
    st = b.steps[0]
    skip = torch.arange(0, len(EDGE_LENGTHS), 3, device="cuda")
    nv_store_kvcache(st["k"][skip].contiguous(), st["v"][skip].contiguous(), b.kc, b.vc,
                     st["slots"][skip].contiguous())
    slots = st["slots"].clone()
    slots[skip] = -1
    out = torch.empty_like(b.out)
    nv_paged_decode_store(out, st["q"], st["k"], st["v"], slots, b.kc, b.vc, st["tables"],
                          st["lens"], st["max_len"], case.shape.scale, workspace=b.workspace,
                          schedule=st["schedule"])
    torch.cuda.synchronize()
    assert_close(to_host_f64(out), want, TOL[dtype], "fused with skipped slots")
    for x, y in ((a.kc, b.kc), (a.vc, b.vc)):
        assert np.array_equal(to_host_bits(x).view(np.uint8), to_host_bits(y).view(np.uint8))


def test_graph_replay_matches_eager():
    """Fused store + decode steps captured as HIP graphs: every replay, interleaved with
    eager work and synchronisations, reproduces the eager outputs and pool bits."""
    from paged_kv_cache_319_amd.harness import DeviceDecode, to_host_bits
    banner("graph replay")
    case = decode_config("C3", batch=64, steps=4)
    eager = DeviceDecode(case)
    want = [to_host_bits(eager.step_fused(t)).copy() for t in range(4)]
    g = DeviceDecode(case)
    g.capture_graphs()
    other = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        for t in range(4):
            out = to_host_bits(g.replay(t)).copy()
            assert np.array_equal(out, want[t]), f"replay {rep} step {t}"
            other.mul_(1.0001)                      # eager work between replays
            torch.cuda.synchronize()
    for x, y in ((eager.kc, g.kc), (eager.vc, g.vc)):
        assert np.array_equal(to_host_bits(x).view(np.uint8), to_host_bits(y).view(np.uint8))


def test_multi_step_graph_matches_eager():
    """Six fused steps (split plan, shared workspace) captured into ONE HIP graph, each
    step writing its own output: every replay, with eager work and synchronisations
    between replays, reproduces the eager outputs of all six steps and the pool bits."""
    from paged_kv_cache_319_amd.harness import DeviceDecode, to_host_bits
    banner("multi-step graph replay")
    case = decode_config("C3", batch=64, steps=6)
    eager = DeviceDecode(case)
    want = [to_host_bits(eager.step_fused(t)).copy() for t in range(6)]
    g = DeviceDecode(case)
    g.capture_sequence(range(6))
    other = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        g.seq_graph.replay()
        torch.cuda.synchronize()
        for t in range(6):
            assert np.array_equal(to_host_bits(g.seq_outs[t]), want[t]), f"replay {rep} step {t}"
        other.mul_(1.0001)                          # eager work between replays
        torch.cuda.synchronize()
    for x, y in ((eager.kc, g.kc), (eager.vc, g.vc)):
        assert np.array_equal(to_host_bits(x).view(np.uint8), to_host_bits(y).view(np.uint8))


@pytest.mark.parametrize("scale", [-0.09, 0.0])
def test_decode_negative_and_zero_scale(scale):
    """Scores take the caller's scale as given: a negative one reverses the weighting and
    zero gives the plain mean of the visible V rows (the oracle's definition)."""
    from paged_kv_cache_319_amd import nv_paged_decode
    from paged_kv_cache_319_amd.harness import DeviceDecode, to_host_f64
    banner(f"decode scale={scale}")
    sh = Shape("f32", 8, 2, 128, 16, 300, 1.0)
    case = build_decode("scale", sh, np.array([1, 17, 300, 1500]), seed=31)
    dev = DeviceDecode(case)
    dev.store(0)
    s = dev.steps[0]
    out = torch.empty_like(dev.out)
    nv_paged_decode(out, s["q"], dev.kc, dev.vc, s["tables"], s["lens"], s["max_len"], scale,
                    workspace=dev.workspace, schedule=s["schedule"])
    want = OracleDecode(case).run_to(0, scale=scale)
    assert_close(to_host_f64(out), want, TOL["f32"], f"decode scale {scale}")


@pytest.mark.parametrize("dtype,hq,hkv,bs,batch,width", [
    ("bf16", 16, 8, 256, 16, 64), ("bf16", 32, 8, 256, 4, 128), ("f32", 2, 1, 16, 4, 64)])
def test_decode_loose_length_bound(dtype, hq, hkv, bs, batch, width):
    """max_context_len is only a host-side upper bound: with block tables wide enough for
    width * block_size tokens, a bound of that size (many times the longest context)
    changes the work split (more, shorter chunks; chunks past a sequence's end exit at
    once and the merge takes only the chunks that hold tokens) but not the result, which
    stays within tolerance of the oracle and of the tight bound's."""
    from paged_kv_cache_319_amd import nv_paged_decode_workspace_size
    from paged_kv_cache_319_amd.harness import DeviceDecode, to_host_f64
    banner(f"decode loose length bound {dtype} hq{hq} hkv{hkv} bs{bs} batch{batch}")
    rng = np.random.default_rng(batch * 7 + bs)
    lengths = rng.integers(1, 3 * bs, endpoint=True, size=batch)
    nb = int(sum(-(-(int(L) + 1) // bs) for L in lengths)) + 4
    sh = Shape(dtype, hq, hkv, 128 if dtype == "bf16" else 64, bs, nb,
               0.5 if dtype == "bf16" else 1.0)
    case = build_decode("loose", sh, lengths, seed=batch + bs, table_width=width)
    dev = DeviceDecode(case)
    tight = dev.steps[0]["max_len"]
    loose = width * bs
    need = nv_paged_decode_workspace_size(batch, hq, hkv, sh.head_dim, loose)
    assert need > 0
    dev.workspace = torch.empty(max(need, dev.workspace.numel()), dtype=torch.uint8,
                                device="cuda")
    dev.store(0)
    got_tight = to_host_f64(dev.decode(0)).copy()
    got = to_host_f64(dev.decode(0, max_len=loose))
    want = OracleDecode(case).run_to(0)
    assert_close(got, want, TOL[dtype], f"bound {loose} (longest {tight})")
    assert_close(got, got_tight, TOL[dtype], "loose vs tight bound")


def test_prepared_fused_call_matches_eager():
    """The prepared form of nv_paged_decode_store (arguments marshalled once) enqueues the
    same launch: outputs and pool bits identical to the eager calls, step after step, and
    a repeated prepared call of one step gives the same bits again."""
    from paged_kv_cache_319_amd.harness import DeviceDecode, to_host_bits
    banner("prepared fused call")
    case = decode_config("C3", batch=64, steps=3)
    a = DeviceDecode(case)
    b = DeviceDecode(case)
    calls = [b.prepare_fused(t) for t in range(3)]
    for t in range(3):
        x = to_host_bits(a.step_fused(t)).copy()
        calls[t]()
        assert np.array_equal(x, to_host_bits(b.out))
    calls[2]()
    assert np.array_equal(x, to_host_bits(b.out))
    for p, q in ((a.kc, b.kc), (a.vc, b.vc)):
        assert np.array_equal(to_host_bits(p).view(np.uint8), to_host_bits(q).view(np.uint8))


def test_decode_largest_batch():
    """65 535 sequences (the largest batch the launch grid takes) of 1-20 tokens, fp32,
    block size 16: store + decode and the fused step, against the oracle on every 97th
    sequence; every output finite."""
    from paged_kv_cache_319_amd.harness import DeviceDecode, to_host_f64
    banner("decode largest batch 65535")
    B = 65535
    rng = np.random.default_rng(7)
    lengths = rng.integers(1, 20, endpoint=True, size=B)
    bs = 16
    nb = int(sum(-(-(int(L) + 1) // bs) for L in lengths)) + 4
    sh = Shape("f32", 2, 1, 64, bs, nb, 1.0)
    case = build_decode("maxb", sh, lengths, seed=3, steps=1)
    seqs = np.arange(0, B, 97)
    want = OracleDecode(case).run_to(0, seqs=seqs)
    dev = DeviceDecode(case)
    dev.store(0)
    got = to_host_f64(dev.decode(0))
    assert np.all(np.isfinite(got))
    assert_close(got[seqs], want, TOL["f32"], "batch 65535 decode")
    dev2 = DeviceDecode(case)
    got2 = to_host_f64(dev2.step_fused(0))
    assert np.all(np.isfinite(got2))
    assert_close(got2[seqs], want, TOL["f32"], "batch 65535 fused step")


def test_prepared_call_keeps_its_cached_workspace():
    """A prepared fused call made without a workspace on a split plan (batch 8, 4 KV
    heads: sequences cut into chunks) writes its partials into the binding's cached
    buffer.  A later decode that needs more workspace on the same stream replaces the
    cached buffer, and new allocations overwrite the freed one; the prepared call still
    owns its buffer and matches the oracle."""
    from paged_kv_cache_319_amd import api
    from paged_kv_cache_319_amd.harness import DeviceDecode, to_host_f64
    banner("prepared call keeps its cached workspace")
    sh = Shape("bf16", 16, 4, 128, 256, 64, 0.5)
    case = build_decode("prep-ws", sh, [700, 1500, 300, 2000, 1024, 257, 1800, 999], seed=21)
    dev = DeviceDecode(case)
    s = dev.steps[0]
    api._ws_cache.clear()
    launch = api.prepare_paged_decode_store(dev.out, s["q"], s["k"], s["v"], s["slots"], dev.kc,
                                            dev.vc, s["tables"], s["lens"], s["max_len"],
                                            sh.scale)
    need = api.nv_paged_decode_workspace_size(8, 16, 4, 128, s["max_len"])
    assert need > 0
    first = next(iter(api._ws_cache.values()))
    # grow the cache: a bound of 64 blocks' tokens needs more chunks, more partials
    bigger = api.decode_workspace("cuda:0", 64 * need)
    assert bigger is not first
    del first
    junk = [torch.full((need // 4 + 64,), float("nan"), device="cuda") for _ in range(8)]
    launch()
    got = to_host_f64(dev.out)
    want = OracleDecode(case).run_to(0)
    assert_close(got, want, TOL["bf16"], "prepared call after the cache grew")
    del junk


def test_bench_launch_path_matches_oracle():
    """The launch path the benchmark times: the full batch-256 workload through one
    prepared fused call per step, cycled.  A second pass over the 50 steps (each step
    rewrites the same rows) gives outputs bit-identical to the first pass's, and steps
    0, 19 and 49 match the oracle."""
    from paged_kv_cache_319_amd.harness import DeviceDecode, to_host_bits, to_host_f64
    banner("bench launch path: prepared fused calls, two passes")
    case = decode_config("C3")
    dev = DeviceDecode(case, poison=True)
    n = len(case.steps)
    launches = [dev.prepare_fused(t) for t in range(n)]
    first = {}
    for t in range(n):
        launches[t]()
        if t in (0, 19, 49):
            first[t] = to_host_bits(dev.out).copy()
    orc = OracleDecode(case)
    for t in range(n):
        launches[t]()
        if t in first:
            assert np.array_equal(to_host_bits(dev.out), first[t]), f"pass 2 differs at step {t}"
            assert_close(to_host_f64(dev.out), orc.run_to(t), TOL["bf16"], f"C3 step {t}")
