"""GPU: cache blocks that sit more than 2**32 elements into their pool.

A KV pool on a 288 GB part holds far more than 4 GiB, so every cache address is a 64-bit
offset.  Each test runs a workload on its usual small pool, then again with every block id
moved up by a shift that puts the used blocks past 2**32 elements (and 2**32 bytes) of a
large pool whose other blocks hold NaN.  Store, decode, fused store+decode and prefill must
give the same bits in both placements: a read from the wrong place pulls in NaN, a write to
the wrong place leaves the moved blocks stale and NaN blocks overwritten.  The small-pool
run is checked against the oracle, as in the other parity tests."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from workloads import decode_config, build_decode, build_prefill, Shape
from oracle_runs import OracleDecode, oracle_prefill
from gpu_common import TOL, assert_close, banner


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from paged_kv_cache_319_amd import load_library
    load_library()
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    yield
    torch.cuda.empty_cache()


def _shift(shape) -> int:
    """Block-id shift that places block 0 of the moved range past 2**32 elements."""
    per_block = shape.block_size * shape.num_kv_heads * shape.head_dim
    return (1 << 32) // per_block + 3


def _moved_pools(kc, vc, shift):
    """Large NaN pools holding a copy of kc / vc at block ids shift .. shift + nb - 1."""
    size = (shift + kc.shape[0],) + tuple(kc.shape[1:])
    kb = torch.full(size, float("nan"), dtype=kc.dtype, device=kc.device)
    vb = torch.full(size, float("nan"), dtype=vc.dtype, device=vc.device)
    kb[shift:] = kc
    vb[shift:] = vc
    return kb, vb


def _moved_tables(bt: np.ndarray, shift: int) -> np.ndarray:
    return np.where(bt >= 0, bt + shift, -1).astype(np.int32)


def _moved_slots(slots: torch.Tensor, shift: int, block_size: int) -> torch.Tensor:
    return torch.where(slots >= 0, slots + shift * block_size, slots)


def _below_shift_untouched(pool: torch.Tensor, shift: int):
    """Every block under the moved range still holds NaN (checked in slices, so the
    temporary mask stays small)."""
    step = max(1, (1 << 28) // pool[0].numel())
    for i in range(0, shift, step):
        assert bool(torch.isnan(pool[i:min(i + step, shift)]).all()), f"block range {i}.. written"


def _same_moved_blocks(big: torch.Tensor, small: torch.Tensor, shift: int):
    from paged_kv_cache_319_amd.harness import to_host_bits
    assert np.array_equal(to_host_bits(big[shift:]).view(np.uint8),
                          to_host_bits(small).view(np.uint8))


DECODE_CASES = [
    # the prefix-sharing workload, shrunk: bf16, 256-token blocks
    ("C3", lambda: decode_config("C3", batch=24, steps=1, num_blocks=240)),
    # fp32 with 48-token blocks (no power of two), lengths across chunk edges
    ("f32 bs48", lambda: build_decode(
        "edge", Shape("f32", 8, 2, 64, 48, 60, 1.0), [1, 47, 48, 49, 300, 511, 1025],
        seed=48)),
]


@pytest.mark.parametrize("name,make", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_store_and_decode_past_4g_elements(name, make):
    from paged_kv_cache_319_amd import nv_store_kvcache, nv_paged_decode, nv_paged_decode_store
    from paged_kv_cache_319_amd.harness import DeviceDecode, to_host_bits, to_host_f64, i32
    banner(f"large pool decode {name}")
    case = make()
    sh = case.shape
    shift = _shift(sh)
    dev = DeviceDecode(case)
    kb, vb = _moved_pools(dev.kc, dev.vc, shift)        # pre-store contents, moved
    kf, vf = dev.kc.clone(), dev.vc.clone()             # pre-store contents, in place
    s = dev.steps[0]
    tables = i32(_moved_tables(case.steps[0].block_tables, shift), "cuda")
    slots = _moved_slots(s["slots"], shift, sh.block_size)
    want = OracleDecode(case).run_to(0)

    # fused store + decode: small pool, then the large one
    fused_small, fused_big = torch.empty_like(dev.out), torch.empty_like(dev.out)
    nv_paged_decode_store(fused_small, s["q"], s["k"], s["v"], s["slots"], kf, vf, s["tables"],
                          s["lens"], s["max_len"], sh.scale, workspace=dev.workspace,
                          schedule=s["schedule"])
    nv_paged_decode_store(fused_big, s["q"], s["k"], s["v"], slots, kb, vb, tables, s["lens"],
                          s["max_len"], sh.scale, workspace=dev.workspace,
                          schedule=s["schedule"])
    torch.cuda.synchronize()
    assert_close(to_host_f64(fused_small), want, TOL[sh.dtype], f"{name} fused")
    assert np.array_equal(to_host_bits(fused_big), to_host_bits(fused_small))
    _same_moved_blocks(kb, kf, shift)
    _same_moved_blocks(vb, vf, shift)
    del kf, vf

    # plain store + decode: small pool, then the large one (its rows already hold the
    # stored values, so the store must leave them as they are)
    dev.store(0)
    base = to_host_bits(dev.decode(0)).copy()
    torch.cuda.synchronize()
    assert_close(to_host_f64(dev.out), want, TOL[sh.dtype], name)
    nv_store_kvcache(s["k"], s["v"], kb, vb, slots)
    out = torch.empty_like(dev.out)
    nv_paged_decode(out, s["q"], kb, vb, tables, s["lens"], s["max_len"], sh.scale,
                    workspace=dev.workspace, schedule=s["schedule"])
    assert np.array_equal(to_host_bits(out), base)
    _same_moved_blocks(kb, dev.kc, shift)
    _same_moved_blocks(vb, dev.vc, shift)
    _below_shift_untouched(kb, shift)
    _below_shift_untouched(vb, shift)
    del kb, vb
    torch.cuda.empty_cache()


PREFILL_CASES = [
    # bf16, 256-token blocks (block lookups by shift)
    ("bf16 bs256", Shape("bf16", 32, 8, 128, 256, 12, 0.5), [300, 1, 700], [512, 0, 256]),
    # fp32, 48-token blocks (block lookups by division)
    ("f32 bs48", Shape("f32", 8, 2, 64, 48, 40, 1.0), [130, 33, 400], [96, 7, 300]),
]


@pytest.mark.parametrize("name,sh,new,cached", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_store_and_prefill_past_4g_elements(name, sh, new, cached):
    from paged_kv_cache_319_amd import nv_store_kvcache, nv_paged_prefill
    from paged_kv_cache_319_amd.harness import DevicePrefill, to_host_bits, to_host_f64, i32
    banner(f"large pool prefill {name}")
    case = build_prefill("large", sh, new, cached, seed=sh.block_size + sh.head_dim,
                         pad_to=128, causal=True)
    shift = _shift(sh)
    dev = DevicePrefill(case)
    kb, vb = _moved_pools(dev.kc, dev.vc, shift)        # prefix rows stored, new rows not yet
    dev.store()
    base = to_host_bits(dev.attend()).copy()
    torch.cuda.synchronize()
    want, _, _, _ = oracle_prefill(case)
    assert_close(to_host_f64(dev.out), want, TOL[sh.dtype], name)

    nv_store_kvcache(dev.k, dev.v, kb, vb, _moved_slots(dev.slots, shift, sh.block_size))
    _same_moved_blocks(kb, dev.kc, shift)
    _same_moved_blocks(vb, dev.vc, shift)
    out = torch.empty_like(dev.out)
    nv_paged_prefill(out, dev.q, kb, vb, dev.cu_q, dev.cu_k, dev.max_q, dev.max_k,
                     i32(_moved_tables(case.block_tables, shift), "cuda"), sh.scale, True,
                     tile_schedule=dev.tiles)
    assert np.array_equal(to_host_bits(out), base)
    _below_shift_untouched(kb, shift)
    _below_shift_untouched(vb, shift)
    del kb, vb
    torch.cuda.empty_cache()
