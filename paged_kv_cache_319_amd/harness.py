"""Device-side replay of generated workloads through the C ABI.

Used by the GPU tests, the benchmark and the smoke check.  Slots and cu_seqlens
come from the library's own host builders (nv_prepare_decode / nv_prepare_prefill),
cache rows are written by nv_store_kvcache, and attention runs in the HIP kernels.
"""
from __future__ import annotations

import numpy as np
import torch

from .api import (nv_prepare_decode, nv_prepare_prefill, nv_store_kvcache, nv_paged_decode,
                  nv_paged_decode_store, nv_paged_prefill, nv_paged_prefill_tile_rows,
                  nv_paged_decode_workspace_size, NV_BF16, NV_F32)

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}
NV_DTYPE = {"f32": NV_F32, "bf16": NV_BF16}


def to_device(arr: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Storage-form array (float32, or bf16 bits as uint16) -> device tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> storage-form numpy (float32, or bf16 bits as uint16)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def to_host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def i32(a, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def new_pools(shape, device, poison: bool = True):
    dt = TORCH_DTYPE[shape.dtype]
    size = (shape.num_blocks, shape.block_size, shape.num_kv_heads, shape.head_dim)
    kc = torch.full(size, float("nan") if poison else 0.0, dtype=dt, device=device)
    vc = torch.full(size, float("nan") if poison else 0.0, dtype=dt, device=device)
    return kc, vc


def store_fill(shape, fill, kc, vc):
    """Write a Fill's rows through the library's prefill metadata builder and store kernel."""
    if fill.num_rows == 0:
        return
    dev = kc.device
    _, _, _, _, slots = nv_prepare_prefill(fill.block_tables, fill.start, fill.end - fill.start,
                                           shape.block_size, shape.num_blocks, 1)
    nv_store_kvcache(to_device(fill.k, shape.dtype, dev), to_device(fill.v, shape.dtype, dev),
                     kc, vc, i32(slots, dev))


class DeviceDecode:
    """A decode workload resident on the device: pools (fill rows stored) and, per step,
    q / new rows / tables / lengths / slots as device tensors."""

    def __init__(self, case, device="cuda:0", poison: bool = True, scheduled: bool = True):
        sh = case.shape
        self.case = case
        self.device = torch.device(device)
        self.kc, self.vc = new_pools(sh, self.device, poison)
        store_fill(sh, case.fill, self.kc, self.vc)
        self.steps = []
        max_len = 0
        for st in case.steps:
            slots, sched, mx = nv_prepare_decode(st.block_tables, st.context_lens,
                                                 sh.block_size, sh.num_blocks, with_schedule=True)
            max_len = max(max_len, mx)
            self.steps.append(dict(
                q=to_device(st.q, sh.dtype, self.device),
                k=to_device(st.k_new, sh.dtype, self.device),
                v=to_device(st.v_new, sh.dtype, self.device),
                tables=i32(st.block_tables, self.device),
                lens=i32(st.context_lens, self.device),
                slots=i32(slots, self.device),
                schedule=i32(sched, self.device) if scheduled else None, max_len=mx))
        B = case.batch
        self.out = torch.empty((B, sh.num_q_heads, sh.head_dim), dtype=TORCH_DTYPE[sh.dtype],
                               device=self.device)
        ws = nv_paged_decode_workspace_size(B, sh.num_q_heads, sh.num_kv_heads, sh.head_dim,
                                            max(max_len, 1))
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=self.device)

    def store(self, t: int):
        s = self.steps[t]
        nv_store_kvcache(s["k"], s["v"], self.kc, self.vc, s["slots"])

    def decode(self, t: int, out=None, max_len=None):
        s = self.steps[t]
        out = self.out if out is None else out
        nv_paged_decode(out, s["q"], self.kc, self.vc, s["tables"], s["lens"],
                        s["max_len"] if max_len is None else max_len, self.case.shape.scale,
                        workspace=self.workspace, schedule=s["schedule"])
        return out

    def step(self, t: int):
        self.store(t)
        return self.decode(t)

    def step_fused(self, t: int, out=None):
        """Store + decode of step t through the fused entry point."""
        s = self.steps[t]
        out = self.out if out is None else out
        nv_paged_decode_store(out, s["q"], s["k"], s["v"], s["slots"], self.kc, self.vc,
                              s["tables"], s["lens"], s["max_len"], self.case.shape.scale,
                              workspace=self.workspace, schedule=s["schedule"])
        return out

    def prepare_store(self, t: int):
        """A callable that enqueues step t's store with the arguments marshalled once."""
        from .api import prepare_store_kvcache
        s = self.steps[t]
        return prepare_store_kvcache(s["k"], s["v"], self.kc, self.vc, s["slots"])

    def prepare_fused(self, t: int):
        """A callable that enqueues step t's fused store + decode with the arguments
        marshalled once (nv_paged_decode_store's prepared form)."""
        from .api import prepare_paged_decode_store
        s = self.steps[t]
        return prepare_paged_decode_store(self.out, s["q"], s["k"], s["v"], s["slots"], self.kc,
                                          self.vc, s["tables"], s["lens"], s["max_len"],
                                          self.case.shape.scale, workspace=self.workspace,
                                          schedule=s["schedule"])

    def capture_graphs(self, steps=None):
        """Capture one HIP graph per step holding the fused store + decode launch(es).
        All buffers are pre-allocated, so the graphs record kernel nodes only."""
        steps = range(len(self.steps)) if steps is None else steps
        self.graphs = {}
        for t in steps:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.step_fused(t)
            self.graphs[t] = g
        torch.cuda.synchronize()
        return self.graphs

    def replay(self, t: int):
        self.graphs[t].replay()
        return self.out

    def capture_sequence(self, steps):
        """Capture the fused store + decode of several steps, in order, into ONE HIP graph
        (one replay runs them all, so the per-launch cost of a graph is paid once);
        step t writes its own output buffer ``self.seq_outs[t]``."""
        sh = self.case.shape
        self.seq_outs = {t: torch.empty((self.case.batch, sh.num_q_heads, sh.head_dim),
                                        dtype=TORCH_DTYPE[sh.dtype], device=self.device)
                         for t in steps}
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for t in steps:
                self.step_fused(t, out=self.seq_outs[t])
        torch.cuda.synchronize()
        self.seq_graph = g
        return g


class DevicePrefill:
    def __init__(self, case, device="cuda:0", poison: bool = True, scheduled: bool = True):
        sh = case.shape
        self.case = case
        self.device = torch.device(device)
        self.kc, self.vc = new_pools(sh, self.device, poison)
        store_fill(sh, case.fill, self.kc, self.vc)
        rows = nv_paged_prefill_tile_rows(sh.num_q_heads, sh.num_kv_heads)
        cu_q, cu_k, mq, mk, slots, tiles = nv_prepare_prefill(
            case.block_tables, case.num_cached, case.num_new, sh.block_size, sh.num_blocks,
            case.pad_to, tile_rows=rows)
        self.meta = (cu_q, cu_k, mq, mk, slots)
        self.tiles = i32(tiles, self.device) if scheduled and len(tiles) else None
        self.cu_q, self.cu_k = i32(cu_q, self.device), i32(cu_k, self.device)
        self.max_q, self.max_k = mq, mk
        self.slots = i32(slots, self.device)
        self.tables = i32(case.block_tables, self.device)
        self.q = to_device(case.q, sh.dtype, self.device)
        self.k = to_device(case.k_new, sh.dtype, self.device)
        self.v = to_device(case.v_new, sh.dtype, self.device)
        self.out = torch.empty_like(self.q)

    def store(self):
        nv_store_kvcache(self.k, self.v, self.kc, self.vc, self.slots)

    def prepare_store(self):
        """A callable that enqueues this workload's store with the arguments marshalled once."""
        from .api import prepare_store_kvcache
        return prepare_store_kvcache(self.k, self.v, self.kc, self.vc, self.slots)

    def attend(self, out=None):
        out = self.out if out is None else out
        nv_paged_prefill(out, self.q, self.kc, self.vc, self.cu_q, self.cu_k, self.max_q,
                         self.max_k, self.tables, self.case.shape.scale, self.case.causal,
                         tile_schedule=self.tiles)
        return out

    def step(self):
        self.store()
        return self.attend()


class DeviceSampler:
    """A sampler workload resident on the device: logits, temperatures, Gumbel noise."""

    def __init__(self, case, device="cuda:0"):
        from .api import nv_sample_workspace_size
        self.case = case
        self.logits = to_device(case.logits, case.dtype, device)
        self.temps = torch.from_numpy(np.ascontiguousarray(case.temperatures,
                                                           dtype=np.float32)).to(device)
        self.gumbel = torch.from_numpy(np.ascontiguousarray(case.gumbel, dtype=np.float32)).to(device)
        self.tokens = torch.empty(case.batch, dtype=torch.int32, device=device)
        n = nv_sample_workspace_size(case.batch, case.vocab)
        self.ws = torch.empty(max(n, 1), dtype=torch.uint8, device=device)

    def sample(self):
        from .api import nv_sample
        nv_sample(self.tokens, self.logits, self.temps, self.gumbel, workspace=self.ws)
        return self.tokens
