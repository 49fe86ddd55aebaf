"""The binding's cached scratch buffers (no GPU): one per (device, stream), grown on
demand, and a prepared call holds the buffer its arguments point into."""
import pytest
import torch

from paged_kv_cache_319_amd import api


@pytest.fixture
def host_buffers(monkeypatch):
    """Stand-ins: streams are plain integers and 'device' buffers are host tensors."""
    real_empty = torch.empty
    monkeypatch.setattr(api, "_stream", lambda stream, device: 7 if stream is None else int(stream))
    monkeypatch.setattr(api.torch, "empty",
                        lambda n, dtype=None, device=None: real_empty(n, dtype=dtype))
    monkeypatch.setattr(api, "_ws_cache", {})
    return api


def test_one_buffer_per_device_and_stream(host_buffers):
    a = api.decode_workspace("cuda:0", 1024, stream=11)
    b = api.decode_workspace("cuda:0", 1024, stream=12)
    c = api.decode_workspace("cuda:1", 1024, stream=11)
    assert len({id(a), id(b), id(c)}) == 3                       # never shared across streams
    assert api.decode_workspace("cuda:0", 512, stream=11) is a   # reused on its stream
    assert api.decode_workspace("cuda:0", 1024) is api.decode_workspace("cuda:0", 1000, 7)
    assert api.decode_workspace("cuda:0", 0, stream=11) is None


def test_growth_replaces_only_that_streams_buffer(host_buffers):
    a = api.decode_workspace("cuda:0", 1024, stream=11)
    b = api.decode_workspace("cuda:0", 1024, stream=12)
    big = api.decode_workspace("cuda:0", 4096, stream=11)
    assert big is not a and big.numel() >= 4096
    assert api.decode_workspace("cuda:0", 100, stream=11) is big
    assert api.decode_workspace("cuda:0", 100, stream=12) is b


def test_prepared_fused_call_keeps_the_cached_workspace(host_buffers, monkeypatch):
    """prepare_paged_decode_store without a workspace: the callable's kept references
    include the cached buffer it was prepared with, so a later call that grows the cache
    cannot free memory the prepared launch still writes."""
    sentinel = api.decode_workspace("cuda:0", 64, stream=3)

    def fake_call(*a, **kw):
        return (lambda *x: api.NV_OK), (), sentinel
    monkeypatch.setattr(api, "_decode_store_call", fake_call)
    monkeypatch.setattr(api, "_prepared", lambda name, fn, args, keep: keep)
    keep = api.prepare_paged_decode_store(*([None] * 11))
    assert any(k is sentinel for k in keep)
    grown = api.decode_workspace("cuda:0", 1 << 20, stream=3)
    assert grown is not sentinel and any(k is sentinel for k in keep)
