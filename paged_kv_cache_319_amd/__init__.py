"""nvpaged: paged KV-cache attention for AMD Instinct MI355X (gfx950).

Python face of libnvpaged.so (see include/nvpaged.h).  The entry points keep
the C names; they marshal torch device tensors / numpy host arrays into the C
ABI and raise NvError on a non-OK status.  The library must be built
(python -m paged_kv_cache_319_amd.build); there is no fallback implementation.
"""
from .api import (  # noqa: F401
    NV_OK, NV_F32, NV_BF16, NvError,
    nv_status_string, nv_store_kvcache, prepare_store_kvcache, nv_paged_decode_workspace_size, nv_paged_decode,
    nv_paged_decode_store, prepare_paged_decode_store, nv_paged_decode_store_noalloc,
    nv_paged_prefill, nv_paged_prefill_tile_rows, nv_prepare_decode, nv_prepare_prefill,
    decode_workspace, nv_sample_workspace_size, nv_sample, nv_set_check_mode, nv_check_message,
)
from .blocks import BlockManager, nv_bm_xxh64  # noqa: F401
from ._native import LIB_PATH, load as load_library  # noqa: F401
