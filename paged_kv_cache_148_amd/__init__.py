"""paged_kv_cache_148_amd -- PagedAttention decode for AMD MI355X (gfx950).

The GPU work runs in libpkv.so (hand-written HIP kernels behind the C ABI of
include/pkv.h); this package holds its Python binding and the host-side block
manager that builds block tables, slot mappings and copy-on-write pairs.
"""
from .binding import (PKV_DTYPE_BF16, PKV_DTYPE_F32, PKV_PATH_MFMA, PKV_PATH_NONE, PKV_PATH_VECTOR, PkvError,
                      attention_path, attention_workspace_size, copy_blocks, lib, paged_attention_decode,
                      paged_kv_write, status_string)
from .block_manager import BlockManager, Sequence

__all__ = [
    "paged_kv_write", "paged_attention_decode", "copy_blocks", "attention_workspace_size", "attention_path",
    "status_string", "lib", "PkvError", "BlockManager", "Sequence",
    "PKV_DTYPE_F32", "PKV_DTYPE_BF16", "PKV_PATH_NONE", "PKV_PATH_VECTOR", "PKV_PATH_MFMA",
]
