"""pkdecode: batched decode attention over a paged, ragged KV cache on MI355X.

The computation runs in libpkdecode.so (hand-written HIP kernels for gfx950
behind a C ABI, ``include/pkdecode.h``); this package is its Python binding.
"""
from ._lib import LIB_PATH, PkdError, load  # noqa: F401
from .wrapper import (  # noqa: F401
    DEFAULT_WORKSPACE_BYTES,
    BatchDecodeWithPagedKVCacheWrapper,
    CascadeBatchDecodeWrapper,
    Plan,
    merge_state,
    plan_partition,
    stream_read,
)

__all__ = [
    "BatchDecodeWithPagedKVCacheWrapper",
    "CascadeBatchDecodeWrapper",
    "merge_state",
    "Plan",
    "PkdError",
    "plan_partition",
    "stream_read",
    "load",
    "LIB_PATH",
    "DEFAULT_WORKSPACE_BYTES",
]
