"""Paged-KV attention for AMD MI355X (gfx950): thin Python binding of ``libpagedattn.so``.

The binding only marshals arguments (tensor data pointers, strides, the current
HIP stream) into the C ABI declared in ``include/pagedattn.h``; every step of the
computation runs in the library's HIP kernels.  PyTorch supplies device memory
and streams.  If the library is missing the calls raise: there is no fallback.
"""
from .ops import (  # noqa: F401
    AttnError,
    PreparedCall,
    CacheDesc,
    cache_write,
    decode_splitkv,
    decode_splitkv_append,
    decode_splitkv_noalloc,
    load_library,
    merge_lse,
    new_workspace,
    prefill_causal,
    splitkv_workspace_bytes,
    verify,
    library_path,
)
