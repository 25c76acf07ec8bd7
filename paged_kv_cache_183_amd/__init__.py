"""Paged KV-cache hot path for AMD MI355X (gfx950).

The work happens in ``libvllm_paged.so`` (hand-written HIP kernels behind a C
ABI declared in ``include/vllm_paged.h``); this package only builds it
(``build``) and binds it (``binding``).  Importing the package loads the
library and raises ImportError if it has not been built.
"""
from .binding import (  # noqa: F401
    BLOCK_SIZE,
    VllmError,
    vllm_abi_version,
    vllm_last_error,
    vllm_paged_attn_decode,
    vllm_paged_attn_decode_noalloc,
    vllm_paged_attn_decode_shared_prefix,
    vllm_paged_attn_prefill,
    vllm_paged_attn_shared_prefix_workspace_size,
    vllm_paged_attn_prefill_workspace_size,
    vllm_paged_attn_workspace_size,
    vllm_block_manager_init,
    vllm_block_manager_release,
    vllm_block_manager_schedule,
    vllm_block_manager_state_layout,
    vllm_block_manager_state_size,
    vllm_block_manager_workspace_size,
    vllm_paged_attn_decode_append,
    vllm_paged_cache_write,
    vllm_paged_chunked_local_plan,
    vllm_paged_chunked_local_virtual_count,
    vllm_paged_read_pages,
    vllm_paged_recycle_pages,
)
