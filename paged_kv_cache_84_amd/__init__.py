"""Paged KV cache hot path for AMD Instinct MI355X (gfx950).

A thin Python binding over the C ABI of ``libpagedkv.so`` (declared in
``include/pagedkv.h``).  The functions here have the same names as the
library's entry points and only marshal arguments: every step of the path
runs in the library's HIP kernels.  PyTorch supplies device memory and the
current stream.

The library is loaded on first use; if it is missing or does not load, every
call raises ``LibraryNotBuilt`` -- there is no fallback implementation.
"""

from . import blocks, step  # noqa: F401
from ._binding import (  # noqa: F401
    BLOCK_SIZE,
    LibraryNotBuilt,
    PagedKVError,
    compute_slot_mapping,
    copy_blocks,
    decode_num_chunks,
    decode_workspace_size,
    kv_bytes_per_token,
    library,
    library_path,
    measure_hbm_read,
    measure_mfma_bf16,
    measure_mfma_valu,
    varlen_workspace_size,
    paged_attention_decode,
    paged_attention_decode_append,
    paged_attention_decode_int4,
    paged_attention_decode_noalloc,
    paged_attention_decode_nvfp4,
    paged_attention_decode_sliding,
    paged_attention_prefill_chunk,
    paged_attention_varlen,
    reshape_and_cache,
    reshape_and_cache_from_schedule,
    reshape_and_cache_int4,
    reshape_and_cache_nvfp4,
    swap_blocks,
)
