"""Paged KV-cache attention for MI355X (gfx950): a C-ABI HIP library and its Python binding.

The library (``libpagedkv.so``, declared in ``include/pagedkv.h``) holds the kernels:
``pa_kv_append`` (scatter of new tokens into pool slots), ``pa_decode`` (split-context
paged decode with a log-sum-exp merge), ``pa_prefill_chunk`` (causal chunked prefill on
the matrix cores), ``pa_gather_kv``, the pool-layout helpers, step capture into HIP graphs
(``StepGraph``) and the host block manager (``BlockManager``). The functions below
only marshal torch tensors into the C calls.
"""

from ._lib import (  # noqa: F401
    LIB_PATH,
    SIGNATURES,
    BlockManager,
    KVCacheExhausted,
    PagedKVError,
    StepGraph,
    load,
    pa_abi_version,
    pa_block_bytes,
    pa_copy_blocks,
    pa_copy_blocks_fp8,
    pa_blocks_for_len,
    pa_decode,
    pa_decode_fp8,
    pa_decode_noalloc,
    pa_decode_shared_prefix,
    pa_decode_shared_prefix_fp8,
    pa_decode_shared_prefix_workspace_bytes,
    pa_decode_workspace_bytes,
    pa_gather_kv,
    pa_kv_append,
    pa_kv_append_fp8,
    pa_kv_elem_offset,
    pa_move_blocks,
    pa_num_blocks_fit,
    pa_num_partitions,
    pa_decode_default_partition_size,
    pa_pool_bytes,
    pa_prefill_chunk,
    pa_prefill_chunk_fp8,
    pa_prefill_workspace_bytes,
    pa_slot,
    pa_stream_read,
    pa_stream_read_sink_len,
    PA_DECODE_KV_STREAM,
    PA_DECODE_NOALLOC_SCRATCH_BYTES,
    PA_OK,
    PA_ERR_INVALID,
    PA_ERR_UNSUPPORTED,
    PA_ERR_WORKSPACE,
    PA_ERR_HIP,
    PA_ERR_EXHAUSTED,
)
