"""CPU oracle for paged KV-cache attention: test infrastructure, not product code.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. It is plain fp64 NumPy, shares no code with the HIP library and
never imports it.
"""

from .block_manager import BlockManager, copy_blocks, move_blocks  # noqa: F401
from .paged_attention import (  # noqa: F401
    BlockAllocator,
    KVCacheExhausted,
    blocks_needed,
    decode,
    decode_partitioned,
    decode_rows,
    expected_slots,
    gather_kv,
    kv_append,
    kv_head_of,
    prefill_chunk,
    slot_of,
    softmax_attention,
)
