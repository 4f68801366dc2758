"""Seeded synthetic inputs for paged KV-cache attention.

Shared by the CPU oracle's tests, the GPU parity tests and the benchmark. It
draws values, assigns physical blocks to sequences and lays the drawn tokens
into a block pool. It holds no attention arithmetic.
"""

from .synth import (  # noqa: F401
    POISON_F16,
    PagedInputs,
    build,
    tiny_decode,
    tiny_decode_full_append,
    decode_256seq,
    long_context_32k,
    shared_prompt_groups,
    mixed_prefill_decode,
    long_prompt_prefill,
    decode_case,
    mixed_case,
    prefix_shared_case,
    repermute,
    unshare_prefix,
    WORKLOADS,
)
