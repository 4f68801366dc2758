"""CPU oracle of the block manager and the block copies (test infrastructure only).

A plain statement of how sequences get, share, copy and return pool blocks. Only
the tests, the smoke check and the benchmark's CPU-baseline leg may import it; it
shares no code with the library.

What the pages fix and what is read into them:

* The free list starts as ``0 .. num_blocks-1``; blocks are taken from its front and
  a sequence of n tokens holds ceil(n / block_size) blocks (page "vLLM 部署深度指南",
  section "PagedAttention 原理", code listing of the simplified KV-cache class).
* A sequence takes a new block only when its last block is full (page "vLLM GitHub
  项目 …", section 二, item 1).
* Sequences that share a prefix (parallel sampling, beam search) point their tables
  at the same physical blocks (same section, item 4): ``fork`` gives the child the
  parent's blocks and counts the references.

Readings (the pages are silent; the plainest reading that the rest supports):

* A token appended to a sequence whose last block is shared and partly filled must not
  change what the other sequences see, so that block is first copied to a fresh block
  (copy-on-write); the copy is reported as a (source, destination) pair for the device.
* A freed sequence drops one reference from each of its blocks, in table order; a
  block whose count reaches zero goes to the back of the free list.
* ``allocate`` and ``append_token`` either succeed or raise ``KVCacheExhausted`` with
  nothing taken. (The listing's simplified loop keeps the blocks it took before running
  dry; ``oracle.BlockAllocator`` reproduces that listing as printed.)
* ``usage`` is the fraction of pool blocks in use, the ``gpu_cache_usage_perc`` gauge of
  the monitoring table on page "vLLM 部署深度指南"; ``slot_utilisation`` is the fraction
  of slots in used blocks that hold a token (the "KV Cache 利用率" row of the same page's
  comparison table).
"""

from __future__ import annotations

import numpy as np

from .paged_attention import KVCacheExhausted, blocks_needed


class BlockManager:
    """Tables, lengths and reference counts of the sequences in one block pool."""

    def __init__(self, num_blocks: int, block_size: int = 16):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.free_blocks = list(range(self.num_blocks))
        self.refs = [0] * self.num_blocks
        self.tables = {}
        self.lengths = {}

    def _take(self) -> int:
        block = self.free_blocks.pop(0)
        self.refs[block] = 1
        return block

    def allocate(self, seq_id, num_tokens: int):
        """A new sequence holding ``num_tokens`` tokens; returns its table."""
        if seq_id in self.tables or num_tokens < 0:
            raise ValueError("sequence exists or negative length")
        need = blocks_needed(num_tokens, self.block_size)
        if need > len(self.free_blocks):
            raise KVCacheExhausted("KV cache exhausted")
        self.tables[seq_id] = [self._take() for _ in range(need)]
        self.lengths[seq_id] = int(num_tokens)
        return list(self.tables[seq_id])

    def append_token(self, seq_id):
        """Reserve the slot of the sequence's next token.

        Returns ``(slot, copy)``: ``copy`` is ``(src_block, dst_block)`` when the last
        block was shared and partly filled (copy-on-write), else ``None``.
        """
        if seq_id not in self.tables:
            raise ValueError("unknown sequence")
        table = self.tables[seq_id]
        pos = self.lengths[seq_id]
        copy = None
        if pos == len(table) * self.block_size:
            if not self.free_blocks:
                raise KVCacheExhausted("KV cache exhausted")
            table.append(self._take())
        elif self.refs[table[-1]] > 1:
            if not self.free_blocks:
                raise KVCacheExhausted("KV cache exhausted")
            old = table[-1]
            new = self._take()
            self.refs[old] -= 1
            table[-1] = new
            copy = (old, new)
        self.lengths[seq_id] = pos + 1
        block = table[pos // self.block_size]
        return block * self.block_size + pos % self.block_size, copy

    def fork(self, parent, child):
        """``child`` starts as a copy of ``parent`` sharing every block."""
        if child in self.tables or parent not in self.tables:
            raise ValueError("child exists or parent unknown")
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        for b in self.tables[child]:
            self.refs[b] += 1
        return list(self.tables[child])

    def free(self, seq_id):
        if seq_id not in self.tables:
            raise ValueError("unknown sequence")
        for b in self.tables.pop(seq_id):
            self.refs[b] -= 1
            if self.refs[b] == 0:
                self.free_blocks.append(b)
        del self.lengths[seq_id]

    def usage(self) -> float:
        return 1.0 - len(self.free_blocks) / self.num_blocks

    def slot_utilisation(self) -> float:
        filled = {}
        for s, table in self.tables.items():
            n = self.lengths[s]
            for j, b in enumerate(table):
                filled[b] = max(filled.get(b, 0), min(self.block_size, n - j * self.block_size))
        used = self.num_blocks - len(self.free_blocks)
        return sum(filled.values()) / (used * self.block_size) if used else 0.0

    def block_table_rows(self, seq_ids, max_blocks: int, pad: int):
        """Padded ``[len(seq_ids), max_blocks]`` int32 tables and int32 lengths."""
        tables = np.full((len(seq_ids), max_blocks), pad, dtype=np.int32)
        lens = np.zeros(len(seq_ids), dtype=np.int32)
        for i, s in enumerate(seq_ids):
            row = self.tables[s]
            if len(row) > max_blocks:
                raise ValueError("table longer than max_blocks")
            tables[i, : len(row)] = row
            lens[i] = self.lengths[s]
        return tables, lens


# ---------------------------------------------------------------------------------------
# block copies on the pool
# ---------------------------------------------------------------------------------------

def copy_blocks(pool: np.ndarray, pairs) -> np.ndarray:
    """Copy of ``pool`` after ``pool[dst] = pool[src]`` for each (src, dst) pair in order.

    The device half of copy-on-write above: the destination block starts as the shared
    block's contents before the sequence's own token is written into it.
    """
    out = pool.copy()
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        out[dst] = out[src]
    return out


def move_blocks(dst: np.ndarray, src: np.ndarray, pairs) -> np.ndarray:
    """Copy of ``dst`` after ``dst[d] = src[s]`` for each (s, d) pair: blocks swapped out
    of the pool to host memory or back in (the ``--swap-space`` CPU area in the flag table
    of page "vLLM 部署深度指南")."""
    out = dst.copy()
    for s, d in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        out[d] = src[s]
    return out
