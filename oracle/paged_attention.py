"""CPU oracle for paged KV-cache attention (test infrastructure only).

This module is a plain, slow, fp64 statement of what the paged attention path
computes. Only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import it; the product path never does. It shares no code with the HIP
library and imports nothing from it.

What the pages fix and what is read into them:

* The pool is ``[num_blocks, block_size, 2, num_heads, head_size]`` fp16, one
  per layer, and each sequence owns a list of physical block indices (page
  "vLLM 部署深度指南", section "PagedAttention 原理", code listing of the
  simplified KV-cache class). Index 0 of the axis of size 2 holds keys, index 1
  values; under grouped-query attention the pool's head axis counts KV heads.
* Blocks hold 16 tokens (same page, section "PagedAttention 方案", and the
  ``--block-size`` default in the table of launch flags). The functions below
  take the block size from the pool's shape.
* A sequence of n tokens holds ceil(n / block_size) blocks (same code listing,
  ``allocate``). Logical block j of a sequence lives in physical block
  ``table[j]``; blocks need not be contiguous (page "vLLM GitHub 项目 …",
  section 二, item 1) and may be shared by several sequences (item 4).
* The attention itself is softmax attention of one query row over the
  sequence's keys and values in logical order, scaled by ``scale``
  (1/sqrt(head_size)); the pages name it but print no formula, so the textbook
  definition is used. Query head h reads KV head ``h // (Hq // Hkv)``.
* A decode query sits at the last position and sees every cached token,
  including the one appended this step. A prefill chunk of C queries after P
  cached tokens is causal, bottom-right aligned: chunk row i sees positions
  ``0 .. P + i``.
* A sequence of length 0 yields an all-zero output row.
"""

from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------------------------------
# block bookkeeping
# ---------------------------------------------------------------------------------------

def blocks_needed(num_tokens: int, block_size: int = 16) -> int:
    """Blocks a sequence of ``num_tokens`` occupies: ceil(num_tokens / block_size).

    Page "vLLM 部署深度指南", section "PagedAttention 原理", ``allocate`` in the
    code listing.
    """
    return (int(num_tokens) + block_size - 1) // block_size


def slot_of(block_table_row, pos: int, block_size: int = 16) -> int:
    """Flat slot of logical position ``pos``: physical block * block_size + offset in it."""
    logical_block = pos // block_size
    offset = pos % block_size
    return int(block_table_row[logical_block]) * block_size + offset


class KVCacheExhausted(RuntimeError):
    """Raised when the free list is empty (the listing raises an OOM error there)."""


class BlockAllocator:
    """Block bookkeeping of the simplified KV-cache class on page "vLLM 部署深度指南".

    The free list starts as ``0 .. num_blocks-1`` and blocks are taken from its
    front. ``allocate`` gives a sequence ceil(n / block_size) blocks and fails
    when the list runs dry. ``append_token`` takes a new block only when the
    sequence's last block is full (page "vLLM GitHub 项目 …", section 二, item 1).
    """

    def __init__(self, num_blocks: int, block_size: int = 16):
        self.block_size = block_size
        self.free_blocks = list(range(num_blocks))
        self.block_tables = {}
        self.lengths = {}

    def _take(self) -> int:
        if not self.free_blocks:
            raise KVCacheExhausted("KV cache exhausted")
        return self.free_blocks.pop(0)

    def allocate(self, seq_id, num_tokens: int):
        table = []
        for _ in range(blocks_needed(num_tokens, self.block_size)):
            table.append(self._take())
        self.block_tables[seq_id] = table
        self.lengths[seq_id] = int(num_tokens)
        return table

    def append_token(self, seq_id) -> int:
        """Reserve the slot of the sequence's next token and return it."""
        table = self.block_tables[seq_id]
        pos = self.lengths[seq_id]
        if pos == len(table) * self.block_size:
            table.append(self._take())
        self.lengths[seq_id] = pos + 1
        return slot_of(table, pos, self.block_size)


# ---------------------------------------------------------------------------------------
# writing and reading the pool
# ---------------------------------------------------------------------------------------

def expected_slots(block_tables, seq_lens, cached_lens, block_size: int = 16) -> np.ndarray:
    """Slots of the tokens appended this step, in sequence order (positions cached..len-1)."""
    out = []
    for b in range(len(seq_lens)):
        for pos in range(int(cached_lens[b]), int(seq_lens[b])):
            out.append(slot_of(block_tables[b], pos, block_size))
    return np.asarray(out, dtype=np.int64)


def kv_append(pool: np.ndarray, key: np.ndarray, value: np.ndarray, slot_mapping) -> np.ndarray:
    """Copy of ``pool`` with token t's key and value written at slot ``slot_mapping[t]``.

    A negative slot means "no token" and is skipped. Page "vLLM 部署深度指南",
    ``append_kv`` in the code listing: new K/V go to the sequence's physical block.
    """
    out = pool.copy()
    block_size = pool.shape[1]
    for t, slot in enumerate(np.asarray(slot_mapping)):
        slot = int(slot)
        if slot < 0:
            continue
        block, offset = slot // block_size, slot % block_size
        out[block, offset, 0] = key[t]
        out[block, offset, 1] = value[t]
    return out


def gather_kv(pool: np.ndarray, block_table_row, length: int):
    """Keys and values of a sequence's logical positions 0..length-1, in pool dtype.

    Returns ``(K, V)``, each ``[length, num_kv_heads, head_size]``.
    """
    block_size = pool.shape[1]
    n = blocks_needed(length, block_size)
    assert len(block_table_row) >= n
    pos = np.arange(length)
    phys = np.asarray(block_table_row)[pos // block_size]
    off = pos % block_size
    rows = pool[phys, off]  # [length, 2, Hkv, D]
    return rows[:, 0].copy(), rows[:, 1].copy()


# ---------------------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------------------

def kv_head_of(q_head: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head ``q_head``: consecutive groups of Hq/Hkv query heads."""
    group = num_q_heads // num_kv_heads
    return q_head // group


def softmax_attention(q_row: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float):
    """Textbook attention of one query over n keys/values, fp64.

    s_t = scale * <q, k_t>;  p_t = exp(s_t - max s);  out = sum_t p_t v_t / sum_t p_t.
    """
    if keys.shape[0] == 0:
        return np.zeros(values.shape[1], dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    s = scale * (keys @ np.asarray(q_row, dtype=np.float64))
    p = np.exp(s - s.max())
    return (p @ values) / p.sum()


def decode(q, pool, block_tables, context_lens, scale):
    """One decode step: query b attends to its sequence's first ``context_lens[b]`` tokens.

    ``q`` is ``[B, Hq, D]``; the result is fp64 ``[B, Hq, D]``.
    """
    B, Hq, D = q.shape
    Hkv = pool.shape[3]
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        if L == 0:
            continue
        K, V = gather_kv(pool, block_tables[b], L)
        K, V = K.astype(np.float64), V.astype(np.float64)  # fp16 -> fp64 is exact
        for h in range(Hq):
            k = kv_head_of(h, Hq, Hkv)
            out[b, h] = softmax_attention(q[b, h], K[:, k], V[:, k], scale)
    return out


def decode_rows(q, pool, block_tables, context_lens, scale, pairs):
    """Decode output of selected (sequence, query head) pairs only: fp64 ``[len(pairs), D]``."""
    Hq = q.shape[1]
    Hkv = pool.shape[3]
    out = np.zeros((len(pairs), q.shape[2]), dtype=np.float64)
    cache = {}
    for i, (b, h) in enumerate(pairs):
        L = int(context_lens[b])
        if L == 0:
            continue
        if b not in cache:
            cache.clear()
            cache[b] = gather_kv(pool, block_tables[b], L)
        K, V = cache[b]
        k = kv_head_of(h, Hq, Hkv)
        out[i] = softmax_attention(q[b, h], K[:, k], V[:, k], scale)
    return out


def decode_partitioned(q, pool, block_tables, context_lens, scale, partition_size):
    """Decode computed partition by partition and merged by log-sum-exp.

    Partition p of a sequence holds positions [p*size, (p+1)*size). For each
    partition: m_p = max_t s_t, l_p = sum_t exp(s_t - m_p),
    o_p = sum_t exp(s_t - m_p) v_t / l_p. Merge: M = max_p m_p,
    w_p = l_p exp(m_p - M), out = sum_p w_p o_p / sum_p w_p. Algebraically the
    same value as :func:`decode`; the tests hold it to rounding.
    """
    B, Hq, D = q.shape
    Hkv = pool.shape[3]
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        if L == 0:
            continue
        K, V = gather_kv(pool, block_tables[b], L)
        for h in range(Hq):
            k = kv_head_of(h, Hq, Hkv)
            ms, ls, os_ = [], [], []
            for start in range(0, L, partition_size):
                Kp = K[start: start + partition_size, k].astype(np.float64)
                Vp = V[start: start + partition_size, k].astype(np.float64)
                s = scale * (Kp @ q[b, h].astype(np.float64))
                m = s.max()
                e = np.exp(s - m)
                ms.append(m)
                ls.append(e.sum())
                os_.append((e @ Vp) / e.sum())
            M = max(ms)
            w = np.array([l * np.exp(m - M) for m, l in zip(ms, ls)])
            out[b, h] = (w @ np.array(os_)) / w.sum()
    return out


def prefill_chunk(q, pool, block_tables, query_start_loc, seq_lens, scale, rows=None):
    """Causal attention of prefill chunks over their paged context.

    Request r has ``C = query_start_loc[r+1] - query_start_loc[r]`` query rows
    and ``S = seq_lens[r]`` tokens in the pool (its chunk already appended), so
    ``P = S - C`` tokens precede the chunk. Chunk row i sits at position P + i
    and sees positions 0 .. P + i. Returns fp64 ``[total_q, Hq, D]``; with
    ``rows`` (a set of global query rows) only those rows are computed, the
    rest stay zero.
    """
    total_q, Hq, D = q.shape
    Hkv = pool.shape[3]
    out = np.zeros((total_q, Hq, D), dtype=np.float64)
    R = len(seq_lens)
    for r in range(R):
        q0, q1 = int(query_start_loc[r]), int(query_start_loc[r + 1])
        C, S = q1 - q0, int(seq_lens[r])
        P = S - C
        assert P >= 0
        wanted = [i for i in range(C) if rows is None or (q0 + i) in rows]
        if not wanted:
            continue
        K, V = gather_kv(pool, block_tables[r], S)
        K, V = K.astype(np.float64), V.astype(np.float64)  # fp16 -> fp64 is exact
        for i in wanted:
            visible = P + i + 1
            for h in range(Hq):
                k = kv_head_of(h, Hq, Hkv)
                out[q0 + i, h] = softmax_attention(q[q0 + i, h], K[:visible, k], V[:visible, k], scale)
    return out
