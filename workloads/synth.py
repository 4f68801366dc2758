"""Seeded synthetic workloads for paged KV-cache attention.

Pool layout: ``[num_blocks, block_size, 2, num_kv_heads, head_size]`` fp16, the
per-layer pool tensor of the page "vLLM 部署深度指南" (section "PagedAttention
原理", code listing of the simplified KV-cache class). Index 0 of the axis of
size 2 holds keys, index 1 values. Each sequence reaches its blocks through a
row of ``block_tables``; blocks sit anywhere in the pool (page "vLLM GitHub 项目
…", section 二, item 1) and prefix blocks may be shared between sequences
(same section, item 4).

Recipe shared by every case:

1. lengths, drawn by the case function from ``numpy.random.default_rng(seed)``,
2. ``rng.permutation(num_blocks)`` from the same generator: sequences take
   physical blocks in that order, logical block by logical block; the last
   entry of the permutation is never handed out and serves as the all-NaN
   padding block,
3. every other value comes from its own child stream
   ``default_rng(SeedSequence(seed, spawn_key=key))``, so no value depends on
   the order in which threads fill the pool:

   * key ``(1, b, c)``: cached K/V of sequence ``b``, its private tokens
     ``[1024c, 1024c + 1024)`` counted from its first private token,
     shape ``[n, 2, Hkv, D]``,
   * key ``(2, g, c)``: the same for the shared prompt of group ``g``,
   * key ``(3,)``: the queries ``[sum(q_lens), Hq, D]``,
   * key ``(4,)``: the K/V of the tokens appended this step ``[T, 2, Hkv, D]``.

Values are N(0, 1) drawn in fp32 and rounded to fp16 (round to nearest even).
Every pool slot that holds no cached token holds the fp16 quiet NaN 0x7E00, so a
stray read of an unused block, a tail slot or a not-yet-appended slot shows up
as NaN.

Nothing here computes attention. The helpers that place tokens use the pool's
row index (block, offset) of each logical position, which the oracle derives
again on its own.
"""

from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Optional, Sequence

import numpy as np

POISON_F16 = np.uint16(0x7E00)  # fp16 quiet NaN


@dataclasses.dataclass
class PagedInputs:
    """One batch of sequences over one block pool.

    Sequence ``b`` attends to ``seq_lens[b]`` tokens after this step's append.
    Tokens ``[cached_lens[b], seq_lens[b])`` are appended this step (their K/V
    are rows of ``key_new``/``value_new``, their pool slots hold NaN until the
    append). Its queries are the last ``q_lens[b]`` positions, stored in ``q``
    from row ``query_start_loc[b]``. The first ``num_prefill`` sequences are
    prefill chunks; the rest have one query each (decode).
    """

    pool: np.ndarray  # fp16 [NB, BS, 2, Hkv, D]
    block_tables: np.ndarray  # int32 [S, max_blocks]
    seq_lens: np.ndarray  # int32 [S]
    cached_lens: np.ndarray  # int32 [S]
    q_lens: np.ndarray  # int32 [S]
    query_start_loc: np.ndarray  # int32 [S+1]
    q: np.ndarray  # fp16 [sum(q_lens), Hq, D]
    key_new: np.ndarray  # fp16 [T, Hkv, D]
    value_new: np.ndarray  # fp16 [T, Hkv, D]
    slot_mapping: np.ndarray  # int64 [T]
    num_q_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    scale: float
    poison_block: int
    num_prefill: int
    seed: int
    name: str = ""
    logical_kv: Optional[list] = None  # per sequence fp16 [len, 2, Hkv, D]
    groups: Optional[np.ndarray] = None  # int [S] prefix-sharing group or -1
    prefix_blocks: int = 0

    # ---- views used by the callers -------------------------------------------------
    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.pool.shape[0])

    @property
    def num_decode(self) -> int:
        return self.num_seqs - self.num_prefill

    @property
    def num_prefill_tokens(self) -> int:
        return int(self.query_start_loc[self.num_prefill])

    def decode_part(self):
        """(q, block_tables, context_lens) of the decode sequences."""
        p = self.num_prefill
        q = self.q[self.num_prefill_tokens:]
        return q, self.block_tables[p:], self.seq_lens[p:]

    def prefill_part(self):
        """(q, block_tables, query_start_loc, seq_lens) of the prefill chunks."""
        p = self.num_prefill
        qsl = self.query_start_loc[: p + 1]
        return self.q[: int(qsl[-1])], self.block_tables[:p], qsl.copy(), self.seq_lens[:p]

    def pool_before_append(self) -> np.ndarray:
        return self.pool


_CHUNK = 1024  # cached tokens per child stream


def _child(seed: int, key) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=tuple(key)))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _draw(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float16)


def _num_blocks_for(n_tokens: int, block_size: int) -> int:
    return -(-int(n_tokens) // block_size)


def _token_rows(block_row: np.ndarray, n_tokens: int, block_size: int) -> np.ndarray:
    """Pool row (flattened over [num_blocks, block_size]) of logical positions 0..n-1."""
    nb = _num_blocks_for(n_tokens, block_size)
    rows = np.arange(block_size, dtype=np.int64)[None, :] + (
        block_row[:nb].astype(np.int64)[:, None] * block_size
    )
    return rows.reshape(-1)[:n_tokens]


def build(
    rng: np.random.Generator,
    seed: int,
    seq_lens: Sequence[int],
    cached_lens: Sequence[int],
    q_lens: Sequence[int],
    num_q_heads: int,
    num_kv_heads: int,
    head_size: int,
    *,
    block_size: int = 16,
    num_blocks: Optional[int] = None,
    slack: float = 1.05,
    num_prefill: int = 0,
    groups: Optional[Sequence[int]] = None,
    prefix_blocks: int = 0,
    keep_logical: bool = False,
    max_blocks: Optional[int] = None,
    scale: Optional[float] = None,
    name: str = "",
) -> PagedInputs:
    """Draw one batch after its lengths were drawn (steps 2-5 of the recipe)."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    cached_lens = np.asarray(cached_lens, dtype=np.int64)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    S = seq_lens.shape[0]
    assert cached_lens.shape == (S,) and q_lens.shape == (S,)
    assert np.all(cached_lens <= seq_lens)
    # a decode row of an empty sequence still has its query (its output is zero)
    assert np.all((q_lens <= seq_lens) | ((seq_lens == 0) & (q_lens == 1)))
    assert num_q_heads % num_kv_heads == 0
    BS, Hkv, D, Hq = block_size, num_kv_heads, head_size, num_q_heads
    grp = np.full(S, -1, dtype=np.int64) if groups is None else np.asarray(groups, dtype=np.int64)
    prefix_tokens = prefix_blocks * BS
    for b in range(S):
        if grp[b] >= 0:
            assert cached_lens[b] >= prefix_tokens, "a shared prefix must be cached"

    # -- step 2: physical blocks -----------------------------------------------------
    nblk = np.array([_num_blocks_for(L, BS) for L in seq_lens], dtype=np.int64)
    shared_seen = {}
    needed = 0
    for b in range(S):
        if grp[b] >= 0:
            if grp[b] not in shared_seen:
                shared_seen[grp[b]] = True
                needed += prefix_blocks
            needed += nblk[b] - prefix_blocks
        else:
            needed += nblk[b]
    if num_blocks is None:
        num_blocks = int(math.ceil(slack * needed)) + 1
    assert needed <= num_blocks - 1, "pool too small for the batch"
    perm = rng.permutation(num_blocks)
    poison_block = int(perm[-1])
    if max_blocks is None:
        max_blocks = max(1, int(nblk.max()) if S else 1)
    assert max_blocks >= (int(nblk.max()) if S else 0)
    tables = np.full((S, max_blocks), poison_block, dtype=np.int32)
    cursor = 0
    group_blocks = {}
    for b in range(S):
        j0 = 0
        if grp[b] >= 0:
            g = int(grp[b])
            if g not in group_blocks:
                group_blocks[g] = perm[cursor: cursor + prefix_blocks].copy()
                cursor += prefix_blocks
            tables[b, :prefix_blocks] = group_blocks[g]
            j0 = prefix_blocks
        n = int(nblk[b]) - j0
        tables[b, j0: j0 + n] = perm[cursor: cursor + n]
        cursor += n

    # -- step 3: cached K/V, placed through the tables ----------------------------------
    pool = np.empty((num_blocks, BS, 2, Hkv, D), dtype=np.float16)
    pool.view(np.uint16).fill(POISON_F16)
    flat = pool.reshape(num_blocks * BS, 2, Hkv, D)

    jobs = []  # (spawn key, pool rows) for every chunk of cached tokens
    seen = set()
    for b in range(S):
        rows = _token_rows(tables[b], int(seq_lens[b]), BS)
        start = 0
        if grp[b] >= 0:
            g = int(grp[b])
            if g not in seen:
                seen.add(g)
                for c in range(0, prefix_tokens, _CHUNK):
                    jobs.append(((2, g, c // _CHUNK), rows[c: min(c + _CHUNK, prefix_tokens)]))
            start = prefix_tokens
        n_priv = int(cached_lens[b]) - start
        for c in range(0, n_priv, _CHUNK):
            jobs.append(((1, b, c // _CHUNK), rows[start + c: start + min(c + _CHUNK, n_priv)]))

    drawn = {}

    def fill(job):
        key, rows = job
        kv = _draw(_child(seed, key), (len(rows), 2, Hkv, D))
        flat[rows] = kv
        if keep_logical:
            drawn[key] = kv

    if jobs:
        with concurrent.futures.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, jobs))

    # -- queries and this step's new tokens ----------------------------------------------
    qsl = np.zeros(S + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(q_lens)
    q = _draw(_child(seed, (3,)), (int(qsl[-1]), Hq, D))
    new_lens = seq_lens - cached_lens
    T = int(new_lens.sum())
    kv_new = _draw(_child(seed, (4,)), (T, 2, Hkv, D))
    slots = np.empty(T, dtype=np.int64)
    t0 = 0
    for b in range(S):
        n = int(new_lens[b])
        if n:
            rows = _token_rows(tables[b], int(seq_lens[b]), BS)
            slots[t0: t0 + n] = rows[int(cached_lens[b]):]
        t0 += n

    logical = None
    if keep_logical:
        # each sequence's drawn values in logical order: shared prompt, private cached
        # tokens, then this step's new tokens
        logical = []
        t0 = 0
        empty = np.empty((0, 2, Hkv, D), np.float16)
        for b in range(S):
            parts = []
            start = 0
            if grp[b] >= 0:
                parts += [drawn[(2, int(grp[b]), c)] for c in range(-(-prefix_tokens // _CHUNK))]
                start = prefix_tokens
            n_priv = int(cached_lens[b]) - start
            parts += [drawn[(1, b, c)] for c in range(-(-n_priv // _CHUNK))]
            n_new = int(new_lens[b])
            parts.append(kv_new[t0: t0 + n_new])
            t0 += n_new
            logical.append(np.concatenate(parts, axis=0) if parts else empty)

    return PagedInputs(
        pool=pool,
        block_tables=tables,
        seq_lens=seq_lens.astype(np.int32),
        cached_lens=cached_lens.astype(np.int32),
        q_lens=q_lens.astype(np.int32),
        query_start_loc=qsl,
        q=q,
        key_new=np.ascontiguousarray(kv_new[:, 0]),
        value_new=np.ascontiguousarray(kv_new[:, 1]),
        slot_mapping=slots,
        num_q_heads=Hq,
        num_kv_heads=Hkv,
        head_size=D,
        block_size=BS,
        scale=float(1.0 / math.sqrt(D)) if scale is None else float(scale),
        poison_block=poison_block,
        num_prefill=int(num_prefill),
        seed=int(seed),
        name=name,
        logical_kv=logical,
        groups=None if groups is None else grp,
        prefix_blocks=int(prefix_blocks),
    )


# ---------------------------------------------------------------------------------------
# generic cases (tests use these at small sizes)
# ---------------------------------------------------------------------------------------

def decode_case(seed, lens, num_q_heads, num_kv_heads, head_size, *, append=True,
                keep_logical=False, num_blocks=None, slack=1.05, max_blocks=None, name=""):
    """Decode batch: one query per sequence; with ``append`` the last token is new."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    cached = lens - 1 if append else lens.copy()
    cached = np.maximum(cached, 0)
    qlens = np.ones_like(lens)
    return build(rng, seed, lens, cached, qlens, num_q_heads, num_kv_heads, head_size,
                 num_blocks=num_blocks, slack=slack, keep_logical=keep_logical,
                 max_blocks=max_blocks, name=name)


def mixed_case(seed, prefill_priors, chunk_lens, decode_lens, num_q_heads, num_kv_heads,
               head_size, *, keep_logical=False, slack=1.05, max_blocks=None, name=""):
    """Prefill chunks (prior P_r cached, chunk C_r new and queried) then decodes."""
    rng = np.random.default_rng(seed)
    pri = np.asarray(prefill_priors, dtype=np.int64)
    ch = np.asarray(chunk_lens, dtype=np.int64)
    dl = np.asarray(decode_lens, dtype=np.int64)
    lens = np.concatenate([pri + ch, dl])
    cached = np.concatenate([pri, dl - 1])
    qlens = np.concatenate([ch, np.ones_like(dl)])
    return build(rng, seed, lens, cached, qlens, num_q_heads, num_kv_heads, head_size,
                 num_prefill=len(pri), slack=slack, keep_logical=keep_logical,
                 max_blocks=max_blocks, name=name)


def prefix_shared_case(seed, num_groups, samples, prefix_blocks, private_lens, num_q_heads,
                       num_kv_heads, head_size, *, keep_logical=False, slack=1.05, name=""):
    """Groups of ``samples`` sequences whose first ``prefix_blocks`` blocks are shared."""
    rng = np.random.default_rng(seed)
    priv = np.asarray(private_lens, dtype=np.int64)
    assert priv.shape == (num_groups * samples,)
    lens = prefix_blocks * 16 + priv
    groups = np.repeat(np.arange(num_groups), samples)
    return build(rng, seed, lens, lens.copy(), np.ones_like(lens), num_q_heads, num_kv_heads,
                 head_size, groups=groups, prefix_blocks=prefix_blocks, slack=slack,
                 keep_logical=keep_logical, name=name)


# ---------------------------------------------------------------------------------------
# the five frozen workloads
# ---------------------------------------------------------------------------------------

def tiny_decode(keep_logical=True) -> PagedInputs:
    """Tiny paged decode: lengths {1, 15, 16, 33}, 4 heads x 64, 16 physical blocks."""
    rng = np.random.default_rng(1)
    lens = np.array([1, 15, 16, 33])
    return build(rng, 1, lens, lens.copy(), np.ones(4, np.int64), 4, 4, 64, num_blocks=16,
                 keep_logical=keep_logical, scale=1.0 / 8.0, name="tiny-decode-4x{1,15,16,33}")


def tiny_decode_full_append() -> PagedInputs:
    """The tiny decode batch with every one of its 65 tokens appended into an all-NaN pool."""
    base = tiny_decode(keep_logical=True)
    inp = dataclasses.replace(base)
    pool = np.empty_like(base.pool)
    pool.view(np.uint16).fill(POISON_F16)
    kv = np.concatenate(base.logical_kv, axis=0)
    slots = np.concatenate([
        _token_rows(base.block_tables[b], int(base.seq_lens[b]), base.block_size)
        for b in range(base.num_seqs)
    ])
    inp.pool = pool
    inp.cached_lens = np.zeros_like(base.seq_lens)
    inp.key_new = np.ascontiguousarray(kv[:, 0])
    inp.value_new = np.ascontiguousarray(kv[:, 1])
    inp.slot_mapping = slots.astype(np.int64)
    inp.name = "tiny-append-65"
    return inp


def decode_256seq(keep_logical=False) -> PagedInputs:
    """Llama-7B-layer-shaped decode: 256 sequences, lengths U{128..2048}, 32 x 128, append."""
    rng = np.random.default_rng(2)
    lens = rng.integers(128, 2048, size=256, endpoint=True)
    return build(rng, 2, lens, lens - 1, np.ones(256, np.int64), 32, 32, 128,
                 keep_logical=keep_logical, name="decode-256seq-U[128,2048]-32x128")


def long_context_32k(keep_logical=False) -> PagedInputs:
    """Long-context decode: 8 sequences of 32768 tokens, 32 x 128."""
    rng = np.random.default_rng(3)
    lens = np.full(8, 32768)
    return build(rng, 3, lens, lens.copy(), np.ones(8, np.int64), 32, 32, 128,
                 num_blocks=8 * 2048 + 1, keep_logical=keep_logical,
                 name="decode-8seq-32768-32x128")


def shared_prompt_groups(keep_logical=False) -> PagedInputs:
    """Prefix-shared GQA decode: 64 groups x 4 samples, 64 shared blocks, 32q/8kv x 128."""
    rng = np.random.default_rng(4)
    priv = rng.integers(64, 256, size=256, endpoint=True)
    lens = 1024 + priv
    groups = np.repeat(np.arange(64), 4)
    return build(rng, 4, lens, lens.copy(), np.ones(256, np.int64), 32, 8, 128, groups=groups,
                 prefix_blocks=64, keep_logical=keep_logical,
                 name="gqa-prefix-shared-64x4-32q8kv")


def mixed_prefill_decode(keep_logical=False) -> PagedInputs:
    """Mixed step: 8 prefill chunks of 512 over priors U{0..3584}, 248 decodes U{256..4096}."""
    rng = np.random.default_rng(5)
    pri = np.empty(8, np.int64)
    pri[0], pri[7] = 0, 3584
    pri[1:7] = rng.integers(0, 3584, size=6, endpoint=True)
    dl = rng.integers(256, 4096, size=248, endpoint=True)
    lens = np.concatenate([pri + 512, dl])
    cached = np.concatenate([pri, dl - 1])
    qlens = np.concatenate([np.full(8, 512), np.ones(248, np.int64)])
    return build(rng, 5, lens, cached, qlens, 32, 32, 128, num_prefill=8,
                 keep_logical=keep_logical, name="mixed-8x512prefill+248decode-32x128")


def long_prompt_prefill(keep_logical=False) -> PagedInputs:
    """The last 512-row chunk of a 32768-token prompt (32256 tokens cached before it) in a
    step with 8 decodes U{256..4096}: few row tiles next to a long context."""
    rng = np.random.default_rng(6)
    dl = rng.integers(256, 4096, size=8, endpoint=True)
    return mixed_case(6, [32256], [512], dl.tolist(), 32, 32, 128, keep_logical=keep_logical,
                      name="long-prompt-chunk-512of32768+8decode-32x128")


WORKLOADS = {"tiny": tiny_decode, "decode256": decode_256seq, "long32k": long_context_32k,
             "prefix-groups": shared_prompt_groups, "mixed": mixed_prefill_decode,
             "long-prefill": long_prompt_prefill}


# ---------------------------------------------------------------------------------------
# variants that move blocks but keep every logical value
# ---------------------------------------------------------------------------------------

def _rebuild_slots(inp: PagedInputs, tables: np.ndarray) -> np.ndarray:
    out = np.empty_like(inp.slot_mapping)
    t0 = 0
    for b in range(inp.num_seqs):
        n = int(inp.seq_lens[b] - inp.cached_lens[b])
        if n:
            rows = _token_rows(tables[b], int(inp.seq_lens[b]), inp.block_size)
            out[t0: t0 + n] = rows[int(inp.cached_lens[b]):]
        t0 += n
    return out


def repermute(inp: PagedInputs, seed: int) -> PagedInputs:
    """Move every physical block to a new place (block i goes to sigma[i])."""
    rng = np.random.default_rng(seed)
    sigma = rng.permutation(inp.num_blocks)
    pool = np.empty_like(inp.pool)
    pool[sigma] = inp.pool
    tables = sigma[inp.block_tables].astype(np.int32)
    out = dataclasses.replace(inp)
    out.pool = pool
    out.block_tables = tables
    out.poison_block = int(sigma[inp.poison_block])
    out.slot_mapping = _rebuild_slots(inp, tables)
    return out


def unshare_prefix(inp: PagedInputs) -> PagedInputs:
    """Give every sequence of a sharing group private copies of the shared blocks."""
    assert inp.groups is not None and inp.prefix_blocks > 0
    S, pb = inp.num_seqs, inp.prefix_blocks
    n_new = S * pb
    pool = np.empty((inp.num_blocks + n_new,) + inp.pool.shape[1:], dtype=inp.pool.dtype)
    pool[: inp.num_blocks] = inp.pool
    tables = inp.block_tables.copy()
    nxt = inp.num_blocks
    for b in range(S):
        if inp.groups[b] < 0:
            continue
        for j in range(pb):
            pool[nxt] = inp.pool[inp.block_tables[b, j]]
            tables[b, j] = nxt
            nxt += 1
    out = dataclasses.replace(inp)
    out.pool = pool[:nxt]
    out.block_tables = tables
    out.groups = None
    out.prefix_blocks = 0
    out.slot_mapping = _rebuild_slots(inp, tables)
    return out
