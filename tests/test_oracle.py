"""The CPU oracle against its pins (no GPU needed)."""

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st, HealthCheck

import oracle
from oracle import paged_attention as opa
import workloads

import pins


# ---------------------------------------------------------------------------------------
# small cases shared by the tests
# ---------------------------------------------------------------------------------------

def mha_case():
    # ragged lengths across block and partition edges; last token appended this step
    return workloads.decode_case(21, [1, 2, 15, 16, 17, 33, 64, 100], 3, 3, 32, keep_logical=True)


def gqa_case():
    return workloads.decode_case(22, [5, 16, 31, 70], 8, 2, 16, keep_logical=True)


def shared_case():
    return workloads.prefix_shared_case(23, 3, 4, 2, [1, 5, 16, 20, 3, 9, 17, 2, 30, 1, 8, 16],
                                        4, 2, 16, keep_logical=True)


def mixed_case():
    return workloads.mixed_case(24, [0, 5, 37], [9, 16, 23], [3, 40], 4, 2, 16, keep_logical=True)


# ---------------------------------------------------------------------------------------
# pins on the oracle as written
# ---------------------------------------------------------------------------------------

def test_golden_block_table_figure():
    pins.check_block_table_figure()


def test_golden_allocator_listing():
    pins.check_allocator_listing()


def test_blocks_needed_closed_form():
    pins.check_blocks_needed_closed_form()


def test_allocator_grows_only_when_full():
    alloc = opa.BlockAllocator(4, 16)
    alloc.allocate("s", 15)
    assert alloc.block_tables["s"] == [0]
    assert alloc.append_token("s") == 15  # position 15 still fits block 0
    assert alloc.block_tables["s"] == [0]
    assert alloc.append_token("s") == 16 * 1 + 0  # position 16 opens block 1
    assert alloc.block_tables["s"] == [0, 1]
    assert len(alloc.block_tables["s"]) == opa.blocks_needed(alloc.lengths["s"])


@pytest.mark.parametrize("make", [mha_case, gqa_case, shared_case, mixed_case])
def test_gather_matches_logical(make):
    pins.check_gather_matches_logical(make())


def test_gather_tiny():
    pins.check_gather_matches_logical(workloads.tiny_decode())


@pytest.mark.parametrize("make", [mha_case, gqa_case, mixed_case])
def test_decode_vs_sdpa(make):
    pins.check_decode_vs_sdpa(make())


def test_decode_vs_sdpa_tiny():
    pins.check_decode_vs_sdpa(workloads.tiny_decode())


def test_decode_vs_brute_force():
    inp = workloads.decode_case(25, [1, 3, 17, 20], 2, 1, 8, keep_logical=True)
    pins.check_decode_vs_brute_force(inp)


def test_closed_forms():
    pins.check_closed_forms()


@pytest.mark.parametrize("make", [mha_case, gqa_case, mixed_case])
def test_permutation_invariance(make):
    pins.check_permutation_invariance(make())


def test_prefix_sharing():
    pins.check_prefix_sharing(shared_case())


def test_partitioned_equals_direct():
    pins.check_partitioned(mha_case())


def test_partitioned_boundaries():
    inp = workloads.decode_case(26, [511, 512, 513, 1024, 1025], 2, 2, 16, keep_logical=True)
    pins.check_partitioned(inp, sizes=(512, 256, 16))


def test_gqa_equals_mha():
    pins.check_gqa_equals_mha(gqa_case())


def test_prefill_vs_sdpa():
    pins.check_prefill_vs_sdpa(mixed_case())


def test_prefill_row_is_decode():
    pins.check_prefill_row_is_decode(mixed_case())


def test_prefill_chunk_split():
    inp = workloads.mixed_case(27, [0, 19], [16, 10], [], 2, 2, 16, keep_logical=True)
    pins.check_prefill_chunk_split(inp)


@pytest.mark.parametrize("make", [mha_case, shared_case, mixed_case])
def test_kv_append(make):
    pins.check_kv_append(make())


def test_kv_append_full_tiny():
    """All 65 tokens of the tiny batch appended into an all-NaN pool rebuild its pool bit for bit."""
    base = workloads.tiny_decode()
    full = workloads.tiny_decode_full_append()
    pins.check_kv_append(full)
    out = opa.kv_append(full.pool, full.key_new, full.value_new, full.slot_mapping)
    assert np.array_equal(out.view(np.uint16), base.pool.view(np.uint16))


def test_kv_append_skips_negative_slots():
    inp = mha_case()
    slots = inp.slot_mapping.copy()
    slots[::2] = -1
    out = opa.kv_append(inp.pool, inp.key_new, inp.value_new, slots)
    for t in range(0, len(slots), 2):
        s = inp.slot_mapping[t]
        assert np.array_equal(out[s // 16, s % 16].view(np.uint16), inp.pool[s // 16, s % 16].view(np.uint16))


def test_length_zero_gives_zeros():
    inp = workloads.decode_case(28, [0, 5], 2, 2, 16, append=False)
    out = oracle.decode(inp.q, inp.pool, inp.block_tables, inp.seq_lens, inp.scale)
    assert np.all(out[0] == 0)
    assert np.all(np.isfinite(out[1]))


def test_decode_rows_matches_decode():
    inp = mha_case()
    pool = opa.kv_append(inp.pool, inp.key_new, inp.value_new, inp.slot_mapping)
    full = oracle.decode(inp.q, pool, inp.block_tables, inp.seq_lens, inp.scale)
    pairs = [(0, 0), (3, 2), (7, 1), (7, 0)]
    rows = oracle.decode_rows(inp.q, pool, inp.block_tables, inp.seq_lens, inp.scale, pairs)
    for i, (b, h) in enumerate(pairs):
        assert np.array_equal(rows[i], full[b, h])


# ---------------------------------------------------------------------------------------
# property tests: random lengths, placements and sharing
# ---------------------------------------------------------------------------------------

@settings(max_examples=25, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(
    lens=st.lists(st.integers(min_value=1, max_value=80), min_size=1, max_size=5),
    g=st.sampled_from([1, 2, 4]),
    seed=st.integers(min_value=0, max_value=2**31 - 1),
)
def test_property_invariants(lens, g, seed):
    inp = workloads.decode_case(seed, lens, 2 * g, 2, 8, keep_logical=True)
    pins.check_gather_matches_logical(inp)
    pins.check_permutation_invariance(inp, seed=seed + 1, require_moved=False)
    pins.check_partitioned(inp, sizes=(16, 32))
    pins.check_kv_append(inp)
    for b, L in enumerate(lens):
        nb = opa.blocks_needed(L)
        assert nb == -(-L // 16)
        assert np.all(inp.block_tables[b, nb:] == inp.poison_block)


# ---------------------------------------------------------------------------------------
# planted mistakes: each pin must notice a plausible error in the oracle
# ---------------------------------------------------------------------------------------

def _expect_failure(check, *args):
    with pytest.raises(AssertionError):
        check(*args)


def test_pins_catch_dropped_scale(monkeypatch):
    real = opa.softmax_attention
    monkeypatch.setattr(opa, "softmax_attention", lambda q, K, V, scale: real(q, K, V, 1.0))
    _expect_failure(pins.check_decode_vs_sdpa, mha_case())


def test_pins_catch_dropped_last_key(monkeypatch):
    real = opa.softmax_attention
    monkeypatch.setattr(opa, "softmax_attention",
                        lambda q, K, V, scale: real(q, K[:-1], V[:-1], scale) if len(K) > 1 else real(q, K, V, scale))
    _expect_failure(pins.check_decode_vs_sdpa, mha_case())
    _expect_failure(pins.check_prefill_vs_sdpa, mixed_case())


def test_pins_catch_wrong_kv_head(monkeypatch):
    monkeypatch.setattr(opa, "kv_head_of", lambda h, hq, hkv: h % hkv)
    _expect_failure(pins.check_gqa_equals_mha, gqa_case())
    _expect_failure(pins.check_decode_vs_sdpa, gqa_case())


def test_pins_catch_swapped_k_and_v(monkeypatch):
    real = opa.gather_kv
    monkeypatch.setattr(opa, "gather_kv", lambda pool, row, L: real(pool, row, L)[::-1])
    _expect_failure(pins.check_gather_matches_logical, mha_case())
    _expect_failure(pins.check_decode_vs_sdpa, mha_case())


def test_pins_catch_reversed_offsets(monkeypatch):
    def bad_gather(pool, row, L):
        bs = pool.shape[1]
        pos = np.arange(L)
        rows = pool[np.asarray(row)[pos // bs], bs - 1 - pos % bs]
        return rows[:, 0].copy(), rows[:, 1].copy()
    monkeypatch.setattr(opa, "gather_kv", bad_gather)
    _expect_failure(pins.check_gather_matches_logical, mha_case())


def test_pins_catch_wrong_block_count(monkeypatch):
    monkeypatch.setattr(opa, "blocks_needed", lambda n, bs=16: n // bs)
    _expect_failure(pins.check_blocks_needed_closed_form)
    _expect_failure(pins.check_block_table_figure)


def test_pins_catch_lifo_allocator(monkeypatch):
    def take_back(self):
        if not self.free_blocks:
            raise opa.KVCacheExhausted("x")
        return self.free_blocks.pop()
    monkeypatch.setattr(opa.BlockAllocator, "_take", take_back)
    _expect_failure(pins.check_allocator_listing)


def test_pins_catch_top_left_causal(monkeypatch):
    # visible = i + 1 instead of P + i + 1 (top-left alignment)
    real = opa.softmax_attention

    def fake_prefill(q, pool, bt, qsl, lens, scale, rows=None):
        out = np.zeros(q.shape, np.float64)
        for r in range(len(lens)):
            q0, q1 = int(qsl[r]), int(qsl[r + 1])
            K, V = opa.gather_kv(pool, bt[r], int(lens[r]))
            for i in range(q1 - q0):
                for h in range(q.shape[1]):
                    k = opa.kv_head_of(h, q.shape[1], pool.shape[3])
                    out[q0 + i, h] = real(q[q0 + i, h], K[: i + 1, k], V[: i + 1, k], scale)
        return out
    monkeypatch.setattr(oracle, "prefill_chunk", fake_prefill)
    _expect_failure(pins.check_prefill_vs_sdpa, mixed_case())


def test_pins_catch_unweighted_partition_merge(monkeypatch):
    def bad(q, pool, bt, lens, scale, ps):
        # average of partition outputs without the l_p * exp(m_p - M) weights
        out = np.zeros(q.shape, np.float64)
        for b in range(q.shape[0]):
            L = int(lens[b])
            K, V = opa.gather_kv(pool, bt[b], L)
            for h in range(q.shape[1]):
                k = opa.kv_head_of(h, q.shape[1], pool.shape[3])
                parts = [opa.softmax_attention(q[b, h], K[s:s + ps, k], V[s:s + ps, k], scale)
                         for s in range(0, L, ps)]
                out[b, h] = np.mean(parts, axis=0)
        return out
    monkeypatch.setattr(oracle, "decode_partitioned", bad)
    _expect_failure(pins.check_partitioned, mha_case())


def test_pins_catch_append_to_wrong_half(monkeypatch):
    def bad_append(pool, key, value, slots):
        out = pool.copy()
        bs = pool.shape[1]
        for t, s in enumerate(slots):
            out[s // bs, s % bs, 1] = key[t]
            out[s // bs, s % bs, 0] = value[t]
        return out
    monkeypatch.setattr(opa, "kv_append", bad_append)
    _expect_failure(pins.check_kv_append, mha_case())


# ---------------------------------------------------------------------------------------
# block manager (refcounts, fork, copy-on-write, free) and block copies
# ---------------------------------------------------------------------------------------

def test_golden_block_manager_trace():
    pins.check_block_manager_golden()


@pytest.mark.parametrize("seed", range(6))
def test_block_manager_semantics(seed):
    pins.check_block_manager_semantics(seed)


@pytest.mark.parametrize("seed", range(4))
def test_block_manager_without_forks_is_the_listing(seed):
    pins.check_block_manager_without_forks_is_the_listing(seed)


def test_block_copies():
    pins.check_block_copies()


def test_block_manager_fresh_and_full():
    m = oracle.BlockManager(10)
    assert m.usage() == 0.0 and m.slot_utilisation() == 0.0
    m.allocate("x", 48)
    assert m.usage() == pytest.approx(0.3) and m.slot_utilisation() == 1.0
    with pytest.raises(oracle.KVCacheExhausted):
        m.allocate("y", 16 * 8)  # 8 blocks > 7 free: nothing taken
    assert len(m.free_blocks) == 7


def _bm_planted(monkeypatch, name, fn, checks):
    from oracle import block_manager as obm
    monkeypatch.setattr(obm.BlockManager, name, fn)
    for check in checks:
        with pytest.raises(AssertionError):
            check()


def test_pins_catch_lifo_free_list(monkeypatch):
    def _take(self):
        b = self.free_blocks.pop()
        self.refs[b] = 1
        return b
    _bm_planted(monkeypatch, "_take", _take, [pins.check_block_manager_golden])


def test_pins_catch_missing_copy_on_write(monkeypatch):
    from oracle import block_manager as obm
    orig = obm.BlockManager.append_token

    def append_token(self, seq_id):
        table, pos = self.tables[seq_id], self.lengths[seq_id]
        if pos < len(table) * self.block_size:  # write into the last block even if shared
            self.lengths[seq_id] = pos + 1
            return table[pos // self.block_size] * self.block_size + pos % self.block_size, None
        return orig(self, seq_id)
    _bm_planted(monkeypatch, "append_token", append_token,
                [pins.check_block_manager_golden, lambda: pins.check_block_manager_semantics(0)])


def test_pins_catch_reversed_copy(monkeypatch):
    from oracle import block_manager as obm
    orig = obm.BlockManager.append_token

    def append_token(self, seq_id):
        slot, copy = orig(self, seq_id)
        return slot, None if copy is None else (copy[1], copy[0])
    _bm_planted(monkeypatch, "append_token", append_token,
                [lambda: pins.check_block_manager_semantics(0)])


def test_pins_catch_free_to_front(monkeypatch):
    def free(self, seq_id):
        for b in self.tables.pop(seq_id):
            self.refs[b] -= 1
            if self.refs[b] == 0:
                self.free_blocks.insert(0, b)
        del self.lengths[seq_id]
    _bm_planted(monkeypatch, "free", free, [pins.check_block_manager_golden])


def test_pins_catch_refcount_kept_on_copy(monkeypatch):
    from oracle import block_manager as obm
    orig = obm.BlockManager.append_token

    def append_token(self, seq_id):
        slot, copy = orig(self, seq_id)
        if copy is not None:
            self.refs[copy[0]] += 1  # forget to drop the shared block's reference
        return slot, copy
    _bm_planted(monkeypatch, "append_token", append_token,
                [lambda: pins.check_block_manager_semantics(1)])
