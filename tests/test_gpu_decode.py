"""GPU parity of kv_append, gather and paged decode against the CPU oracle (MI355X)."""

import dataclasses
import functools

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_294_amd as pkv
import workloads
from gpu_util import (bits, check_attention, dev, host, note, tie_base, tie_expectations,
                      write_tie_values)

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------------------
# running the library on a generated batch
# ---------------------------------------------------------------------------------------

class Dev:
    """Device copies of a batch, with the step's tokens appended on the GPU."""

    def __init__(self, inp, append=True):
        self.inp = inp
        self.pool = dev(inp.pool)
        self.q = dev(inp.q)
        self.bt = dev(inp.block_tables)
        self.lens = dev(inp.seq_lens)
        self.qsl = dev(inp.query_start_loc)
        if append and len(inp.slot_mapping):
            pkv.pa_kv_append(self.pool, dev(inp.key_new), dev(inp.value_new), dev(inp.slot_mapping))

    def decode(self, partition_size=512, max_context_len=None, flags=0):
        inp = self.inp
        p = inp.num_prefill
        q = self.q[inp.num_prefill_tokens:]
        bt, lens = self.bt[p:], self.lens[p:]
        out = torch.empty_like(q)
        mcl = int(inp.seq_lens[p:].max()) if max_context_len is None else max_context_len
        pkv.pa_decode(out, q, self.pool, bt, lens, mcl, inp.scale, partition_size, flags=flags)
        return host(out)


def oracle_pool(inp):
    return oracle.kv_append(inp.pool, inp.key_new, inp.value_new, inp.slot_mapping)


def oracle_decode(inp, pool=None):
    pool = oracle_pool(inp) if pool is None else pool
    q, bt, lens = inp.decode_part()
    return oracle.decode(q, pool, bt, lens, inp.scale)


@functools.lru_cache(maxsize=2)
def cfg(name):
    note(f"generating workload {name}")
    return workloads.WORKLOADS[name]()


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------------------
# kv_append: bit-exact, whole pool compared
# ---------------------------------------------------------------------------------------

def check_append(inp):
    d = Dev(inp, append=True)
    got = host(d.pool)
    ref = oracle_pool(inp)
    assert np.array_equal(bits(got), bits(ref)), "pool differs from the oracle's append"
    del d
    free()


def test_append_tiny_full_into_nan_pool():
    inp = workloads.tiny_decode_full_append()
    check_append(inp)
    # the appended pool is the tiny decode batch's pool
    d = Dev(inp, append=True)
    assert np.array_equal(bits(host(d.pool)), bits(workloads.tiny_decode().pool))


def test_append_small_mixed_and_ragged():
    check_append(workloads.mixed_case(31, [0, 5, 37, 100], [9, 16, 23, 64], [1, 3, 40, 17], 4, 2, 64))
    check_append(workloads.decode_case(32, [1, 15, 16, 17, 31, 32, 33], 8, 8, 128))


def test_append_skips_negative_and_out_of_pool_slots():
    inp = workloads.decode_case(33, [5, 20, 40, 7], 4, 4, 64)
    slots = inp.slot_mapping.copy()
    slots[0] = -1
    slots[2] = inp.num_blocks * 16 + 5  # beyond the pool: skipped
    bad = dataclasses.replace(inp, slot_mapping=slots)
    d = Dev(bad, append=True)
    got = host(d.pool)
    ref = oracle.kv_append(inp.pool, inp.key_new, inp.value_new,
                           np.where(slots >= inp.num_blocks * 16, -1, slots))
    assert np.array_equal(bits(got), bits(ref))


def test_append_strided_rows():
    inp = workloads.decode_case(34, [3, 9, 30], 4, 4, 128)
    T, H, D = inp.key_new.shape
    # key/value as views into a fused [T, 3, H, D] projection output
    fused = np.zeros((T, 3, H, D), np.float16)
    fused[:, 1] = inp.key_new
    fused[:, 2] = inp.value_new
    f = dev(fused)
    pool = dev(inp.pool)
    pkv.pa_kv_append(pool, f[:, 1], f[:, 2], dev(inp.slot_mapping))
    assert np.array_equal(bits(host(pool)), bits(oracle_pool(inp)))


def test_append_decode256_full():
    check_append(cfg("decode256"))


def test_append_mixed_full():
    check_append(cfg("mixed"))


# ---------------------------------------------------------------------------------------
# gather: block-table indexing, bit-exact
# ---------------------------------------------------------------------------------------

def check_gather(inp, seqs=None):
    d = Dev(inp, append=True)
    pool = oracle_pool(inp)
    for b in (range(inp.num_seqs) if seqs is None else seqs):
        L = int(inp.seq_lens[b])
        k = torch.empty((L, inp.num_kv_heads, inp.head_size), dtype=torch.float16, device="cuda")
        v = torch.empty_like(k)
        pkv.pa_gather_kv(k, v, d.pool, d.bt[b], L)
        K, V = oracle.gather_kv(pool, inp.block_tables[b], L)
        assert np.array_equal(bits(host(k)), bits(K)), b
        assert np.array_equal(bits(host(v)), bits(V)), b


def test_gather_tiny():
    check_gather(workloads.tiny_decode())


def test_gather_shared_and_mixed():
    check_gather(workloads.prefix_shared_case(35, 3, 4, 2, list(range(1, 13)), 8, 2, 64))
    check_gather(workloads.mixed_case(36, [0, 33], [17, 40], [2, 100], 4, 4, 128))


def test_gather_decode256_sampled():
    check_gather(cfg("decode256"), seqs=[0, 1, 77, 255])
    free()


# ---------------------------------------------------------------------------------------
# decode parity
# ---------------------------------------------------------------------------------------

def test_decode_tiny():
    inp = workloads.tiny_decode()
    got = Dev(inp).decode()
    ref = oracle_decode(inp)
    check_attention(got, ref, "tiny")
    # a context of one token returns that token's value row exactly
    v0 = inp.pool[inp.block_tables[0, 0], 0, 1]
    assert np.array_equal(bits(got[0]), bits(v0))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("ps", [16, 64, 512])
def test_decode_small(D, G, ps):
    lens = [1, 2, 15, 16, 17, 31, 33, 64, 100, 257, 511, 512, 513, 700]
    hkv = 4 if G < 8 else 2
    inp = workloads.decode_case(40 + D + G + ps, lens, hkv * G, hkv, D)
    note(f"decode D={D} G={G} partition={ps}")
    got = Dev(inp).decode(partition_size=ps)
    check_attention(got, oracle_decode(inp), f"D{D} G{G} ps{ps}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_past_64_blocks_per_partition(D, G):
    """Partitions of 128 and 256 blocks: each wave reloads its vector of table entries
    every 64 blocks. One partition per sequence (ps 4096) and 2048-token partitions."""
    lens = [1100, 1500, 2100, 17, 1024, 1025, 4096, 3000]
    hkv = 4 if G < 8 else 2
    inp = workloads.decode_case(70 + D + G, lens, hkv * G, hkv, D)
    ref = oracle_decode(inp)
    d = Dev(inp)
    for ps in (2048, 4096):
        for flags in (0, pkv.PA_DECODE_KV_STREAM):
            note(f"decode past 64 blocks D={D} G={G} ps={ps} flags={flags}")
            check_attention(d.decode(partition_size=ps, flags=flags), ref,
                            f"D{D} G{G} ps{ps} flags{flags}")


@pytest.mark.parametrize("G,D,n,ps", [(1, 128, 2, 512), (1, 64, 2, 512), (1, 128, 32, 16),
                                      (2, 64, 32, 16), (4, 128, 2, 512), (4, 128, 32, 16),
                                      (8, 128, 2, 512)])
def test_output_store_rounds_to_nearest_even(G, D, n, ps):
    """With q = 0 every weight is 1, so a row is the exact mean of its value rows, built
    here to lie exactly halfway between two fp16 numbers (n = 2 tokens, or 32 tokens over
    two 16-token partitions merged by the reduce kernel). The fp16 store must give the
    neighbour with the even last bit: truncation and rounding half away from zero each
    give a different result on some of these elements."""
    hkv = 2
    inp = workloads.decode_case(60 + G + D + n, [n] * 3, hkv * G, hkv, D, append=False)
    x, u = tie_base(np.random.default_rng(61 + G + n), (hkv, D))
    pool = inp.pool.copy()
    for b in range(3):
        write_tie_values(pool, inp.block_tables[b], n, x, u)
    case = dataclasses.replace(inp, pool=pool, q=np.zeros_like(inp.q))
    note(f"fp16 store rounding G={G} D={D} tokens={n} ps={ps}")
    got = Dev(case, append=False).decode(partition_size=ps)
    rne, toward0, away = tie_expectations(x, u)
    want = rne[np.arange(hkv * G) // G]  # query head h reads KV head h // G
    for b in range(3):
        assert np.array_equal(bits(got[b]), bits(want)), b
    assert (bits(rne) != bits(toward0)).any() and (bits(rne) != bits(away)).any()


def test_decode_on_a_side_stream():
    """The call's kernels on a stream other than the current one, with the workspace
    the binding allocates (recorded on that stream)."""
    inp = workloads.decode_case(48, [700, 1300, 2000, 33], 8, 8, 128)
    d = Dev(inp)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    q = d.q
    out = torch.empty_like(q)
    pkv.pa_decode(out, q, d.pool, d.bt, d.lens, 2000, inp.scale, 256, stream=side)
    # another allocation on the current stream while the call may still run on `side`
    scratch = torch.full((1 << 20,), 7, dtype=torch.uint8, device="cuda")
    torch.cuda.current_stream().wait_stream(side)
    check_attention(host(out), oracle_decode(inp), "side stream")
    del scratch


@pytest.mark.parametrize("hkv,G", [(3, 1), (5, 1), (3, 2), (5, 4), (6, 8)])
def test_decode_kv_heads_not_a_multiple_of_four(hkv, G):
    """A workgroup holds four KV heads of one (sequence, partition): with 3, 5 or 6 KV heads
    the last group is partly empty. One partition and several, ordered and not."""
    inp = workloads.decode_case(75 + hkv + G, [1, 17, 300, 700, 1200, 64], hkv * G, hkv, 128)
    ref = oracle_decode(inp)
    d = Dev(inp)
    for ps, flags in ((4096, 0), (256, 0), (256, pkv.PA_DECODE_KV_STREAM)):
        note(f"decode Hkv={hkv} G={G} ps={ps} flags={flags}")
        check_attention(d.decode(partition_size=ps, flags=flags), ref, f"Hkv{hkv} G{G} ps{ps}")


@pytest.mark.parametrize("G", [1, 4])
def test_decode_many_short_sequences_ordered(G):
    """5000 short sequences (more items than the GPU holds, up to five partitions each):
    the longest-first pre-pass sorts 25k items; every row against the oracle."""
    rng = np.random.default_rng(110 + G)
    lens = rng.integers(1, 300, 5000)
    inp = workloads.decode_case(110 + G, lens, 2 * G, 2, 64)
    ref = oracle_decode(inp)
    d = Dev(inp)
    for ps, flags in ((64, pkv.PA_DECODE_KV_STREAM), (64, 0), (512, pkv.PA_DECODE_KV_STREAM)):
        note(f"decode 5000 sequences G={G} ps={ps} flags={flags}")
        check_attention(d.decode(partition_size=ps, flags=flags), ref, f"5000 seqs G{G} ps{ps}")


def test_decode_length_one_rows_are_exact():
    inp = workloads.decode_case(41, [1] * 8, 16, 4, 128)
    got = Dev(inp).decode()
    # the single (appended) token's value row, per query head's KV head
    for b in range(8):
        for h in range(16):
            assert np.array_equal(bits(got[b, h]), bits(inp.value_new[b, h // 4]))


def bench_partition_size(inp):
    """The partition size bench.py runs a workload's decode with."""
    return pkv.pa_decode_default_partition_size(inp.num_seqs - inp.num_prefill, inp.num_q_heads,
                                                inp.num_kv_heads, int(inp.seq_lens.max()))


def test_decode_decode256_full():
    inp = cfg("decode256")
    d = Dev(inp)
    got = d.decode(partition_size=256)
    streamed = d.decode(partition_size=256, flags=pkv.PA_DECODE_KV_STREAM)
    # bench.py's launch: its default partition size, no block shared (longest first)
    ps = bench_partition_size(inp)
    as_bench = d.decode(partition_size=ps, flags=pkv.PA_DECODE_KV_STREAM)
    del d
    free()
    ref = oracle_decode(inp)
    check_attention(got, ref, "decode256")
    check_attention(as_bench, ref, f"decode256 as bench.py runs it (ps {ps})")
    # the cache hint changes no result bit
    assert np.array_equal(bits(got), bits(streamed))


def test_decode_long32k_full():
    """All 8 x 32 rows of the long-context workload, at the 512-token partitions it is
    specified with (64 partitions per sequence, merged by the reduce kernel) and at 2048
    tokens (16 partitions, the library's default size for it)."""
    inp = cfg("long32k")
    assert len(inp.slot_mapping) == 0  # cache pre-filled, nothing appended
    d = Dev(inp, append=False)
    sizes = (512, 2048)
    outs = {ps: d.decode(partition_size=ps, flags=pkv.PA_DECODE_KV_STREAM) for ps in sizes}
    del d
    free()
    note("oracle decode of long32k (8 x 32768 tokens x 32 heads)")
    ref = oracle.decode(inp.q, inp.pool, inp.block_tables, inp.seq_lens, inp.scale)
    for ps, got in outs.items():
        check_attention(got, ref, f"long32k ps{ps}")
    for ps in sizes:
        assert np.abs(outs[ps].astype(np.float64) - outs[512].astype(np.float64)).max() <= 1e-4


def test_decode_prefix_groups_full_and_shared_equals_private():
    inp = cfg("prefix-groups")
    got = Dev(inp).decode()
    free()
    check_attention(got, oracle_decode(inp), "prefix-groups")
    priv = workloads.unshare_prefix(inp)
    dp = Dev(priv)
    got2 = dp.decode()
    # the private-copy workload (c4p) as bench.py runs it: no block shared
    as_bench = dp.decode(partition_size=bench_partition_size(priv), flags=pkv.PA_DECODE_KV_STREAM)
    del dp
    free()
    assert np.array_equal(bits(got), bits(got2)), "shared prefix blocks change the output"
    check_attention(as_bench, oracle_decode(inp), "prefix-groups private copies as bench.py runs it")


def test_decode_mixed_decode_part():
    inp = cfg("mixed")
    d = Dev(inp)
    got = d.decode(partition_size=512)
    ps = bench_partition_size(inp)
    as_bench = d.decode(partition_size=ps, flags=pkv.PA_DECODE_KV_STREAM)
    del d
    free()
    ref = oracle_decode(inp)
    check_attention(got, ref, "mixed decode")
    check_attention(as_bench, ref, f"mixed decode as bench.py runs it (ps {ps})")


# ---------------------------------------------------------------------------------------
# invariants on the GPU
# ---------------------------------------------------------------------------------------

def test_decode_block_permutation_is_bit_identical():
    lens = np.random.default_rng(42).integers(100, 1500, 24)
    inp = workloads.decode_case(42, lens, 32, 32, 128)
    a = Dev(inp).decode()
    b = Dev(workloads.repermute(inp, 7)).decode()
    assert np.array_equal(bits(a), bits(b))


def test_decode_partition_sweep():
    lens = [1, 255, 256, 257, 511, 512, 513, 1023, 1024, 1025, 3000]
    inp = workloads.decode_case(43, lens, 8, 8, 128)
    ref = oracle_decode(inp)
    d = Dev(inp)
    outs = {ps: d.decode(partition_size=ps) for ps in (256, 512, 1024, 1 << 16)}
    for ps, got in outs.items():
        check_attention(got, ref, f"sweep ps{ps}")
    base = outs[1 << 16].astype(np.float64)
    for ps, got in outs.items():
        assert np.abs(got.astype(np.float64) - base).max() <= 1e-4, ps


def test_decode_max_context_bound_larger_than_lengths():
    inp = workloads.decode_case(44, [5, 40, 300], 4, 4, 64)
    got = Dev(inp).decode(max_context_len=4096)  # more partitions than any sequence has
    check_attention(got, oracle_decode(inp), "loose max_context_len")


def test_decode_zero_length_and_bad_rows():
    inp = workloads.decode_case(45, [0, 30, 600, 600, 20], 8, 4, 128, append=False)
    d = Dev(inp, append=False)
    lens = inp.seq_lens.copy()
    lens[4] = 10_000  # beyond max_context_len and the table: NaN row
    d.lens = dev(lens)
    bt = inp.block_tables.copy()
    bt[2, 20] = inp.num_blocks + 3  # outside the pool, in partition 1 of 3: NaN row
    bt[1, 0] = -1                    # outside the pool, single partition: NaN row
    d.bt = dev(bt)
    got = d.decode(partition_size=256, max_context_len=600).astype(np.float64)
    assert np.all(got[0] == 0)
    assert np.all(np.isnan(got[1])) and np.all(np.isnan(got[2])) and np.all(np.isnan(got[4]))
    ref = oracle.decode(inp.q, inp.pool, inp.block_tables, inp.seq_lens, inp.scale)
    check_attention(got[3:4], ref[3:4], "good row next to bad ones")


def _raw_decode_no_workspace(d, partition_size, flags):
    """pa_decode through the C ABI with no workspace (allowed with one partition)."""
    inp = d.inp
    out = torch.empty_like(d.q)
    nb, bs, _, hkv, D = d.pool.shape
    st = pkv.load().pa_decode(out.data_ptr(), d.q.data_ptr(), d.pool.data_ptr(), d.bt.data_ptr(),
                              d.lens.data_ptr(), d.q.shape[0], d.q.shape[1], hkv, D, bs,
                              d.bt.shape[1], nb, int(inp.seq_lens.max()), inp.scale,
                              partition_size, None, 0, flags, None)
    assert st == pkv.PA_OK, st
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("G", [1, 4])
def test_decode_longest_first_order_is_bit_identical(G):
    """PA_DECODE_KV_STREAM schedules the (sequence, partition) items longest first when they
    do not all fit on the GPU at once (1100 sequences x 8 KV heads = 8800 waves per
    partition, above the 8192 the smallest kernel keeps resident); results are those of
    launch order, with several partitions, one, and one without workspace."""
    rng = np.random.default_rng(46 + G)
    lens = rng.integers(1, 1000, 1100)
    lens[:3] = [0, 1, 16]
    inp = workloads.decode_case(46 + G, lens, 8 * G, 8, 64)
    pairs = list(zip(rng.integers(0, 1100, 300).tolist(), rng.integers(0, 8 * G, 300).tolist()))
    q, bt, ln = inp.decode_part()
    ref = oracle.decode_rows(q, oracle_pool(inp), bt, ln, inp.scale, pairs)
    d = Dev(inp)
    for ps in (256, 1024, 1 << 16):
        plain = d.decode(partition_size=ps)
        ordered = d.decode(partition_size=ps, flags=pkv.PA_DECODE_KV_STREAM)
        note(f"order G={G} ps={ps}")
        check_attention(np.stack([ordered[b, h] for b, h in pairs]), ref, f"ordered G{G} ps{ps}")
        assert np.array_equal(bits(plain), bits(ordered)), ps
    bare = _raw_decode_no_workspace(d, 1 << 16, pkv.PA_DECODE_KV_STREAM)
    assert np.array_equal(bits(bare), bits(plain))
    del d
    free()


@pytest.mark.parametrize("ps", [256, 1 << 16])
def test_decode_zero_length_and_bad_rows_ordered(ps):
    inp = workloads.decode_case(47, [0, 30, 600, 600, 20], 8, 4, 128, append=False)
    d = Dev(inp, append=False)
    lens = inp.seq_lens.copy()
    lens[4] = 10_000  # beyond max_context_len and the table: NaN row
    d.lens = dev(lens)
    bt = inp.block_tables.copy()
    bt[2, 20] = inp.num_blocks + 3  # outside the pool: NaN row
    bt[1, 0] = -1                    # outside the pool, first block: NaN row
    d.bt = dev(bt)
    got = d.decode(partition_size=ps, max_context_len=600,
                   flags=pkv.PA_DECODE_KV_STREAM).astype(np.float64)
    assert np.all(got[0] == 0)
    assert np.all(np.isnan(got[1])) and np.all(np.isnan(got[2])) and np.all(np.isnan(got[4]))
    ref = oracle.decode(inp.q, inp.pool, inp.block_tables, inp.seq_lens, inp.scale)
    check_attention(got[3:4], ref[3:4], "good row next to bad ones (ordered)")


def test_stream_read_runs():
    buf = torch.ones(1 << 24, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(pkv.pa_stream_read_sink_len(buf.numel()), dtype=torch.float32, device="cuda")
    pkv.pa_stream_read(buf, sink)
    assert np.isfinite(host(sink)).all()
