"""GPU parity of the MFMA chunked-prefill kernel against the CPU oracle (MI355X)."""

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


def gpu_prefill(inp, pool=None, bt=None, lens=None, qsl=None, max_q_len=None):
    """Append the batch's new tokens on the GPU, then run the prefill chunks."""
    pool_d = dev(inp.pool) if pool is None else pool
    if pool is None and len(inp.slot_mapping):
        pkv.pa_kv_append(pool_d, dev(inp.key_new), dev(inp.value_new), dev(inp.slot_mapping))
    q, bt_h, qsl_h, lens_h = inp.prefill_part()
    bt = dev(bt_h) if bt is None else bt
    lens = dev(lens_h) if lens is None else lens
    qsl = dev(qsl_h) if qsl is None else qsl
    qd = dev(q)
    out = torch.empty_like(qd)
    mq = int(np.diff(qsl_h).max()) if max_q_len is None else max_q_len
    pkv.pa_prefill_chunk(out, qd, pool_d, bt, qsl, lens, mq, int(lens_h.max()), inp.scale)
    return host(out), pool_d


def oracle_prefill(inp, rows=None):
    pool = oracle.kv_append(inp.pool, inp.key_new, inp.value_new, inp.slot_mapping)
    q, bt, qsl, lens = inp.prefill_part()
    return oracle.prefill_chunk(q, pool, bt, qsl, lens, inp.scale, rows=rows)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 4])
def test_prefill_small_ragged(D, G):
    priors = [0, 5, 100, 700, 31]
    chunks = [1, 17, 64, 130, 300]
    inp = workloads.mixed_case(50 + D + G, priors, chunks, [9], 4 * G, 4, D)
    note(f"prefill D={D} G={G}")
    got, _ = gpu_prefill(inp)
    check_attention(got, oracle_prefill(inp), f"prefill D{D} G{G}")


def test_prefill_pure_causal_chunks():
    inp = workloads.mixed_case(51, [0, 0, 0], [128, 129, 255], [], 8, 8, 128)
    got, _ = gpu_prefill(inp)
    check_attention(got, oracle_prefill(inp), "P=0 causal")


def test_prefill_long_prior():
    inp = workloads.mixed_case(52, [3584, 1000], [512, 77], [], 32, 8, 128)
    got, _ = gpu_prefill(inp)
    check_attention(got, oracle_prefill(inp), "long prior")


@functools.lru_cache(maxsize=1)
def mixed_workload():
    note("generating mixed")
    return workloads.mixed_prefill_decode()


def test_prefill_mixed_full():
    inp = mixed_workload()
    got, pool = gpu_prefill(inp)
    del pool
    torch.cuda.empty_cache()
    note("oracle prefill of mixed (4096 rows x 32 heads)")
    check_attention(got, oracle_prefill(inp), "mixed prefill")


def test_prefill_row_matches_decode_kernel():
    """Chunk row i and a decode query at position P+i over P+i+1 tokens give the same row."""
    inp = workloads.mixed_case(53, [40, 300], [64, 100], [], 8, 4, 128)
    got, pool = gpu_prefill(inp)
    q, bt, qsl, lens = inp.prefill_part()
    rows, qs, bts, ctx = [], [], [], []
    for r in range(2):
        P = int(lens[r]) - int(qsl[r + 1] - qsl[r])
        for i in (0, 1, 31, int(qsl[r + 1] - qsl[r]) - 1):
            rows.append(int(qsl[r]) + i)
            qs.append(q[int(qsl[r]) + i])
            bts.append(bt[r])
            ctx.append(P + i + 1)
    qd = dev(np.stack(qs))
    out = torch.empty_like(qd)
    pkv.pa_decode(out, qd, pool, dev(np.stack(bts)), dev(np.array(ctx, np.int32)), max(ctx),
                  inp.scale, 512)
    dec = host(out).astype(np.float64)
    assert np.abs(dec - got[rows].astype(np.float64)).max() <= 2e-3


def test_prefill_chunk_split_equals_whole():
    """A 512-row chunk equals the same rows run as two 256-row chunks over the same table."""
    inp = workloads.mixed_case(54, [900], [512], [], 8, 8, 128)
    whole, pool = gpu_prefill(inp)
    q, bt, qsl, lens = inp.prefill_part()
    S = int(lens[0])
    qsl2 = dev(np.array([0, 256, 512], np.int32))
    lens2 = dev(np.array([S - 256, S], np.int32))
    bt2 = dev(np.stack([bt[0], bt[0]]))
    out = torch.empty_like(dev(q))
    pkv.pa_prefill_chunk(out, dev(q), pool, bt2, qsl2, lens2, 256, S, inp.scale)
    split = host(out).astype(np.float64)
    assert np.abs(split - whole.astype(np.float64)).max() <= 2e-3
    check_attention(split, oracle_prefill(inp), "split chunk")


def test_prefill_bad_rows_are_nan():
    inp = workloads.mixed_case(55, [20, 50, 10], [30, 40, 20], [], 4, 4, 64)
    pool = dev(oracle.kv_append(inp.pool, inp.key_new, inp.value_new, inp.slot_mapping))
    q, bt, qsl, lens = inp.prefill_part()
    bt = bt.copy()
    bt[1, 2] = inp.num_blocks + 9   # request 1: a table entry outside the pool
    lens = lens.copy()
    lens[2] = 5                     # request 2: shorter than its chunk
    got, _ = gpu_prefill(inp, pool=pool, bt=dev(bt), lens=dev(lens))
    ref = oracle_prefill(inp)
    r0, r1, r2 = int(qsl[1]), int(qsl[2]), int(qsl[3])
    check_attention(got[:r0], ref[:r0], "good request")
    assert np.all(np.isnan(got[r0:r1].astype(np.float64)))
    assert np.all(np.isnan(got[r1:r2].astype(np.float64)))


# ---- split context: long contexts cut into pieces merged by log-sum-exp ----------------

def run_prefill(inp, pool, split, rows_hint=None, workspace=None):
    q, bt, qsl, lens = inp.prefill_part()
    qd = dev(q)
    out = torch.full_like(qd, float("nan"))
    pkv.pa_prefill_chunk(out, qd, pool, dev(bt), dev(qsl), dev(lens), int(np.diff(qsl).max()),
                         int(lens.max()), inp.scale, workspace=workspace, split=split)
    return host(out)


def appended_pool(inp):
    pool = dev(inp.pool)
    pkv.pa_kv_append(pool, dev(inp.key_new), dev(inp.value_new), dev(inp.slot_mapping))
    return pool


def workspace_bytes(inp):
    q, bt, qsl, lens = inp.prefill_part()
    return pkv.pa_prefill_workspace_bytes(len(lens), inp.num_q_heads, int(np.diff(qsl).max()),
                                          int(lens.max()), inp.head_size)


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_split_matches_unsplit_and_oracle(D):
    """Requests with long priors next to short ones: the split launch agrees with the
    oracle and with the unsplit launch (fp32 sums in another order: within 2e-3)."""
    inp = workloads.mixed_case(56 + D, [6000, 2100, 0, 700], [256, 300, 100, 17], [], 16, 4, D)
    assert workspace_bytes(inp) > 0  # the split is taken at these sizes
    pool = appended_pool(inp)
    note(f"prefill split D={D}")
    split = run_prefill(inp, pool, True)
    whole = run_prefill(inp, pool, False)
    rows = np.arange(0, split.shape[0], 3)
    check_attention(split[rows], oracle_prefill(inp, rows=set(rows.tolist()))[rows], f"split D{D}")
    assert np.abs(split.astype(np.float64) - whole.astype(np.float64)).max() <= 2e-3


def test_prefill_split_single_long_request():
    """One 512-row chunk after 15872 cached tokens: 32 row tiles for the whole GPU, so the
    context is cut into the most pieces; sampled rows against the oracle."""
    inp = workloads.mixed_case(57, [15872], [512], [], 8, 8, 128)
    assert workspace_bytes(inp) > 0
    pool = appended_pool(inp)
    note("prefill split, one 16k request")
    got = run_prefill(inp, pool, True)
    rows = np.concatenate([np.arange(0, 512, 37), [127, 128, 255, 256, 511]])
    check_attention(got[rows], oracle_prefill(inp, rows=set(rows.tolist()))[rows], "16k request")
    whole = run_prefill(inp, pool, False)
    assert np.abs(got.astype(np.float64) - whole.astype(np.float64)).max() <= 2e-3


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("prior,chunk", [(20, 1100), (100, 1500), (1000, 1500), (300, 2000)])
def test_prefill_split_piece_boundary_inside_a_wave(D, prior, chunk):
    """Priors that are not a multiple of 32 put a piece's first token inside one wave's 32
    rows, so some rows of that wave see none of the piece while the others do (those rows'
    maxima stay at -inf while the wave rescales): every row against the oracle, no NaN."""
    inp = workloads.mixed_case(62 + prior + D, [prior], [chunk], [], 2, 1, D)
    assert workspace_bytes(inp) > 0
    pool = appended_pool(inp)
    note(f"prefill split, piece boundary inside a wave: D={D} P={prior} C={chunk}")
    got = run_prefill(inp, pool, True)
    check_attention(got, oracle_prefill(inp), f"split boundary D{D} P{prior}")
    whole = run_prefill(inp, pool, False)
    assert np.abs(got.astype(np.float64) - whole.astype(np.float64)).max() <= 2e-3


def test_prefill_split_bad_entry_in_late_piece_is_nan():
    inp = workloads.mixed_case(58, [9000, 3000], [200, 64], [], 8, 8, 128)
    assert workspace_bytes(inp) > 0
    pool = appended_pool(inp)
    q, bt, qsl, lens = inp.prefill_part()
    bt = bt.copy()
    bt[0, 500] = inp.num_blocks + 3  # token 8000 of request 0: in its last pieces
    out = torch.full_like(dev(q), 0.0)
    pkv.pa_prefill_chunk(out, dev(q), pool, dev(bt), dev(qsl), dev(lens),
                         int(np.diff(qsl).max()), int(lens.max()), inp.scale)
    got = host(out).astype(np.float64)
    r0 = int(qsl[1])
    assert np.all(np.isnan(got[:r0]))
    rows = np.arange(r0, got.shape[0], 5)
    check_attention(got[rows], oracle_prefill(inp, rows=set(rows.tolist()))[rows], "good request")


def test_prefill_split_workspace_too_small():
    inp = workloads.mixed_case(59, [4000], [128], [], 8, 8, 128)
    need = workspace_bytes(inp)
    assert need > 0
    pool = appended_pool(inp)
    small = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(pkv.PagedKVError):
        run_prefill(inp, pool, True, workspace=small)
    ok = torch.empty(need, dtype=torch.uint8, device="cuda")
    got = run_prefill(inp, pool, True, workspace=ok)
    # a second call into the same workspace with a shorter chunk
    inp2 = workloads.mixed_case(60, [2500], [40], [], 8, 8, 128)
    assert workspace_bytes(inp2) <= need
    got2 = run_prefill(inp2, appended_pool(inp2), True, workspace=ok)
    rows = np.arange(0, 128, 9)
    check_attention(got[rows], oracle_prefill(inp, rows=set(rows.tolist()))[rows], "first call")
    check_attention(got2, oracle_prefill(inp2), "second call")


def test_prefill_long_prompt_workload_sampled():
    """The long-prompt workload at full size, in the bench's configuration (the step's
    append, then the split prefill): sampled rows of every row tile against the oracle."""
    inp = workloads.long_prompt_prefill()
    assert workspace_bytes(inp) > 0
    note("long-prompt workload: append + split prefill")
    got, pool = gpu_prefill(inp)
    del pool
    torch.cuda.empty_cache()
    rows = np.concatenate([np.arange(0, 512, 23), [127, 128, 383, 384, 511]])
    check_attention(got[rows], oracle_prefill(inp, rows=set(rows.tolist()))[rows], "long prompt")


def test_prefill_many_requests_launch_order():
    """300 short requests (above the 256 that are ranked by length): launch order, no
    split; every row against the oracle."""
    rng = np.random.default_rng(61)
    priors = rng.integers(0, 200, size=300).tolist()
    chunks = rng.integers(1, 6, size=300).tolist()
    inp = workloads.mixed_case(61, priors, chunks, [], 4, 4, 64)
    assert workspace_bytes(inp) == 0
    got, _ = gpu_prefill(inp)
    check_attention(got, oracle_prefill(inp), "300 requests")


@pytest.mark.parametrize("split", [True, False])
def test_prefill_zero_length_chunk_among_others(split):
    """A request with no query rows this step (an empty chunk between two others, its
    context still cached): its neighbours are unaffected and nothing is written for it,
    with and without the context split."""
    inp = workloads.mixed_case(62, [3000, 1200, 2500], [100, 1, 70], [], 8, 8, 128)
    q, bt, qsl, lens = inp.prefill_part()
    pool = appended_pool(inp)
    # request 1 keeps its 1201 cached tokens but asks for no rows
    qsl0 = qsl.copy()
    qsl0[2:] -= 1
    lens0 = lens.copy()
    lens0[1] -= 1
    keep = np.r_[0:int(qsl[1]), int(qsl[2]):int(qsl[3])]
    qd = dev(np.ascontiguousarray(q[keep]))
    out = torch.full_like(qd, float("nan"))
    pkv.pa_prefill_chunk(out, qd, pool, dev(bt), dev(qsl0), dev(lens0),
                         int(np.diff(qsl0).max()), int(lens0.max()), inp.scale, split=split)
    got = host(out)
    ref = oracle.prefill_chunk(q[keep], oracle.kv_append(inp.pool, inp.key_new, inp.value_new,
                                                         inp.slot_mapping),
                               bt, qsl0, lens0, inp.scale)
    check_attention(got, ref, f"empty chunk split={split}")


def test_prefill_2048_row_chunk():
    """One 2048-row chunk (16 row tiles) after 2000 cached tokens next to a short request;
    sampled rows of every tile against the oracle."""
    inp = workloads.mixed_case(63, [2000, 10], [2048, 40], [], 8, 4, 128)
    note("prefill 2048-row chunk")
    got, _ = gpu_prefill(inp)
    rows = np.concatenate([np.arange(0, 2088, 29), [127, 128, 1023, 1024, 2047, 2048, 2087]])
    check_attention(got[rows], oracle_prefill(inp, rows=set(rows.tolist()))[rows], "2048 rows")


@pytest.mark.parametrize("G,D", [(1, 128), (4, 128), (1, 64)])
def test_output_store_rounds_to_nearest_even(G, D):
    """q = 0 makes a chunk row the exact mean of the value rows it sees. Request 0 (no
    prior, chunk of 2): row 1 sees 2 tokens; request 1 (31 prior tokens, chunk of 1): its
    row sees 32. Both means lie halfway between two fp16 numbers, and the store must give
    the neighbour with the even last bit; row 0 of request 0 sees one token, its value."""
    hkv = 2
    inp = workloads.mixed_case(230 + G + D, [0, 31], [2, 1], [], hkv * G, hkv, D)
    pool = oracle.kv_append(inp.pool, inp.key_new, inp.value_new, inp.slot_mapping)
    x, u = tie_base(np.random.default_rng(231), (hkv, D))
    write_tie_values(pool, inp.block_tables[0], 2, x, u)
    write_tie_values(pool, inp.block_tables[1], 32, x, u)
    q, bt, qsl, lens = inp.prefill_part()
    out = torch.empty(q.shape, dtype=torch.float16, device="cuda")
    note(f"prefill fp16 store rounding G={G} D={D}")
    pkv.pa_prefill_chunk(out, dev(np.zeros_like(q)), dev(pool), dev(bt), dev(qsl), dev(lens), 2,
                         32, inp.scale)
    got = host(out)
    rne, toward0, away = tie_expectations(x, u)
    kv = np.arange(hkv * G) // G
    assert np.array_equal(bits(got[0]), bits((x + u).astype(np.float16)[kv]))
    assert np.array_equal(bits(got[1]), bits(rne[kv]))
    assert np.array_equal(bits(got[2]), bits(rne[kv]))
    assert (bits(rne) != bits(toward0)).any() and (bits(rne) != bits(away)).any()
