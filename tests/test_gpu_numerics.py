"""Numerically hard inputs against the oracle: scores spread over hundreds of log2 units
(queries scaled up), and keys whose scores climb along the context by about 4 log2 units
per block, so that the running maximum keeps moving (the lazy rescale of the GQA decode
and the prefill, which waits for 8 units, fires every other block). Decode (MHA and
grouped query), prefill (split and not) and shared-prefix decode, each to the usual bar."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_294_amd as pkv
import workloads
from gpu_util import check_attention, dev, host, note

pytestmark = pytest.mark.gpu


def ramp_keys(inp, seqs, rate):
    """Key dim 0 of every head = rate * (logical position) / 64 for the given sequences'
    contexts (their blocks are their own); with query dim 0 = 4 the scores grow by
    rate / 16 * scale per token along the context."""
    pool = inp.pool.copy()
    for b in seqs:
        L = int(inp.seq_lens[b])
        for t in range(L):
            phys = int(inp.block_tables[b, t // 16])
            pool[phys, t % 16, 0, :, 0] = np.float16(rate * t / 64.0)
    return pool


@pytest.mark.parametrize("G", [1, 4])
@pytest.mark.parametrize("qscale", [30.0, 1.0])
def test_decode_extreme_scores(G, qscale):
    lens = [1, 17, 300, 1024, 2049, 700]
    inp = workloads.decode_case(90 + G, lens, 4 * G, 4, 128, append=False)
    q = inp.q.astype(np.float32) * qscale
    q[:, :, 0] = 4.0
    q = q.astype(np.float16)
    pool = ramp_keys(inp, range(len(lens)), 30.0) if qscale == 1.0 else inp.pool
    _, bt, L = inp.decode_part()
    ref = oracle.decode(q, pool, bt, L, inp.scale)
    for ps, flags in ((4096, 0), (256, pkv.PA_DECODE_KV_STREAM)):
        note(f"decode extreme G={G} qscale={qscale} ps={ps}")
        out = torch.full(q.shape, float("nan"), dtype=torch.float16, device="cuda")
        pkv.pa_decode(out, dev(q), dev(pool), dev(bt), dev(L), int(L.max()), inp.scale, ps, flags=flags)
        check_attention(host(out), ref, f"decode extreme G{G} q{qscale} ps{ps}")


@pytest.mark.parametrize("split", [False, True])
def test_prefill_extreme_scores(split):
    inp = workloads.mixed_case(95, [20, 1500], [1100, 300], [], 4, 2, 128)
    pool = oracle.kv_append(inp.pool, inp.key_new, inp.value_new, inp.slot_mapping)
    # climbing keys over each request's whole context (its blocks are its own)
    for r in range(2):
        for t in range(int(inp.seq_lens[r])):
            pool[int(inp.block_tables[r, t // 16]), t % 16, 0, :, 0] = np.float16(30.0 * t / 64.0)
    q, bt, qsl, lens = inp.prefill_part()
    q = q.astype(np.float32)
    q[:, :, 0] = 4.0
    q = q.astype(np.float16)
    note(f"prefill extreme split={split}")
    out = torch.full(q.shape, float("nan"), dtype=torch.float16, device="cuda")
    pkv.pa_prefill_chunk(out, dev(q), dev(pool), dev(bt), dev(qsl), dev(lens), int(np.diff(qsl).max()),
                         int(lens.max()), inp.scale, split=split)
    check_attention(host(out), oracle.prefill_chunk(q, pool, bt, qsl, lens, inp.scale),
                    f"prefill extreme split={split}")


def test_shared_prefix_extreme_scores():
    rng = np.random.default_rng(96)
    priv = rng.integers(0, 90, 12)
    inp = workloads.prefix_shared_case(96, 3, 4, 5, priv, 16, 4, 128)
    q, bt, L = inp.decode_part()
    q = (q.astype(np.float32) * 30.0).astype(np.float16)
    gs, pl = np.array([0, 4, 8, 12], np.int32), np.array([80, 80, 80], np.int32)
    ref = oracle.decode(q, inp.pool, bt, L, inp.scale)
    for ps in (16, 256):
        note(f"shared prefix extreme ps={ps}")
        out = torch.full(q.shape, float("nan"), dtype=torch.float16, device="cuda")
        pkv.pa_decode_shared_prefix(out, dev(q), dev(inp.pool), dev(bt), dev(L), int(L.max()), dev(gs),
                                    dev(pl), 4, 80, inp.scale, ps)
        check_attention(host(out), ref, f"shared extreme ps{ps}")
