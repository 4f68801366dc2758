"""A step captured into a HIP graph (StepGraph) replays to exactly the eager step's bits.

The step is kv_append -> chunked prefill (its context split, so the merge kernel runs
too) -> decode (grouped-query tile, several partitions, so the log-sum-exp reduce runs
too). Replays are separated by eager work
and host synchronisations, and the queries are changed in place between them. The same
for the step over an E4M3 pool, for shared-prefix decode, and for pa_decode_noalloc (its
fixed scratch rewritten by an eager call before each replay); and for one step replayed
while the batch in its buffers changes (lengths, start offsets, tables and pool)."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_294_amd as pkv
import workloads
from gpu_util import check_attention, dev, host, note

pytestmark = pytest.mark.gpu


class Batch:
    def __init__(self, inp, partition_size=512):
        self.inp = inp
        self.pool = dev(inp.pool)
        self.key, self.value, self.slots = dev(inp.key_new), dev(inp.value_new), dev(inp.slot_mapping)
        qd, btd, lensd = inp.decode_part()
        self.dq, self.dbt, self.dlens = dev(qd), dev(btd), dev(lensd)
        self.mcl = int(lensd.max())
        self.ps = partition_size
        ws = pkv.pa_decode_workspace_bytes(len(lensd), inp.num_q_heads, self.mcl, partition_size,
                                           inp.head_size)
        assert ws > 0  # several partitions: the reduce kernel is part of the step
        self.ws = torch.empty(ws, dtype=torch.uint8, device="cuda")
        qp, btp, qsl, lensp = inp.prefill_part()
        self.pq, self.pbt, self.qsl, self.plens = dev(qp), dev(btp), dev(qsl), dev(lensp)
        self.max_q, self.max_s = int(np.diff(qsl).max()), int(lensp.max())
        pws = pkv.pa_prefill_workspace_bytes(len(lensp), inp.num_q_heads, self.max_q, self.max_s,
                                             inp.head_size)
        assert pws > 0  # the prefill's context split and merge kernel are part of the step
        self.pws = torch.empty(pws, dtype=torch.uint8, device="cuda")
        self.dout = torch.full_like(self.dq, float("nan"))
        self.pout = torch.full_like(self.pq, float("nan"))

    def step(self, stream):
        pkv.pa_kv_append(self.pool, self.key, self.value, self.slots, stream=stream)
        pkv.pa_prefill_chunk(self.pout, self.pq, self.pool, self.pbt, self.qsl, self.plens,
                             self.max_q, self.max_s, self.inp.scale, workspace=self.pws,
                             stream=stream)
        pkv.pa_decode(self.dout, self.dq, self.pool, self.dbt, self.dlens, self.mcl,
                      self.inp.scale, self.ps, self.ws, stream=stream)


def test_captured_step_replays_bit_exact():
    inp = workloads.mixed_case(71, [0, 1500, 40], [64, 100, 33], [1, 50, 700, 2000, 1100], 8, 4, 128)
    side = torch.cuda.Stream()
    b = Batch(inp)
    note("graph: eager reference step")
    with torch.cuda.stream(side):
        b.step(side)
    side.synchronize()
    ref_d, ref_p = b.dout.clone(), b.pout.clone()
    # the eager step itself against the oracle
    pool = oracle.kv_append(inp.pool, inp.key_new, inp.value_new, inp.slot_mapping)
    qd, btd, lensd = inp.decode_part()
    check_attention(host(ref_d), oracle.decode(qd, pool, btd, lensd, inp.scale), "graph eager decode")

    q2_d = torch.randn(b.dq.shape, generator=torch.Generator().manual_seed(5)).half().cuda()
    q2_p = torch.randn(b.pq.shape, generator=torch.Generator().manual_seed(6)).half().cuda()
    b2 = Batch(inp)
    b2.dq.copy_(q2_d)
    b2.pq.copy_(q2_p)
    with torch.cuda.stream(side):
        b2.step(side)
    side.synchronize()
    ref2_d, ref2_p = b2.dout.clone(), b2.pout.clone()

    note("graph: capture")
    g = pkv.StepGraph(side)
    b.dout.fill_(float("nan"))
    b.pout.fill_(float("nan"))
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        with g:
            b.step(side)
    torch.cuda.synchronize()
    # captured, not run
    assert torch.isnan(b.dout.float()).all() and torch.isnan(b.pout.float()).all()
    try:
        for rep, (q_d, q_p, want_d, want_p) in enumerate([
                (None, None, ref_d, ref_p), (q2_d, q2_p, ref2_d, ref2_p), (None, None, ref2_d, ref2_p)]):
            note(f"graph: replay {rep}")
            b.dout.fill_(float("nan"))
            b.pout.fill_(float("nan"))
            if q_d is not None:
                b.dq.copy_(q_d)
                b.pq.copy_(q_p)
            torch.cuda.synchronize()
            g.launch()
            side.synchronize()
            assert torch.equal(b.dout.view(torch.int16), want_d.view(torch.int16)), f"decode replay {rep}"
            assert torch.equal(b.pout.view(torch.int16), want_p.view(torch.int16)), f"prefill replay {rep}"
            _ = (b.dout.float().sum() + 1).item()  # eager work between replays
    finally:
        g.close()


def test_capture_needs_caller_workspace():
    inp = workloads.decode_case(72, [600, 1500], 4, 4, 64)
    side = torch.cuda.Stream()
    q, bt, lens = (dev(a) for a in inp.decode_part())
    pool = dev(inp.pool)
    out = torch.empty_like(q)
    g = pkv.StepGraph(side)
    with pytest.raises(ValueError):
        with torch.cuda.stream(side):
            with g:
                pkv.pa_decode(out, q, pool, bt, lens, 1500, inp.scale, 512, None, stream=side)
    side.synchronize()
    g.close()


def test_captured_noalloc_decode_replays_bit_exact():
    """pa_decode_noalloc (the library's fixed scratch, no allocation) captured into a graph:
    several partitions (so the reduce kernel runs) and PA_DECODE_KV_STREAM (so the
    longest-first order pre-pass runs). Before each replay an eager call on another batch
    rewrites the scratch; every replay still equals pa_decode with a caller workspace,
    before and after the queries change in place."""
    rng = np.random.default_rng(73)
    inp = workloads.decode_case(73, rng.integers(1, 1500, 600), 8, 8, 64)
    other = workloads.decode_case(74, [900, 33, 1400], 8, 8, 64, append=False)
    q, bt, lens = (dev(a) for a in inp.decode_part())
    pool = dev(inp.pool)
    pkv.pa_kv_append(pool, dev(inp.key_new), dev(inp.value_new), dev(inp.slot_mapping))
    mcl = int(inp.seq_lens.max())
    ps, flags = 256, pkv.PA_DECODE_KV_STREAM
    assert pkv.pa_decode_workspace_bytes(600, 8, mcl, ps, 64) <= pkv.PA_DECODE_NOALLOC_SCRATCH_BYTES

    def reference(qq):
        want = torch.empty_like(qq)
        pkv.pa_decode(want, qq, pool, bt, lens, mcl, inp.scale, ps, flags=flags)
        torch.cuda.synchronize()
        return want

    q2 = torch.randn(q.shape, generator=torch.Generator().manual_seed(7)).half().cuda()
    want1, want2 = reference(q), reference(q2)
    oq, obt, olens = (dev(a) for a in other.decode_part())
    opool = dev(other.pool)
    oout = torch.empty_like(oq)

    side = torch.cuda.Stream()
    out = torch.full_like(q, float("nan"))
    g = pkv.StepGraph(side)
    torch.cuda.synchronize()
    note("graph: capture pa_decode_noalloc")
    with torch.cuda.stream(side):
        with g:
            pkv.pa_decode_noalloc(out, q, pool, bt, lens, mcl, inp.scale, ps, flags, stream=side)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()  # captured, not run
    q1 = q.clone()
    try:
        for rep, (qq, want) in enumerate([(q1, want1), (q2, want2), (q1, want1)]):
            q.copy_(qq)
            out.fill_(float("nan"))
            # another batch through the same scratch, eagerly, before the replay
            pkv.pa_decode_noalloc(oout, oq, opool, obt, olens, 1400, other.scale, 128)
            torch.cuda.synchronize()
            note(f"graph: noalloc replay {rep}")
            g.launch()
            side.synchronize()
            assert torch.equal(out.view(torch.int16), want.view(torch.int16)), rep
    finally:
        g.close()
    check_attention(host(out), oracle.decode(inp.q, oracle.kv_append(inp.pool, inp.key_new,
                                                                       inp.value_new, inp.slot_mapping),
                                             inp.block_tables, inp.seq_lens, inp.scale),
                    "noalloc graph replay")


def test_captured_fp8_step_replays_bit_exact():
    """The same step over an E4M3 pool (quantizing append, prefill with its context split,
    decode over several partitions) captured and replayed: every replay equals the eager
    step bit for bit, and the eager step matches the oracle on the dequantized pool."""
    from oracle import fp8
    ks, vs = 0.03, 0.02
    inp = workloads.mixed_case(76, [0, 1500, 40], [64, 100, 33], [1, 50, 700, 2000, 1100], 8, 4, 128)
    pool_u8 = np.concatenate([fp8.quantize(inp.pool[:, :, 0:1], ks),
                              fp8.quantize(inp.pool[:, :, 1:2], vs)], axis=2)
    key, value, slots = dev(inp.key_new), dev(inp.value_new), dev(inp.slot_mapping)
    qd, btd, lensd = inp.decode_part()
    dq, dbt, dlens = dev(qd), dev(btd), dev(lensd)
    qp, btp, qsl, lensp = inp.prefill_part()
    pq, pbt, pqsl, plens = dev(qp), dev(btp), dev(qsl), dev(lensp)
    mcl, max_q, max_s = int(lensd.max()), int(np.diff(qsl).max()), int(lensp.max())
    ws = torch.empty(pkv.pa_decode_workspace_bytes(len(lensd), 8, mcl, 512, 128), dtype=torch.uint8,
                     device="cuda")
    pws_n = pkv.pa_prefill_workspace_bytes(len(lensp), 8, max_q, max_s, 128)
    assert pws_n > 0
    pws = torch.empty(pws_n, dtype=torch.uint8, device="cuda")
    pool = dev(pool_u8)
    dout = torch.full_like(dq, float("nan"))
    pout = torch.full_like(pq, float("nan"))

    def step(stream):
        pkv.pa_kv_append_fp8(pool, key, value, slots, ks, vs, stream=stream)
        pkv.pa_prefill_chunk_fp8(pout, pq, pool, pbt, pqsl, plens, max_q, max_s, inp.scale, ks, vs,
                                 workspace=pws, stream=stream)
        pkv.pa_decode_fp8(dout, dq, pool, dbt, dlens, mcl, inp.scale, ks, vs, 512, ws, stream=stream)

    side = torch.cuda.Stream()
    note("graph fp8: eager step")
    with torch.cuda.stream(side):
        step(side)
    side.synchronize()
    ref_d, ref_p = dout.clone(), pout.clone()
    want_pool = fp8.kv_append_fp8(pool_u8, inp.key_new, inp.value_new, inp.slot_mapping, ks, vs)
    assert np.array_equal(host(pool), want_pool)
    vals = fp8.dequantize_pool(want_pool, ks, vs)
    check_attention(host(ref_d), oracle.decode(qd, vals, btd, lensd, inp.scale), "graph fp8 eager decode")
    check_attention(host(ref_p), oracle.prefill_chunk(qp, vals, btp, qsl, lensp, inp.scale),
                    "graph fp8 eager prefill")

    g = pkv.StepGraph(side)
    dout.fill_(float("nan"))
    pout.fill_(float("nan"))
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        with g:
            step(side)
    torch.cuda.synchronize()
    assert torch.isnan(dout.float()).all() and torch.isnan(pout.float()).all()
    try:
        for rep in range(3):
            note(f"graph fp8: replay {rep}")
            dout.fill_(float("nan"))
            pout.fill_(float("nan"))
            pool.copy_(dev(pool_u8))  # the append rewrites the same slots each replay
            torch.cuda.synchronize()
            g.launch()
            side.synchronize()
            assert torch.equal(dout.view(torch.int16), ref_d.view(torch.int16)), f"decode replay {rep}"
            assert torch.equal(pout.view(torch.int16), ref_p.view(torch.int16)), f"prefill replay {rep}"
            _ = (dout.float().sum() + 1).item()  # eager work between replays
    finally:
        g.close()


def test_captured_shared_prefix_decode_replays_bit_exact():
    """Shared-prefix decode (prefix pass, own-token pass and the cascade reduce) captured
    and replayed, with the queries changed in place between replays."""
    rng = np.random.default_rng(77)
    priv = rng.integers(0, 70, 24)
    inp = workloads.prefix_shared_case(77, 3, 8, 4, priv, 16, 4, 128)
    q, bt, L = inp.decode_part()
    dq, dbt, dL, pool = dev(q), dev(bt), dev(L), dev(inp.pool)
    gs = dev(np.array([0, 8, 16, 24], np.int32))
    pl = dev(np.array([64, 64, 64], np.int32))
    mcl = int(L.max())
    ws = torch.empty(pkv.pa_decode_shared_prefix_workspace_bytes(24, 16, mcl, 64, 32, 128),
                     dtype=torch.uint8, device="cuda")
    out = torch.full_like(dq, float("nan"))

    def call(stream):
        pkv.pa_decode_shared_prefix(out, dq, pool, dbt, dL, mcl, gs, pl, 8, 64, inp.scale, 32,
                                    workspace=ws, stream=stream)

    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        call(side)
    side.synchronize()
    ref1 = out.clone()
    check_attention(host(ref1), oracle.decode(q, inp.pool, bt, L, inp.scale), "graph shared eager")
    q1 = dq.clone()
    q2 = torch.randn(dq.shape, generator=torch.Generator().manual_seed(8)).half().cuda()
    dq.copy_(q2)
    with torch.cuda.stream(side):
        call(side)
    side.synchronize()
    ref2 = out.clone()

    g = pkv.StepGraph(side)
    out.fill_(float("nan"))
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        with g:
            call(side)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
    try:
        for rep, (qq, want) in enumerate([(q1, ref1), (q2, ref2), (q1, ref1)]):
            note(f"graph shared: replay {rep}")
            dq.copy_(qq)
            out.fill_(float("nan"))
            torch.cuda.synchronize()
            g.launch()
            side.synchronize()
            assert torch.equal(out.view(torch.int16), want.view(torch.int16)), rep
            _ = (out.float().sum() + 1).item()
    finally:
        g.close()


def test_replays_follow_changed_lengths_and_tables():
    """A serving loop replays one captured step while the batch changes: the host bounds
    (max_context_len, max_q_len, max_seq_len) stay, the device lengths, start offsets and
    tables change between replays. The decode's longest-first order and the prefill's
    context-split plan are derived on the device from the new contents, so every replay
    must equal an eager call on the same contents."""
    big = workloads.mixed_case(78, [0, 1500, 40], [64, 100, 33], [1, 50, 700, 2000, 1100], 8, 4, 128)
    small = workloads.mixed_case(79, [900, 20, 5], [33, 64, 100], [1600, 3, 1999, 40, 512], 8, 4, 128)
    side = torch.cuda.Stream()
    b = Batch(big)
    # the second batch's metadata, padded to the first one's table width and pool
    qd, btd, lensd = small.decode_part()
    qp, btp, qsl, lensp = small.prefill_part()
    assert btd.shape[1] <= b.dbt.shape[1] and btp.shape[1] <= b.pbt.shape[1]
    assert int(lensd.max()) <= b.mcl and int(np.diff(qsl).max()) <= b.max_q and int(lensp.max()) <= b.max_s
    assert qd.shape == tuple(b.dq.shape) and qp.shape == tuple(b.pq.shape)

    def pad(t, width):
        out = np.full((t.shape[0], width), int(t[0, -1]), np.int32)
        out[:, :t.shape[1]] = t
        return out

    meta2 = dict(dq=dev(qd), dbt=dev(pad(btd, b.dbt.shape[1])), dlens=dev(lensd), pq=dev(qp),
                 pbt=dev(pad(btp, b.pbt.shape[1])), qsl=dev(qsl), plens=dev(lensp))
    meta1 = {k: getattr(b, k).clone() for k in meta2}
    # the second batch's pool inside one of the first one's size (its blocks first, NaN after)
    pool2 = torch.full_like(b.pool, float("nan"))
    assert small.pool.shape[0] <= pool2.shape[0]
    pool2[: small.pool.shape[0]] = dev(small.pool)
    pkv.pa_kv_append(pool2, dev(small.key_new), dev(small.value_new), dev(small.slot_mapping))
    pool1 = b.pool.clone()
    pkv.pa_kv_append(pool1, b.key, b.value, b.slots)

    def eager(meta, pool):
        dout = torch.empty_like(b.dout)
        pout = torch.empty_like(b.pout)
        pkv.pa_prefill_chunk(pout, meta["pq"], pool, meta["pbt"], meta["qsl"], meta["plens"], b.max_q,
                             b.max_s, big.scale, workspace=torch.empty_like(b.pws))
        pkv.pa_decode(dout, meta["dq"], pool, meta["dbt"], meta["dlens"], b.mcl, big.scale, b.ps,
                      torch.empty_like(b.ws), flags=pkv.PA_DECODE_KV_STREAM)
        torch.cuda.synchronize()
        return dout, pout

    want = [eager(meta1, pool1), eager(meta2, pool2)]
    # the step without the append (each pool already holds its batch's tokens)
    work = b.pool

    def step(stream):
        pkv.pa_prefill_chunk(b.pout, b.pq, work, b.pbt, b.qsl, b.plens, b.max_q, b.max_s, big.scale,
                             workspace=b.pws, stream=stream)
        pkv.pa_decode(b.dout, b.dq, work, b.dbt, b.dlens, b.mcl, big.scale, b.ps, b.ws,
                      flags=pkv.PA_DECODE_KV_STREAM, stream=stream)

    g = pkv.StepGraph(side)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        with g:
            step(side)
    torch.cuda.synchronize()
    try:
        for rep, k in enumerate([0, 1, 0, 1]):
            meta, pool = (meta1, pool1) if k == 0 else (meta2, pool2)
            for name, t in meta.items():
                getattr(b, name).copy_(t)
            work.copy_(pool)
            b.dout.fill_(float("nan"))
            b.pout.fill_(float("nan"))
            torch.cuda.synchronize()
            note(f"graph: replay {rep} with batch {k}")
            g.launch()
            side.synchronize()
            assert torch.equal(b.dout.view(torch.int16), want[k][0].view(torch.int16)), rep
            assert torch.equal(b.pout.view(torch.int16), want[k][1].view(torch.int16)), rep
    finally:
        g.close()
    # and the second batch's replay output against the oracle
    vals = oracle.kv_append(small.pool, small.key_new, small.value_new, small.slot_mapping)
    check_attention(host(want[1][0]), oracle.decode(qd, vals, btd, lensd, small.scale), "graph batch 2 decode")
    check_attention(host(want[1][1]), oracle.prefill_chunk(qp, vals, btp, qsl, lensp, small.scale),
                    "graph batch 2 prefill")
