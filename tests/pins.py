"""Checks that pin the CPU oracle to facts outside itself.

Each ``check_*`` raises AssertionError when the oracle disagrees with a value the
pages fix, a closed form, a library routine or a brute-force computation. The
tests call them on the oracle as written, and again with a mistake planted in
the oracle to show that the check notices it.
"""

from __future__ import annotations

import math
import os

import numpy as np
import torch

import oracle
from oracle import paged_attention as opa
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------------------
# golden fixtures from the pages
# ---------------------------------------------------------------------------------------

def read_block_table_figure():
    info, rows = {}, []
    with open(os.path.join(GOLDEN, "block_table_figure.txt"), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] in ("block_size", "num_tokens", "blocks_needed"):
                info[parts[0]] = int(parts[1])
            elif parts[0] == "table":
                info["table"] = [int(x) for x in parts[1:]]
            else:
                rows.append(tuple(int(x) for x in parts))
    return info, rows


def check_block_table_figure():
    info, rows = read_block_table_figure()
    bs = info["block_size"]
    assert opa.blocks_needed(info["num_tokens"], bs) == info["blocks_needed"]
    table = info["table"]
    for pos, phys, off in rows:
        slot = opa.slot_of(table, pos, bs)
        assert (slot // bs, slot % bs) == (phys, off), (pos, slot)
    # gather through the figure's table returns the tokens in logical order
    nb = max(table) + 1
    pool = np.full((nb, bs, 2, 1, 1), -1.0, dtype=np.float16)
    for pos, phys, off in rows:
        pool[phys, off, 0, 0, 0] = pos
        pool[phys, off, 1, 0, 0] = 100 + pos
    K, V = opa.gather_kv(pool, table, info["num_tokens"])
    assert K[:, 0, 0].tolist() == list(range(info["num_tokens"]))
    assert V[:, 0, 0].tolist() == [100 + p for p in range(info["num_tokens"])]


def check_allocator_listing():
    path = os.path.join(GOLDEN, "allocator_listing.txt")
    alloc = None
    with open(path, encoding="utf-8") as f:
        lines = [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]
    nb = int(lines[0].split()[1])
    bs = int(lines[1].split()[1])
    alloc = opa.BlockAllocator(nb, bs)
    for ln in lines[2:]:
        left, free_after = ln.split(";")
        parts = left.split()
        seq, n, expect = parts[1], int(parts[2]), parts[4:]
        if expect == ["OOM"]:
            try:
                alloc.allocate(seq, n)
            except opa.KVCacheExhausted:
                pass
            else:
                raise AssertionError("allocation past the free list must raise")
        else:
            assert alloc.allocate(seq, n) == [int(x) for x in expect]
        fa = free_after.split()
        assert alloc.free_blocks == ([] if fa == ["-"] else [int(x) for x in fa])


def check_blocks_needed_closed_form():
    for bs in (1, 4, 16):
        for n in range(0, 200):
            assert opa.blocks_needed(n, bs) == math.ceil(n / bs)


# ---------------------------------------------------------------------------------------
# gather (block-table indexing)
# ---------------------------------------------------------------------------------------

def check_gather_matches_logical(inp):
    """PIN-1: every sequence's gathered K/V equal the values drawn before paging, bit for bit."""
    pool = opa.kv_append(inp.pool, inp.key_new, inp.value_new, inp.slot_mapping)
    for b in range(inp.num_seqs):
        L = int(inp.seq_lens[b])
        K, V = opa.gather_kv(pool, inp.block_tables[b], L)
        ref = inp.logical_kv[b]
        assert np.array_equal(K.view(np.uint16), ref[:, 0].view(np.uint16)), b
        assert np.array_equal(V.view(np.uint16), ref[:, 1].view(np.uint16)), b


# ---------------------------------------------------------------------------------------
# attention against a library routine and brute force
# ---------------------------------------------------------------------------------------

def sdpa_f64(q_rows, K, V, scale, mask=None, causal=False):
    """torch scaled_dot_product_attention in fp64 on CPU; q_rows [H, n, D], K/V [H, L, D]."""
    qt = torch.from_numpy(_f64(q_rows))
    kt = torch.from_numpy(_f64(K))
    vt = torch.from_numpy(_f64(V))
    m = None if mask is None else torch.from_numpy(mask)
    with torch.no_grad():
        out = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=m, is_causal=causal, scale=scale)
    return out.numpy()


def check_decode_vs_sdpa(inp, rtol=1e-12):
    """PIN-2: paged decode equals SDPA on the contiguous pre-paging tensors (KV heads expanded)."""
    pool = opa.kv_append(inp.pool, inp.key_new, inp.value_new, inp.slot_mapping)
    q, bt, lens = inp.decode_part()
    got = oracle.decode(q, pool, bt, lens, inp.scale)
    G = inp.num_q_heads // inp.num_kv_heads
    p = inp.num_prefill
    for i in range(q.shape[0]):
        kv = inp.logical_kv[p + i]
        K = np.repeat(kv[:, 0].transpose(1, 0, 2), G, axis=0)  # [Hq, L, D]
        V = np.repeat(kv[:, 1].transpose(1, 0, 2), G, axis=0)
        ref = sdpa_f64(q[i][:, None, :], K, V, inp.scale)[:, 0, :]
        err = np.abs(got[i] - ref).max()
        assert err <= rtol * max(1.0, np.abs(ref).max()), (i, err)


def brute_force_attention(q_row, K, V, scale):
    """Pure-Python softmax attention with math.exp, no NumPy arithmetic."""
    q_row = [float(x) for x in q_row]
    s = [scale * sum(qd * float(kd) for qd, kd in zip(q_row, k)) for k in K]
    mx = max(s)
    w = [math.exp(x - mx) for x in s]
    tot = sum(w)
    D = len(V[0])
    return [sum(w[t] * float(V[t][d]) for t in range(len(V))) / tot for d in range(D)]


def check_decode_vs_brute_force(inp, tol=1e-12):
    pool = opa.kv_append(inp.pool, inp.key_new, inp.value_new, inp.slot_mapping)
    q, bt, lens = inp.decode_part()
    got = oracle.decode(q, pool, bt, lens, inp.scale)
    G = inp.num_q_heads // inp.num_kv_heads
    p = inp.num_prefill
    for i in range(q.shape[0]):
        kv = inp.logical_kv[p + i]
        for h in range(inp.num_q_heads):
            ref = brute_force_attention(q[i, h], kv[:, 0, h // G], kv[:, 1, h // G], inp.scale)
            assert np.abs(got[i, h] - np.array(ref)).max() <= tol, (i, h)


def check_closed_forms():
    """L=1 gives V_0 exactly; q=0 gives the mean of V; one dominant key gives its V row."""
    inp = workloads.decode_case(11, [1, 7, 40], 2, 2, 16, append=False, keep_logical=True)
    # L = 1: p = 1, so the output is V_0 exactly
    out = oracle.decode(inp.q, inp.pool, inp.block_tables, inp.seq_lens, inp.scale)
    v0 = inp.logical_kv[0][0, 1].astype(np.float64)
    assert np.array_equal(out[0], v0)
    # q = 0: all scores equal, the output is the plain mean of V
    qz = np.zeros_like(inp.q)
    outz = oracle.decode(qz, inp.pool, inp.block_tables, inp.seq_lens, inp.scale)
    for b in range(inp.num_seqs):
        mean = inp.logical_kv[b][:, 1].astype(np.float64).mean(axis=0)  # [H, D]
        assert np.abs(outz[b] - mean).max() <= 1e-14
    # one key along q with a huge score: the output is that token's V row
    b, t_star = 2, 17
    pool = inp.pool.copy()
    phys, off = inp.block_tables[b][t_star // 16], t_star % 16
    for h in range(2):
        qh = inp.q[b, h].astype(np.float64)
        pool[phys, off, 0, h] = (qh * 40.0 / np.linalg.norm(qh)).astype(np.float16)
    out2 = oracle.decode(inp.q, pool, inp.block_tables, inp.seq_lens, 1.0)
    for h in range(2):
        assert np.abs(out2[b, h] - inp.logical_kv[b][t_star, 1, h].astype(np.float64)).max() < 1e-6


# ---------------------------------------------------------------------------------------
# paging invariants
# ---------------------------------------------------------------------------------------

def check_permutation_invariance(inp, seed=99, require_moved=True):
    """PIN-3: moving physical blocks (and rewriting the tables) changes nothing."""
    moved = workloads.repermute(inp, seed)
    a = opa.kv_append(inp.pool, inp.key_new, inp.value_new, inp.slot_mapping)
    b = opa.kv_append(moved.pool, moved.key_new, moved.value_new, moved.slot_mapping)
    qa, bta, la = inp.decode_part()
    qb, btb, lb = moved.decode_part()
    if require_moved:
        assert not np.array_equal(bta, btb)
    oa = oracle.decode(qa, a, bta, la, inp.scale)
    ob = oracle.decode(qb, b, btb, lb, moved.scale)
    assert np.array_equal(oa, ob)


def check_prefix_sharing(inp):
    """PIN-4: sequences sharing prefix blocks give the output of private copies."""
    priv = workloads.unshare_prefix(inp)
    assert len(np.unique(inp.block_tables[:, : inp.prefix_blocks])) < inp.num_seqs * inp.prefix_blocks
    assert len(np.unique(priv.block_tables[:, : inp.prefix_blocks])) == inp.num_seqs * inp.prefix_blocks
    a = oracle.decode(inp.q, inp.pool, inp.block_tables, inp.seq_lens, inp.scale)
    b = oracle.decode(priv.q, priv.pool, priv.block_tables, priv.seq_lens, priv.scale)
    assert np.array_equal(a, b)


def check_partitioned(inp, sizes=(16, 48, 512), rtol=1e-12):
    """PIN-6: partitions merged by log-sum-exp equal the direct softmax."""
    pool = opa.kv_append(inp.pool, inp.key_new, inp.value_new, inp.slot_mapping)
    q, bt, lens = inp.decode_part()
    ref = oracle.decode(q, pool, bt, lens, inp.scale)
    scale_ref = max(1.0, np.abs(ref).max())
    for ps in sizes:
        got = oracle.decode_partitioned(q, pool, bt, lens, inp.scale, ps)
        assert np.abs(got - ref).max() <= rtol * scale_ref, ps


def check_gqa_equals_mha(inp):
    """PIN-8: GQA equals MHA over a pool whose KV heads are each repeated G times."""
    G = inp.num_q_heads // inp.num_kv_heads
    assert G > 1
    pool = opa.kv_append(inp.pool, inp.key_new, inp.value_new, inp.slot_mapping)
    q, bt, lens = inp.decode_part()
    got = oracle.decode(q, pool, bt, lens, inp.scale)
    wide = np.repeat(pool, G, axis=3)
    ref = oracle.decode(q, wide, bt, lens, inp.scale)
    assert np.array_equal(got, ref)
    # and against SDPA with its own GQA broadcasting
    for i in range(q.shape[0]):
        kv = inp.logical_kv[inp.num_prefill + i]
        qt = torch.from_numpy(_f64(q[i][:, None, :]))
        kt = torch.from_numpy(_f64(kv[:, 0].transpose(1, 0, 2)))
        vt = torch.from_numpy(_f64(kv[:, 1].transpose(1, 0, 2)))
        with torch.no_grad():
            r = torch.nn.functional.scaled_dot_product_attention(
                qt, kt, vt, scale=inp.scale, enable_gqa=True).numpy()[:, 0]
        assert np.abs(r - got[i]).max() <= 1e-12 * max(1.0, np.abs(r).max())


# ---------------------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------------------

def check_prefill_vs_sdpa(inp, rtol=1e-12):
    """PIN-7: a chunk after P cached tokens equals SDPA with a bottom-right causal mask;
    with P = 0 it equals SDPA's own causal mode."""
    pool = opa.kv_append(inp.pool, inp.key_new, inp.value_new, inp.slot_mapping)
    q, bt, qsl, lens = inp.prefill_part()
    got = oracle.prefill_chunk(q, pool, bt, qsl, lens, inp.scale)
    G = inp.num_q_heads // inp.num_kv_heads
    for r in range(len(lens)):
        q0, q1 = int(qsl[r]), int(qsl[r + 1])
        C, S = q1 - q0, int(lens[r])
        P = S - C
        kv = inp.logical_kv[r]
        K = np.repeat(kv[:, 0].transpose(1, 0, 2), G, axis=0)
        V = np.repeat(kv[:, 1].transpose(1, 0, 2), G, axis=0)
        Q = q[q0:q1].transpose(1, 0, 2)  # [Hq, C, D]
        if P == 0:
            ref = sdpa_f64(Q, K, V, inp.scale, causal=True)
        else:
            mask = np.arange(S)[None, :] <= (P + np.arange(C))[:, None]
            ref = sdpa_f64(Q, K, V, inp.scale, mask=mask)
        ref = ref.transpose(1, 0, 2)
        err = np.abs(got[q0:q1] - ref).max()
        assert err <= rtol * max(1.0, np.abs(ref).max()), (r, err)


def check_prefill_row_is_decode(inp):
    """Chunk row i equals a decode query at position P+i over context P+i+1."""
    pool = opa.kv_append(inp.pool, inp.key_new, inp.value_new, inp.slot_mapping)
    q, bt, qsl, lens = inp.prefill_part()
    got = oracle.prefill_chunk(q, pool, bt, qsl, lens, inp.scale)
    for r in range(len(lens)):
        q0, q1 = int(qsl[r]), int(qsl[r + 1])
        P = int(lens[r]) - (q1 - q0)
        for i in range(q1 - q0):
            d = oracle.decode(q[q0 + i][None], pool, bt[r][None], np.array([P + i + 1]), inp.scale)
            assert np.array_equal(d[0], got[q0 + i]), (r, i)


def check_prefill_chunk_split(inp):
    """A chunk of C rows equals the same rows computed as two chunks of C/2 (same table)."""
    pool = opa.kv_append(inp.pool, inp.key_new, inp.value_new, inp.slot_mapping)
    q, bt, qsl, lens = inp.prefill_part()
    full = oracle.prefill_chunk(q, pool, bt, qsl, lens, inp.scale)
    for r in range(len(lens)):
        q0, q1 = int(qsl[r]), int(qsl[r + 1])
        C, S = q1 - q0, int(lens[r])
        h = C // 2
        qsl2 = np.array([0, h, C], dtype=np.int32)
        lens2 = np.array([S - (C - h), S], dtype=np.int32)
        bt2 = np.stack([bt[r], bt[r]])
        two = oracle.prefill_chunk(q[q0:q1], pool, bt2, qsl2, lens2, inp.scale)
        assert np.array_equal(two, full[q0:q1]), r


# ---------------------------------------------------------------------------------------
# kv_append
# ---------------------------------------------------------------------------------------

def check_kv_append(inp):
    """PIN-9: slots re-derived from the tables; the append writes those slots and nothing else."""
    slots = oracle.expected_slots(inp.block_tables, inp.seq_lens, inp.cached_lens, inp.block_size)
    assert np.array_equal(slots, inp.slot_mapping)
    out = opa.kv_append(inp.pool, inp.key_new, inp.value_new, inp.slot_mapping)
    bs = inp.block_size
    touched = np.zeros(inp.pool.shape[:2], dtype=bool)
    for t, s in enumerate(inp.slot_mapping):
        blk, off = s // bs, s % bs
        touched[blk, off] = True
        assert np.array_equal(out[blk, off, 0].view(np.uint16), inp.key_new[t].view(np.uint16))
        assert np.array_equal(out[blk, off, 1].view(np.uint16), inp.value_new[t].view(np.uint16))
    assert np.array_equal(out[~touched].view(np.uint16), inp.pool[~touched].view(np.uint16))


# ---------------------------------------------------------------------------------------
# block manager and block copies
# ---------------------------------------------------------------------------------------

BLOCK_TRACE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                           "block_manager_trace.txt")


def read_block_trace():
    """(num_blocks, block_size, [(op, args, result_tokens, checks)]) of the golden trace."""
    nb = bs = None
    steps = []
    for raw in open(BLOCK_TRACE, encoding="utf-8"):
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        if line.startswith("num_blocks"):
            nb = int(line.split()[1])
            continue
        if line.startswith("block_size"):
            bs = int(line.split()[1])
            continue
        lhs, rhs = line.split("->")
        parts = [p.strip() for p in rhs.split(";")]
        op, *args = lhs.split()
        steps.append((op, args, parts[0].split(), [p.split() for p in parts[1:]]))
    return nb, bs, steps


def run_block_trace(mgr, steps, exhausted=(opa.KVCacheExhausted,)):
    """Replay the golden trace on ``mgr`` (oracle.BlockManager or an object with the same
    methods and attributes ``free_list()``, ``refs_of(b)``, ``table_of(s)``, ``len_of(s)``)
    and assert every result and check."""
    for n, (op, args, res, checks) in enumerate(steps):
        where = f"trace step {n}: {op} {' '.join(args)}"
        try:
            if op == "allocate":
                got = ["table", *map(str, mgr.allocate(args[0], int(args[1])))]
            elif op == "fork":
                got = ["table", *map(str, mgr.fork(args[0], args[1]))]
            elif op == "append":
                slot, copy = mgr.append_token(args[0])
                got = ["slot", str(slot)] + ([] if copy is None else ["copy", str(copy[0]), str(copy[1])])
            elif op == "free":
                mgr.free(args[0])
                got = []
            else:
                raise AssertionError(f"unknown op {op}")
        except exhausted:
            got = ["OOM"]
        assert got == res, f"{where}: got {got}, want {res}"
        for c in checks:
            kind, vals = c[0], c[1:]
            if kind == "free":
                assert list(map(int, vals)) == list(mgr.free_list()), where
            elif kind == "table":
                assert list(map(int, vals[1:])) == list(mgr.table_of(vals[0])), where
            elif kind == "len":
                assert int(vals[1]) == mgr.len_of(vals[0]), where
            elif kind == "refs":
                for kv in vals:
                    b, cnt = map(int, kv.split(":"))
                    assert mgr.refs_of(b) == cnt, f"{where}: refs of {b}"
            elif kind == "usage":
                assert math.isclose(mgr.usage(), float(vals[0])), where
            elif kind == "utilisation":
                assert math.isclose(mgr.slot_utilisation(), float(vals[0])), where
            else:
                raise AssertionError(f"unknown check {kind}")


def oracle_manager(nb, bs):
    """oracle.BlockManager with the accessors the trace replay uses."""
    from oracle.block_manager import BlockManager

    m = BlockManager(nb, bs)
    m.free_list = lambda: list(m.free_blocks)
    m.refs_of = lambda b: m.refs[b]
    m.table_of = lambda s: list(m.tables[s])
    m.len_of = lambda s: m.lengths[s]
    return m


def check_block_manager_golden():
    nb, bs, steps = read_block_trace()
    run_block_trace(oracle_manager(nb, bs), steps)


def random_block_ops(seed, num_blocks, steps, block_size=16, forks=True):
    """A seeded op sequence over a small pool: allocate / append / fork / free."""
    rng = np.random.default_rng(seed)
    live, next_id, ops = [], 0, []
    for _ in range(steps):
        r = rng.random()
        if not live or r < 0.15:
            ops.append(("allocate", next_id, int(rng.integers(0, 3 * block_size))))
            live.append(next_id)
            next_id += 1
        elif forks and r < 0.25:
            ops.append(("fork", int(rng.choice(live)), next_id))
            live.append(next_id)
            next_id += 1
        elif r < 0.33:
            s = int(rng.choice(live))
            ops.append(("free", s))
            live.remove(s)
        else:
            ops.append(("append", int(rng.choice(live))))
    return ops


def apply_block_op(mgr, op, exhausted=(opa.KVCacheExhausted,)):
    """Run one op; returns its outcome (comparable across implementations). An op on a
    sequence that does not exist (its allocation ran out of blocks) is "invalid"."""
    try:
        if op[0] == "allocate":
            return ("table", tuple(mgr.allocate(op[1], op[2])))
        if op[0] == "fork":
            return ("table", tuple(mgr.fork(op[1], op[2])))
        if op[0] == "free":
            mgr.free(op[1])
            return ("freed",)
        slot, copy = mgr.append_token(op[1])
        return ("slot", slot, copy)
    except exhausted:
        return ("OOM",)
    except (KeyError, ValueError):
        return ("invalid",)


def check_block_manager_semantics(seed, num_blocks=24, steps=400, block_size=4):
    """Token-level meaning of tables, copies and slots: every sequence must read back
    exactly the tokens it was given (its parent's up to the fork, then its own), through
    its table, in a pool that applies each reported copy before the token is written.
    Also: reference counts equal the table references, free + referenced = all blocks,
    the slot written is never shared, table lengths are ceil(len / block_size)."""
    from oracle.block_manager import BlockManager, copy_blocks

    m = BlockManager(num_blocks, block_size)
    pool = np.full((num_blocks, block_size), -1, dtype=np.int64)  # token ids
    history = {}
    token = 0
    for op in random_block_ops(seed, num_blocks, steps, block_size):
        if op[0] != "allocate" and op[1] not in m.tables:
            continue  # its allocation ran out of blocks
        if op[0] == "allocate":
            try:
                table = m.allocate(op[1], op[2])
            except opa.KVCacheExhausted:
                continue
            history[op[1]] = list(range(token, token + op[2]))
            for pos, t in enumerate(history[op[1]]):
                pool[table[pos // block_size], pos % block_size] = t
            token += op[2]
        elif op[0] == "fork":
            m.fork(op[1], op[2])
            history[op[2]] = list(history[op[1]])
        elif op[0] == "free":
            m.free(op[1])
            del history[op[1]]
        else:
            try:
                slot, copy = m.append_token(op[1])
            except opa.KVCacheExhausted:
                continue
            if copy is not None:
                pool = copy_blocks(pool, [copy])
            blk = slot // block_size
            assert m.refs[blk] == 1, "appended into a shared block"
            pool[blk, slot % block_size] = token
            history[op[1]].append(token)
            token += 1
        counts = np.zeros(num_blocks, dtype=np.int64)
        for s, table in m.tables.items():
            assert len(table) == opa.blocks_needed(m.lengths[s], block_size)
            for b in table:
                counts[b] += 1
            got = [pool[table[p // block_size], p % block_size] for p in range(m.lengths[s])]
            assert got == history[s], f"sequence {s} reads wrong tokens"
        assert list(counts) == m.refs
        assert len(m.free_blocks) + int((counts > 0).sum()) == num_blocks
        assert all(counts[b] == 0 for b in m.free_blocks)


def check_block_manager_without_forks_is_the_listing(seed, num_blocks=64, steps=300):
    """With no forks, no frees and no exhaustion the manager hands out exactly the tables
    and slots of the listing's allocator (oracle.BlockAllocator)."""
    from oracle.block_manager import BlockManager

    m = BlockManager(num_blocks)
    a = opa.BlockAllocator(num_blocks)
    for op in random_block_ops(seed, num_blocks, steps, forks=False):
        if op[0] == "free":
            continue
        if op[0] == "allocate":
            need = opa.blocks_needed(op[2])
            if need > len(a.free_blocks):
                break
            assert m.allocate(op[1], op[2]) == a.allocate(op[1], op[2])
        else:
            t = a.block_tables[op[1]]
            if a.lengths[op[1]] == len(t) * 16 and not a.free_blocks:
                break
            slot, copy = m.append_token(op[1])
            assert copy is None and slot == a.append_token(op[1])


def check_block_copies():
    """copy_blocks / move_blocks against NumPy fancy indexing (disjoint pairs)."""
    from oracle.block_manager import copy_blocks, move_blocks

    rng = np.random.default_rng(3)
    pool = rng.standard_normal((12, 16, 2, 2, 8)).astype(np.float16)
    src = np.array([0, 5, 7]); dst = np.array([3, 9, 11])
    want = pool.copy()
    want[dst] = pool[src]
    got = copy_blocks(pool, np.stack([src, dst], 1))
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))
    host = np.zeros((6, 16, 2, 2, 8), np.float16)
    want_h = host.copy()
    want_h[[4, 0, 2]] = pool[[1, 6, 8]]
    got_h = move_blocks(host, pool, [[1, 4], [6, 0], [8, 2]])
    assert np.array_equal(got_h.view(np.uint16), want_h.view(np.uint16))
    # chained pairs apply in order: 0 -> 1, then 1 -> 2 carries block 0's contents
    chain = copy_blocks(pool, [[0, 1], [1, 2]])
    assert np.array_equal(chain[2].view(np.uint16), pool[0].view(np.uint16))
