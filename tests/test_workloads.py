"""The seeded input generator: determinism, recipe structure and the pages' limits (CPU only)."""

import ast
import os

import numpy as np

import workloads
from workloads.synth import POISON_F16

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _same(a, b):
    assert a.pool.shape == b.pool.shape
    assert np.array_equal(a.pool.view(np.uint16), b.pool.view(np.uint16))
    for f in ("block_tables", "seq_lens", "cached_lens", "slot_mapping", "query_start_loc"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    for f in ("q", "key_new", "value_new"):
        assert np.array_equal(getattr(a, f).view(np.uint16), getattr(b, f).view(np.uint16)), f


def test_deterministic_per_seed():
    _same(workloads.tiny_decode(), workloads.tiny_decode())
    a = workloads.mixed_case(3, [0, 40], [16, 20], [5, 70], 4, 2, 32)
    b = workloads.mixed_case(3, [0, 40], [16, 20], [5, 70], 4, 2, 32)
    _same(a, b)
    c = workloads.mixed_case(4, [0, 40], [16, 20], [5, 70], 4, 2, 32)
    assert not np.array_equal(a.q.view(np.uint16), c.q.view(np.uint16))


def test_keep_logical_does_not_change_values():
    a = workloads.decode_case(5, [3, 40, 1500], 4, 2, 16, keep_logical=False)
    b = workloads.decode_case(5, [3, 40, 1500], 4, 2, 16, keep_logical=True)
    _same(a, b)


def test_tiny_recipe():
    inp = workloads.tiny_decode()
    assert inp.pool.shape == (16, 16, 2, 4, 64)
    assert list(inp.seq_lens) == [1, 15, 16, 33]
    assert inp.scale == 1.0 / 8.0
    used = set()
    for b, L in enumerate(inp.seq_lens):
        nb = -(-int(L) // 16)
        used.update(int(x) for x in inp.block_tables[b, :nb])
        assert np.all(inp.block_tables[b, nb:] == inp.poison_block)
    assert len(used) == 6 and inp.poison_block not in used
    # the ten unused blocks hold nothing but NaN
    unused = [i for i in range(16) if i not in used]
    assert len(unused) == 10
    assert np.all(inp.pool[unused].view(np.uint16) == POISON_F16)
    # tail slots of partially filled blocks are NaN too
    last = inp.block_tables[3, 2]
    assert np.all(inp.pool[last, 1:].view(np.uint16) == POISON_F16)
    assert not np.any(np.isnan(inp.pool[last, 0]))


def test_new_token_slots_are_poisoned_before_append():
    inp = workloads.decode_case(6, [1, 17, 32, 33], 2, 2, 16)
    for s in inp.slot_mapping:
        assert np.all(inp.pool[s // 16, s % 16].view(np.uint16) == POISON_F16)
    assert len(np.unique(inp.slot_mapping)) == len(inp.slot_mapping)


def test_repermute_and_unshare_keep_values():
    inp = workloads.prefix_shared_case(7, 2, 3, 2, [1, 5, 16, 20, 3, 9], 4, 2, 16, keep_logical=True)
    moved = workloads.repermute(inp, 1)
    priv = workloads.unshare_prefix(inp)
    for variant in (moved, priv):
        for b in range(inp.num_seqs):
            L = int(inp.seq_lens[b])
            for pos in range(L):
                blk = variant.block_tables[b, pos // 16]
                assert np.array_equal(variant.pool[blk, pos % 16].view(np.uint16),
                                      inp.logical_kv[b][pos].view(np.uint16))


def test_prefix_groups_sharing_structure():
    inp = workloads.shared_prompt_groups()
    assert inp.num_q_heads == 32 and inp.num_kv_heads == 8 and inp.head_size == 128
    assert inp.num_seqs == 256
    for g in range(64):
        rows = inp.block_tables[4 * g: 4 * g + 4, :64]
        assert np.all(rows == rows[0])
    assert len(np.unique(inp.block_tables[:, :64])) == 64 * 64
    priv = inp.seq_lens - 1024
    assert priv.min() >= 64 and priv.max() <= 256


def test_mixed_fits_the_scheduler_limits():
    """The mixed step obeys the scheduler sketch's budget: 8192 tokens, 256 sequences
    (page "vLLM 部署深度指南", continuous-batching scheduler listing)."""
    inp = workloads.mixed_prefill_decode()
    assert inp.num_seqs <= 256
    tokens = int(inp.q_lens.sum())
    assert tokens == 8 * 512 + 248 <= 8192
    pri = inp.seq_lens[:8] - 512
    assert pri[0] == 0 and pri[7] == 3584 and pri.min() >= 0 and pri.max() <= 3584
    assert len(inp.slot_mapping) == 4344
    d = inp.seq_lens[8:]
    assert d.min() >= 256 and d.max() <= 4096


def test_long_prompt_workload_shape():
    """The long-prompt step: one 512-row chunk ending a 32768-token prompt (32256 tokens
    cached), 8 decodes U{256..4096}, 32 heads x 128; its 520 new tokens are appended."""
    inp = workloads.long_prompt_prefill()
    assert inp.num_prefill == 1 and inp.num_seqs == 9
    assert int(inp.seq_lens[0]) == 32768 and int(inp.q_lens[0]) == 512
    assert inp.num_q_heads == 32 and inp.num_kv_heads == 32 and inp.head_size == 128
    d = inp.seq_lens[1:]
    assert d.min() >= 256 and d.max() <= 4096 and np.all(inp.q_lens[1:] == 1)
    assert len(inp.slot_mapping) == 512 + 8
    assert inp.block_tables.shape[1] >= 32768 // 16


# ---------------------------------------------------------------------------------------
# independence of the oracle from the product path
# ---------------------------------------------------------------------------------------

def _imports(path):
    names = set()
    tree = ast.parse(open(path, encoding="utf-8").read())
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module:
            names.add(node.module.split(".")[0])
    return names


def _py_files(d):
    for dp, _, fs in os.walk(os.path.join(ROOT, d)):
        for f in fs:
            if f.endswith(".py"):
                yield os.path.join(dp, f)


def test_oracle_imports_nothing_of_the_product():
    for f in _py_files("oracle"):
        assert not (_imports(f) & {"paged_kv_cache_294_amd", "workloads", "torch"}), f


def test_product_and_generator_never_import_the_oracle():
    for d in ("paged_kv_cache_294_amd", "workloads"):
        for f in _py_files(d):
            assert "oracle" not in _imports(f), f
    for d in ("paged_kv_cache_294_amd",):
        for dp, _, fs in os.walk(os.path.join(ROOT, d)):
            for f in fs:
                if f.endswith((".hip", ".cpp", ".h")):
                    assert "oracle" not in open(os.path.join(dp, f), encoding="utf-8").read(), f
