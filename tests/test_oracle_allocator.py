"""Pins of the oracle's block allocator model (CPU only).

Pinned to the pages' worked examples (tests/golden/block_tables.json), the
block-count closed form ceil(n / 16), the capacity identity printed in the
vllm-musa startup log, the copy-on-write sequence of KVcache-learning s05,
and invariants checked after random op sequences.
"""
import json
import os

import pytest
from hypothesis import given, settings, strategies as st

from oracle.allocator_model import BlockManagerModel


def _golden(golden_dir):
    return json.load(open(os.path.join(golden_dir, "block_tables.json")))


def test_worked_block_table_jsqmd(golden_dir):
    g = _golden(golden_dir)["jsqmd_3_1"]
    phys = g["physical"]
    order = phys + [b for b in range(100) if b not in phys]
    m = BlockManagerModel(100, g["block_size"], order)
    n = sum(g["occupied"])                          # 16 + 16 + 8 = 40 tokens
    assert m.allocate(1, n) == ("ok", None)
    assert m.tables[1] == phys
    st_, slots = m.slots(1, 0, n)
    occupied = [sum(1 for s in slots if s // 16 == b) for b in phys]
    assert occupied == g["occupied"]
    m.check_invariants()


def test_worked_block_table_fairy2021(golden_dir):
    phys = _golden(golden_dir)["fairy2021_s05"]["physical"]
    m = BlockManagerModel(8, 16, phys + [0, 1, 2, 4, 6])
    assert m.allocate(0, 33)[0] == "ok"             # 3 logical blocks
    st_, rows, lens = m.export([0], 4)
    assert rows == [phys + [-1]] and lens == [33]


@pytest.mark.parametrize("n,blocks", [(0, 0), (1, 1), (15, 1), (16, 1), (17, 2), (32, 2),
                                      (33, 3), (4096, 256), (8193, 513)])
def test_block_count_is_ceil(n, blocks):
    m = BlockManagerModel(600, 16)
    assert m.allocate(0, n)[0] == "ok"
    assert len(m.tables[0]) == blocks
    assert len(m.free) == 600 - blocks


def test_capacity_identity_from_startup_log(golden_dir):
    g = _golden(golden_dir)["7yue_3_2"]
    N, bs, L = g["num_gpu_blocks"], g["block_size"], g["tokens_per_request"]
    assert N * bs / L == g["max_concurrency"]
    m = BlockManagerModel(N, bs)
    full = int(g["max_concurrency"])                # 48 whole requests fit
    for s in range(full):
        assert m.allocate(s, L)[0] == "ok"
    free_before = list(m.free)
    tables_before = {k: list(v) for k, v in m.tables.items()}
    assert m.allocate(full, L) == ("enomem", None)  # all-or-nothing: nothing taken
    assert list(m.free) == free_before and m.tables == tables_before
    assert len(m.free) == N - full * (L // bs)
    m.check_invariants()


def test_copy_on_write_sequence():
    """KVcache-learning s05: A and B share blocks; when A writes it copies the
    block, writes into the copy, repoints its table; B keeps the original."""
    m = BlockManagerModel(10, 16)
    assert m.allocate("A", 7)[0] == "ok"            # one partly filled block
    assert m.fork("A", "B") == "ok"
    shared = m.tables["A"][0]
    assert m.ref[shared] == 2
    st_, slot, pair = m.append("A")
    assert st_ == "ok" and pair == (shared, m.tables["A"][0]) and pair[1] != shared
    assert slot == pair[1] * 16 + 7                 # the new token goes into the copy
    assert m.tables["B"] == [shared] and m.ref[shared] == 1
    st_, slot_b, pair_b = m.append("B")              # B now owns the original alone
    assert pair_b is None and slot_b == shared * 16 + 7
    m.check_invariants()


def test_fork_of_full_blocks_needs_no_copy_and_free_order_is_fifo():
    m = BlockManagerModel(6, 16, [5, 4, 3, 2, 1, 0])
    m.allocate(1, 32)                               # blocks 5, 4 (full)
    m.fork(1, 2)
    st_, slot, pair = m.append(2)                    # new block, nothing shared is written
    assert pair is None and slot == 3 * 16
    m.release(1)                                    # 5, 4 still held by 2
    assert list(m.free) == [2, 1, 0]
    m.release(2)                                    # freed in logical order at the tail
    assert list(m.free) == [2, 1, 0, 5, 4, 3]
    m.check_invariants()


def test_error_statuses():
    m = BlockManagerModel(2, 16)
    assert m.append(9)[0] == "enoent"
    assert m.release(9) == "enoent"
    assert m.fork(9, 10) == "enoent"
    m.allocate(1, 5)
    assert m.fork(1, 1) == "eexist"
    assert m.slots(1, 0, 6)[0] == "einval"
    assert m.allocate(2, 33)[0] == "enomem"
    assert 2 not in m.tables


ops = st.lists(st.tuples(st.sampled_from(["alloc", "append", "fork", "free"]),
                         st.integers(0, 5), st.integers(0, 5), st.integers(0, 40)),
               max_size=60)


@settings(max_examples=300, deadline=None)
@given(ops)
def test_invariants_hold_under_random_ops(seq):
    m = BlockManagerModel(24, 16)
    for kind, a, b, n in seq:
        if kind == "alloc":
            m.allocate(a, m.lens.get(a, 0) + n)
        elif kind == "append":
            m.append(a)
        elif kind == "fork":
            m.fork(a, b)
        else:
            m.release(a)
        m.check_invariants()
