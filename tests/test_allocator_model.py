"""Pins of the block-manager reference model (oracle/allocator_model.py).

The model is pinned to the pages' flowchart (a new block exactly when the
last one is full), the worked block-table example, copy-on-write semantics
and the bookkeeping invariants (refcounts equal table references, only the
last block of a sequence is partly filled, free + referenced = pool).
"""
import json
import os

import numpy as np
import pytest

from oracle.allocator_model import BlockManagerModel, NoBlocks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example_table_comes_from_the_free_order():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_block_table.json")))
    phys = ex["physical_blocks"]
    order = phys + [b for b in range(32) if b not in phys]
    m = BlockManagerModel(32, 16, order)
    m.add(0)
    slots = [m.append_slot(0)[0] for _ in range(40)]
    assert m.block_table(0) == phys
    assert slots[0] == 17 * 16 and slots[16] == 4 * 16 and slots[39] == 29 * 16 + 7
    m.check_invariants()


def test_flowchart_new_block_exactly_when_full():
    BS = 4
    m = BlockManagerModel(10, BS)
    m.add(1)
    for i in range(13):
        before = len(m.block_table(1))
        slot, cs, cd = m.append_slot(1)
        after = len(m.block_table(1))
        assert (after == before + 1) == (i % BS == 0)
        assert slot == m.block_table(1)[i // BS] * BS + i % BS
        assert (cs, cd) == (-1, -1)
    assert m.seq_len(1) == 13 and len(m.block_table(1)) == 4
    m.check_invariants()


def test_free_returns_blocks_and_leaves_other_tables_alone():
    m = BlockManagerModel(12, 4)
    for s in (0, 1, 2):
        m.add(s)
    for _ in range(9):
        for s in (0, 1, 2):
            m.append_slot(s)
    t0, t2 = m.block_table(0), m.block_table(2)
    free_before = m.num_free()
    freed = m.block_table(1)
    m.free(1)
    assert m.num_free() == free_before + len(freed)
    assert m.block_table(0) == t0 and m.block_table(2) == t2
    # LIFO: the next block handed out is the last one freed
    m.add(3)
    m.append_slot(3)
    assert m.block_table(3) == [freed[-1]]
    m.check_invariants()


def test_fork_shares_and_copy_on_write_copies_only_partial_shared_tails():
    BS = 4
    m = BlockManagerModel(16, BS, list(range(16)))
    m.add(0)
    for _ in range(6):  # blocks [0, 1], tail 1 half full
        m.append_slot(0)
    m.fork(0, 1)
    assert m.refcount(0) == 2 and m.refcount(1) == 2
    slot, cs, cd = m.append_slot(1)  # child writes into the shared partial tail
    assert (cs, cd) == (1, 2) and slot == 2 * BS + 2
    assert m.block_table(0) == [0, 1] and m.block_table(1) == [0, 2]
    assert m.refcount(1) == 1 and m.refcount(2) == 1 and m.refcount(0) == 2
    slot, cs, cd = m.append_slot(0)  # parent is now the last holder: in place
    assert (cs, cd) == (-1, -1) and slot == 1 * BS + 2
    m.check_invariants()


def test_full_shared_tail_gets_a_new_block_without_copy():
    BS = 4
    m = BlockManagerModel(8, BS, list(range(8)))
    m.add(0)
    for _ in range(8):
        m.append_slot(0)
    m.fork(0, 1)
    slot, cs, cd = m.append_slot(1)
    assert (cs, cd) == (-1, -1) and slot == 2 * BS
    assert m.block_table(1) == [0, 1, 2] and m.refcount(1) == 2
    m.check_invariants()


def test_out_of_blocks_leaves_state_unchanged():
    m = BlockManagerModel(2, 2, [0, 1])
    m.add(0)
    for _ in range(4):
        m.append_slot(0)
    m.fork(0, 1)
    snapshot = (m.block_table(0), m.block_table(1), m.seq_len(1), m.num_free())
    with pytest.raises(NoBlocks):
        m.append_slot(1)  # needs a fresh block, none left
    assert (m.block_table(0), m.block_table(1), m.seq_len(1), m.num_free()) == snapshot
    m.free(0)
    m.free(1)
    assert m.num_free() == 2
    m.check_invariants()


def test_unknown_and_duplicate_sequences_are_errors():
    m = BlockManagerModel(4, 4)
    m.add(0)
    with pytest.raises(KeyError):
        m.add(0)
    with pytest.raises(KeyError):
        m.append_slot(9)
    with pytest.raises(KeyError):
        m.fork(9, 10)
    with pytest.raises(KeyError):
        m.fork(0, 0)
    with pytest.raises(KeyError):
        m.free(9)


@pytest.mark.parametrize("seed", range(5))
def test_random_operation_sequences_keep_invariants(seed):
    rng = np.random.default_rng(seed)
    NB, BS = 64, 4
    m = BlockManagerModel(NB, BS, rng.permutation(NB).tolist())
    live, next_id = [], 0
    for _ in range(600):
        op = rng.integers(0, 10)
        if op == 0 or not live:
            m.add(next_id)
            live.append(next_id)
            next_id += 1
        elif op == 1:
            parent = live[rng.integers(len(live))]
            m.fork(parent, next_id)
            live.append(next_id)
            next_id += 1
        elif op == 2:
            s = live.pop(rng.integers(len(live)))
            m.free(s)
        else:
            s = live[rng.integers(len(live))]
            try:
                m.append_slot(s)
            except NoBlocks:
                pass
        m.check_invariants()
        # waste bound: only the last block of a sequence is partly filled
        for s in live:
            n = m.seq_len(s)
            assert len(m.block_table(s)) * BS - n < BS or n == 0


# ---------------------------------------------------------------------------- prefix cache
# Hand-worked scenarios with block size 4 and the identity free order (blocks
# are handed out 0, 1, 2, ...), following the readings in allocator_model.py.

def _prefill(m, seq, tokens):
    for _ in tokens:
        m.append_slot(seq)


def test_prefix_cache_hand_worked_sharing():
    m = BlockManagerModel(16, 4)
    a = [7, 7, 1, 2, 9, 9, 3, 4, 5, 6]          # 2 full blocks + 2 tokens
    m.add(1)
    _prefill(m, 1, a)                           # blocks 0, 1, 2
    assert m.block_table(1) == [0, 1, 2]
    assert m.register(1, a) == 2                # the two full blocks only
    assert m.num_cache_entries() == 2
    # same 8-token prefix, different tail: both blocks are adopted
    b = a[:8] + [11, 12, 13]
    assert m.match(b) == 8
    assert m.add_cached(2, b) == 8
    assert m.block_table(2) == [0, 1] and m.refcount(0) == 2 and m.refcount(1) == 2
    _prefill(m, 2, b[8:])                       # the suffix takes a new block (3)
    assert m.block_table(2) == [0, 1, 3] and m.seq_len(2) == 11
    m.check_invariants()


def test_prefix_cache_needs_one_token_left_and_exact_prefixes():
    m = BlockManagerModel(16, 4)
    a = list(range(12))                         # exactly 3 full blocks
    m.add(1)
    _prefill(m, 1, a)
    assert m.register(1, a) == 3
    assert m.match(a) == 8                      # the last token must be prefilled: 2 blocks
    assert m.match(a + [99]) == 12
    assert m.match(a[:4] + [0] + a[5:]) == 4    # differs in block 1: stops after block 0
    assert m.match([1] + a[1:]) == 0            # differs in block 0
    assert m.match(a, salt=5) == 0              # another configuration tag
    assert m.match(a[:3]) == 0                  # no full block
    m.check_invariants()


def test_prefix_cache_entries_live_while_blocks_are_referenced():
    m = BlockManagerModel(16, 4)
    a = list(range(9))
    m.add(1)
    _prefill(m, 1, a)
    m.register(1, a)
    m.fork(1, 2)                                # the sibling keeps the blocks alive
    m.free(1)
    assert m.num_cache_entries() == 2 and m.match(a) == 8
    m.free(2)                                   # last holder: blocks back to the pool
    assert m.num_cache_entries() == 0 and m.match(a) == 0
    m.check_invariants()


def test_prefix_cache_first_registration_wins():
    m = BlockManagerModel(16, 4)
    a = list(range(8)) + [50]
    m.add(1)
    _prefill(m, 1, a)                           # blocks 0, 1, 2
    m.add(2)
    _prefill(m, 2, a)                           # the same tokens computed again: 3, 4, 5
    assert m.register(1, a) == 2
    assert m.register(2, a) == 0                # keys already held by sequence 1's blocks
    m.add_cached(3, a)
    assert m.block_table(3) == [0, 1]
    m.free(1)                                   # block 2 returns; 0 and 1 stay with sequence 3
    assert m.match(a) == 8
    m.check_invariants()
