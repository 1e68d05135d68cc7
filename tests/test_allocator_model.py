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
