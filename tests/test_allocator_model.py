"""Pins of the allocator model: the pages' block-count rule, on-demand growth,
release to the pool, copy-on-write only when a shared block is modified, and
conservation invariants under random operation scripts."""
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import workloads as W
from oracle import attention as A
from oracle import sizing as SZ
from oracle.allocator import AllocatorModel, AllocError, OUT_OF_BLOCKS, INVALID_ARG
from tests.shared_script import oracle_shared_run

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def check_invariants(m: AllocatorModel):
    rc, stack = m.state()
    referenced = [b for s in m.seqs.values() for b in s.table]
    # sum of counts = number of table entries
    assert sum(rc) == len(referenced)
    # free stack and referenced blocks partition the ids; count 0 <=> free
    assert len(set(stack)) == len(stack)
    assert set(stack) | set(referenced) == set(range(m.N))
    assert not (set(stack) & set(referenced))
    for b in range(m.N):
        assert (rc[b] == 0) == (b in set(stack))
    # every sequence holds exactly ceil(len / bs) blocks (block-count rule)
    for s in m.seqs.values():
        assert len(s.table) == SZ.blocks_required(s.length, m.bs)


def test_growth_matches_page_block_counts():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "block_counts.txt"))
            if l.strip() and not l.startswith("#")]
    m = AllocatorModel(64, 16)
    for tok, bs, blocks, unused in rows:
        s = m.create()
        # grow one token at a time: a new block only when the last one is full
        for _ in range(int(tok)):
            m.append(s, 1)
        assert len(m.block_table(s)) == int(blocks)
        assert len(m.block_table(s)) * 16 - m.length(s) == int(unused)
    check_invariants(m)
    assert m.stats()["tail_slots"] == sum(int(r[3]) for r in rows)


def test_slots_follow_tables_and_free_order():
    order = [5, 2, 7, 0, 1, 3, 4, 6]
    m = AllocatorModel(8, 16, order)
    s = m.create()
    slots, pairs = m.append(s, 40)
    assert m.block_table(s) == [5, 2, 7] and pairs == []
    assert slots[0] == 80 and slots[16] == 32 and slots[39] == 7 * 16 + 7


def test_release_returns_blocks_and_lifo_reuse():
    m = AllocatorModel(6, 16)
    a = m.create()
    m.append(a, 33)
    assert m.block_table(a) == [0, 1, 2]
    m.release(a)
    rc, stack = m.state()
    assert sum(rc) == 0 and stack[-3:] == [0, 1, 2]
    b = m.create()
    m.append(b, 1)
    assert m.block_table(b) == [2]   # last pushed is reused first
    check_invariants(m)


def test_out_of_blocks_is_all_or_nothing():
    m = AllocatorModel(3, 16)
    a = m.create()
    m.append(a, 20)
    before = (m.state(), m.block_table(a), m.length(a))
    with pytest.raises(AllocError) as e:
        m.append(a, 40)
    assert e.value.code == OUT_OF_BLOCKS
    assert (m.state(), m.block_table(a), m.length(a)) == before
    with pytest.raises(AllocError) as e:
        m.append(a, -1)
    assert e.value.code == INVALID_ARG
    with pytest.raises(AllocError):
        m.release(99)


def test_copy_on_write_only_when_shared_block_modified():
    m = AllocatorModel(16, 16)
    a = m.create()
    m.append(a, 20)               # blocks [0, 1], block 1 partial
    b = m.fork(a)
    c = m.fork(a)
    rc, _ = m.state()
    assert rc[0] == 3 and rc[1] == 3
    slots, pairs = m.append(b, 1)  # writes into shared partial block 1 -> copy
    assert pairs == [(1, 2)] and m.block_table(b) == [0, 2] and slots == [2 * 16 + 4]
    slots, pairs = m.append(c, 1)
    assert pairs == [(1, 3)]
    slots, pairs = m.append(a, 1)  # last holder writes in place
    assert pairs == [] and slots == [1 * 16 + 4]
    rc, _ = m.state()
    assert rc[0] == 3 and rc[1] == rc[2] == rc[3] == 1
    # a fork shares a's partial block again; a's next write copies it
    m.fork(a)
    _, pairs = m.append(a, 11)     # a: 32 tokens, both blocks full
    assert len(pairs) == 1 and m.stats()["cow_copies"] == 3
    # full shared block: appending starts a fresh block, no copy
    e = m.fork(a)
    _, pairs = m.append(e, 1)
    assert pairs == [] and m.stats()["cow_copies"] == 3
    check_invariants(m)


def test_slots_never_land_in_shared_blocks():
    rng = np.random.default_rng(3)
    m = AllocatorModel(200, 16)
    seqs = [m.create()]
    m.append(seqs[0], 37)
    for _ in range(300):
        op = rng.integers(3)
        if op == 0 and len(seqs) < 12:
            seqs.append(m.fork(seqs[rng.integers(len(seqs))]))
        else:
            s = seqs[rng.integers(len(seqs))]
            try:
                slots, _ = m.append(s, int(rng.integers(1, 5)))
            except AllocError:
                continue
            rc, _ = m.state()
            assert all(rc[x // 16] == 1 for x in slots)
    check_invariants(m)


ops = st.lists(st.tuples(st.sampled_from(["create", "append", "fork", "release"]),
                         st.integers(0, 7), st.integers(-1, 40)), min_size=1, max_size=60)


@settings(max_examples=150, deadline=None)
@given(ops, st.integers(0, 24), st.sampled_from([16, 32]))
def test_random_scripts_keep_invariants(script, nblocks, bs):
    m = AllocatorModel(nblocks, bs, list(np.random.default_rng(nblocks).permutation(nblocks)))
    live = []
    for op, who, n in script:
        snap = (m.state(), {k: (list(v.table), v.length) for k, v in m.seqs.items()})
        try:
            if op == "create":
                live.append(m.create())
            elif not live:
                continue
            elif op == "append":
                m.append(live[who % len(live)], n)
            elif op == "fork":
                live.append(m.fork(live[who % len(live)]))
            else:
                m.release(live.pop(who % len(live)))
        except AllocError as e:
            assert e.code in (OUT_OF_BLOCKS, INVALID_ARG)
            assert snap == (m.state(), {k: (list(v.table), v.length) for k, v in m.seqs.items()})
        check_invariants(m)


def test_shared_prefix_block_accounting():
    """Prefix sharing at 16 groups x 4 branches: a 2048-token prefix is whole
    blocks, so no copy fires; a 2040-token prefix leaves a partial shared block
    that the first three branches of each group copy."""
    for mk, copies, blocks in [(W.shared, 0, 3072), (W.shared_cow, 48, 3120)]:
        w = mk()
        g, pool, tables, ctx, m, cps = oracle_shared_run(w)
        assert len(cps) == copies and m.stats()["cow_copies"] == copies
        assert m.stats()["used_blocks"] == blocks == w.num_blocks
        unshared = sum(SZ.blocks_required(int(c), 16) for c in ctx)
        assert unshared == 64 * 144 if w.name == "shared" else True
        check_invariants(m)


def test_shared_pool_decodes_like_unshared_layout():
    """Attention through the shared tables equals attention over each branch's
    own logical tokens (sharing changes storage only)."""
    w = W.shared_cow()
    g, pool, tables, ctx, m, cps = oracle_shared_run(w)
    for s in [0, 1, 3, 61]:
        got = A.paged_decode(pool, g, 0, w.q, tables, ctx, w.scale, seqs=[s])[0]
        K, V = w.seq_kv(s)
        ref = A.decode_one(A.to_f64(w.q[s], "bf16"), A.to_f64(K, "bf16"), A.to_f64(V, "bf16"), w.scale)
        assert np.array_equal(got, ref)
