"""The prefix-sharing fork/append script, run on the oracle side: the allocator
model decides placement and copies, and the oracle's own token write and block
copy build the expected pool."""
import numpy as np

import workloads as W
from oracle import layout as LY
from oracle.allocator import AllocatorModel


def oracle_shared_run(w: W.PagedWorkload, layer: int = 0, num_layers: int = 1):
    sc = w.script
    g = LY.Geometry(num_layers, w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.dtype)
    pool = np.full(g.num_elements, W.POISON_BITS[w.dtype], dtype=np.uint16)
    m = AllocatorModel(w.num_blocks, w.block_size, sc["free_order"])
    B, P, X = sc["branches"], sc["prefix"], sc["private"]
    bs = w.block_size
    copies = []
    for grp in range(sc["groups"]):
        s0 = m.create()
        assert s0 == grp * B
        slots, pairs = m.append(s0, P)
        assert not pairs
        pk, pv = W.shared_prefix_kv(w, grp)
        for p, slot in enumerate(slots):
            LY.write_token(pool, g, layer, slot // bs, slot % bs, pk[p], pv[p])
        for _ in range(B - 1):
            m.fork(s0)
    priv = {s: W.private_kv(w, s) for s in range(w.num_seqs)}
    for step in range(X):
        for s in range(w.num_seqs):
            slots, pairs = m.append(s, 1)
            for old, new in pairs:
                LY.copy_block(pool, g, old, new)
                copies.append((old, new))
            k, v = priv[s]
            LY.write_token(pool, g, layer, slots[0] // bs, slots[0] % bs, k[step], v[step])
    width = max(len(m.block_table(s)) for s in range(w.num_seqs))
    tables = np.full((w.num_seqs, width), -1, dtype=np.int32)
    for s in range(w.num_seqs):
        t = m.block_table(s)
        tables[s, :len(t)] = t
    ctx = np.array([m.length(s) for s in range(w.num_seqs)], dtype=np.int32)
    return g, pool, tables, ctx, m, copies
