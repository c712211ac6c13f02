"""Host-to-device staging of decode inputs (plumbing around the C ABI).

Uploads numpy arrays in a storage dtype (bf16 as uint16 bits) to device
tensors, poisons a pool with quiet NaNs, and fills a pool with a batch's cached
tokens through pa_write_kv, with slots from the library's table translation.
Works with any batch object exposing ``num_seqs``, ``dtype``, ``block_size``,
``block_tables``, ``context_lens``, ``q`` and ``seq_kv(i)``.  Prefix-sharing
batches (``script`` set) are built through the library's block manager:
fork, append, copy-on-write copies and token writes, one decode step at a time.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from . import Pool, TORCH_DTYPE, slots_for_positions

BITS = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}
SIGNED_BITS = {"f32": np.int32, "f16": np.int16, "bf16": np.int16}
TORCH_BITS = {"f32": torch.int32, "f16": torch.int16, "bf16": torch.int16}
POISON_BITS = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0}


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    return np.ascontiguousarray(x).view(BITS[dtype])


def dev_tensor(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Storage-dtype numpy array -> device tensor of the matching torch dtype."""
    t = torch.from_numpy(np.ascontiguousarray(to_bits(x, dtype).view(SIGNED_BITS[dtype])))
    return t.to(device).view(TORCH_DTYPE[dtype])


def poison(pool: Pool):
    v = pool.buf.view(TORCH_BITS[pool.dtype])
    v.fill_(int(np.array(POISON_BITS[pool.dtype], dtype=BITS[pool.dtype]).view(SIGNED_BITS[pool.dtype])))


def make_pool(batch, layers: int = 1, free_order=None, device="cuda") -> Pool:
    pool = Pool(layers, batch.num_blocks, batch.block_size, batch.num_kv_heads, batch.head_dim,
                batch.dtype, free_order=free_order, device=device)
    poison(pool)
    return pool


def fill_pool(pool: Pool, batch, layer: int = 0, chunk_tokens: int = 1 << 22, tables=None,
              device="cuda"):
    """Write every cached token of the batch through pa_write_kv, in chunks of
    whole sequences."""
    tables = batch.block_tables if tables is None else tables
    ctx = batch.context_lens
    i = 0
    with ThreadPoolExecutor(16) as ex:
        while i < batch.num_seqs:
            j, n = i, 0
            while j < batch.num_seqs and (n == 0 or n + ctx[j] <= chunk_tokens):
                n += int(ctx[j])
                j += 1
            parts = list(ex.map(batch.seq_kv, range(i, j)))
            k = np.concatenate([p[0] for p in parts])
            v = np.concatenate([p[1] for p in parts])
            slots = slots_for_positions(tables[i:j], batch.block_size, np.zeros(j - i), ctx[i:j])
            pool.write_kv(layer, dev_tensor(k, batch.dtype, device), dev_tensor(v, batch.dtype, device),
                          torch.from_numpy(slots).to(device))
            del k, v, parts
            i = j
    torch.cuda.synchronize()


def device_inputs(batch, tables=None, ctx=None, device="cuda"):
    """(q, block_tables, context_lens) as device tensors."""
    tables = batch.block_tables if tables is None else tables
    ctx = batch.context_lens if ctx is None else ctx
    return (dev_tensor(batch.q, batch.dtype, device),
            torch.from_numpy(np.ascontiguousarray(tables, dtype=np.int32)).to(device),
            torch.from_numpy(np.ascontiguousarray(ctx, dtype=np.int32)).to(device))


def pool_bits(pool: Pool) -> np.ndarray:
    return pool.buf.view(TORCH_BITS[pool.dtype]).cpu().numpy().view(BITS[pool.dtype])


def contiguous_tables(batch) -> np.ndarray:
    """Block tables that place every sequence's blocks side by side in logical
    order (blocks 0.. for the first sequence, then the next, ...)."""
    bs = batch.block_size
    nb = [-(-int(c) // bs) for c in batch.context_lens]
    tables = np.full((batch.num_seqs, max(nb)), -1, dtype=np.int32)
    off = 0
    for i, n in enumerate(nb):
        tables[i, :n] = np.arange(off, off + n, dtype=np.int32)
        off += n
    return tables


def run_shared_script(pool: Pool, w, prefix_kv, private_kv, layers=(0,), device="cuda"):
    """Build a prefix-sharing batch in ``pool`` through the library's block
    manager: per group the prefix is appended to one sequence and written,
    then the other branches are forked from it; the private tokens are then
    appended one decode step at a time, every sequence in ascending id order,
    with the copy-on-write pairs of a step copied before its tokens are
    written.  Every listed layer receives the same tokens.  ``prefix_kv(w, g)``
    and ``private_kv(w, s)`` give a group's prefix rows and a sequence's
    private rows.  Returns the copy pairs in order."""
    sc = w.script
    B, P, X = sc["branches"], sc["prefix"], sc["private"]
    copies = []
    for grp in range(sc["groups"]):
        s0 = pool.seq_create()
        slots, pairs = pool.seq_append(s0, P)
        assert not pairs
        pk, pv = prefix_kv(w, grp)
        kd, vd = dev_tensor(pk, w.dtype, device), dev_tensor(pv, w.dtype, device)
        sd = torch.from_numpy(slots).to(device)
        for layer in layers:
            pool.write_kv(layer, kd, vd, sd)
        for _ in range(B - 1):
            pool.seq_fork(s0)
    priv = [private_kv(w, s) for s in range(w.num_seqs)]
    pk_all = np.stack([p[0] for p in priv], axis=1)  # [X, S, H, D]
    pv_all = np.stack([p[1] for p in priv], axis=1)
    for step in range(X):
        slots = np.empty(w.num_seqs, dtype=np.int32)
        step_pairs = []
        for s in range(w.num_seqs):
            sl, pairs = pool.seq_append(s, 1)
            slots[s] = sl[0]
            step_pairs += pairs
        if step_pairs:
            pool.copy_blocks(torch.tensor(step_pairs, dtype=torch.int32).to(device))
            copies += step_pairs
        kd = dev_tensor(pk_all[step], w.dtype, device)
        vd = dev_tensor(pv_all[step], w.dtype, device)
        sd = torch.from_numpy(slots).to(device)
        for layer in layers:
            pool.write_kv(layer, kd, vd, sd)
    torch.cuda.synchronize()
    return copies


def prefill_inputs(batch, tables=None, device="cuda"):
    """(q, query_start, block_tables, context_lens) of a prefill batch as
    device tensors."""
    tables = batch.block_tables if tables is None else tables
    return (dev_tensor(batch.q, batch.dtype, device),
            torch.from_numpy(np.ascontiguousarray(batch.query_start, dtype=np.int32)).to(device),
            torch.from_numpy(np.ascontiguousarray(tables, dtype=np.int32)).to(device),
            torch.from_numpy(np.ascontiguousarray(batch.context_lens, dtype=np.int32)).to(device))


def run_prefill_script(pool: Pool, batch, layer: int = 0, device="cuda"):
    """Build a prefill batch in ``pool`` through the library's block manager:
    per sequence, append the cached tokens and write them, then append the new
    tokens (one multi-token append each) and write them in one batched write
    for all sequences.  Returns the host block tables and context lengths."""
    seqs = []
    new_k, new_v, new_slots = [], [], []
    for i in range(batch.num_seqs):
        K, V = batch.seq_kv(i)
        c, n = int(batch.context_lens[i]), int(batch.query_lens[i])
        s = pool.seq_create()
        seqs.append(s)
        if c > n:
            slots, pairs = pool.seq_append(s, c - n)
            assert not pairs
            pool.write_kv(layer, dev_tensor(K[:c - n], batch.dtype, device),
                          dev_tensor(V[:c - n], batch.dtype, device), torch.from_numpy(slots).to(device))
        slots, pairs = pool.seq_append(s, n)
        assert not pairs
        new_k.append(K[c - n:])
        new_v.append(V[c - n:])
        new_slots.append(slots)
    pool.write_kv(layer, dev_tensor(np.concatenate(new_k), batch.dtype, device),
                  dev_tensor(np.concatenate(new_v), batch.dtype, device),
                  torch.from_numpy(np.concatenate(new_slots)).to(device))
    torch.cuda.synchronize()
    width = max(-(-int(c) // batch.block_size) for c in batch.context_lens)
    return pool.batch_tables(seqs, width)


def run_prefix_requests(pool: Pool, w, requests, layer: int = 0, device="cuda"):
    """Admit requests of a shared-prompt batch through the block manager's
    prefix cache: per request, one pa_seq_append_tokens of all its token ids,
    then one batched pa_write_kv of every token the cache did not serve.
    Returns [(sequence id, tokens served by the cache)] in request order."""
    out = []
    ks, vs, sl = [], [], []
    for r in requests:
        ids = w.request_ids(r)
        s = pool.seq_create()
        slots, pairs, n_cached = pool.seq_append_tokens(s, ids)
        assert not pairs
        k, v = w.request_kv(r)
        ks.append(k[n_cached:])
        vs.append(v[n_cached:])
        sl.append(slots[n_cached:])
        out.append((s, n_cached))
    if sum(len(x) for x in sl):
        pool.write_kv(layer, dev_tensor(np.concatenate(ks), w.dtype, device),
                      dev_tensor(np.concatenate(vs), w.dtype, device),
                      torch.from_numpy(np.concatenate(sl)).to(device))
    torch.cuda.synchronize()
    return out


def prefix_prefill_inputs(pool: Pool, w, admitted, requests, device="cuda"):
    """(q, query_start, block_tables, context_lens, max_query_len, max_context_len)
    for prefilling the tokens the cache did not serve, one sequence per request."""
    seqs = [s for s, _ in admitted]
    lens = [len(w.request_ids(r)) for r in requests]
    width = max(-(-n // w.block_size) for n in lens)
    tables, ctx = pool.batch_tables(seqs, width)
    qrows = [w.request_q(r)[nc:] for r, (_, nc) in zip(requests, admitted)]
    qs = np.zeros(len(seqs) + 1, dtype=np.int32)
    qs[1:] = np.cumsum([len(x) for x in qrows])
    return (dev_tensor(np.concatenate(qrows), w.dtype, device), torch.from_numpy(qs).to(device),
            torch.from_numpy(tables).to(device), torch.from_numpy(ctx).to(device),
            int(max(len(x) for x in qrows)), int(ctx.max()))
