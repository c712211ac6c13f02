"""Host-to-device staging of decode inputs (plumbing around the C ABI).

Uploads numpy arrays in a storage dtype (bf16 as uint16 bits) to device
tensors, poisons a pool with quiet NaNs, and fills a pool with a batch's cached
tokens through pa_write_kv, with slots from the library's table translation.
Works with any batch object exposing ``num_seqs``, ``dtype``, ``block_size``,
``block_tables``, ``context_lens``, ``q`` and ``seq_kv(i)``.
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
