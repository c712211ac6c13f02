"""Pool layout, scatter and block-table gather (oracle).

The pages fix only the storage model: the cache is cut into fixed-size blocks
of ``block_size`` token slots, placed anywhere in one physical pool, and a
per-sequence block table maps logical block j to a physical block id ("Paged
Attention Explained", "How Paged Attention Works", Steps 1 and 3; "PagedAttention:
paging the KV cache like an OS pages memory", "How it works").  Token position
p of a sequence therefore lives in physical block ``table[p // bs]`` at slot
``p % bs`` of that block.

Inside the pool the element order is this library's own choice; it is written
out here from its definition, independently of the device code:

  pool = [layer][block][kv_head][K, V][block_size x head_dim tile]

and each tile is a sequence of 16-token sub-tiles (token t of the block lies in
sub-tile t // 16 at row r = t % 16).  With E = 16 / elem_bytes elements per
16-byte chunk, element (r, d) of a sub-tile sits at

  K:  ((d // 4E) * 64 + r + 16 * ((d % 4E) // E)) * E + d % E
  V:  (((d // 16) // (E/4) * 64 + d % 16 + 16 * (r // 4)) * (E/4)
        + (d // 16) % (E/4)) * 4 + r % 4

(block_size a multiple of 16, head_dim a multiple of 4E).  The formula is a
bijection onto each tile; its only job is where bytes sit, so attention does
not depend on it.
"""
from __future__ import annotations

import numpy as np

ITEMSIZE = {"f32": 4, "f16": 2, "bf16": 2}


class Geometry:
    def __init__(self, num_layers, num_blocks, block_size, num_kv_heads, head_dim, dtype):
        self.L = int(num_layers)
        self.N = int(num_blocks)
        self.bs = int(block_size)
        self.H = int(num_kv_heads)
        self.D = int(head_dim)
        self.dtype = dtype
        self.E = 16 // ITEMSIZE[dtype]
        if self.bs % 16 or self.D % (4 * self.E) or self.bs <= 0 or self.D <= 0:
            raise ValueError("block_size must be a multiple of 16 and head_dim of 4*E")

    @property
    def num_elements(self) -> int:
        return 2 * self.L * self.N * self.bs * self.H * self.D


def element_index(g: Geometry, layer, block, head, kv, t, d):
    """Flat element index (int64, broadcasting) of element d of token slot t of
    physical block ``block``, kv head ``head``, tensor kv (0 = K, 1 = V)."""
    layer, block, head, kv, t, d = (np.asarray(a, dtype=np.int64) for a in (layer, block, head, kv, t, d))
    E, D, bs = g.E, g.D, g.bs
    region = ((layer * g.N + block) * g.H + head) * (2 * bs * D)
    sub, r = t // 16, t % 16
    base = region + kv * (bs * D) + sub * (16 * D)
    k_off = ((d // (4 * E)) * 64 + r + 16 * ((d % (4 * E)) // E)) * E + d % E
    R = E // 4
    nd = d // 16
    v_off = (((nd // R) * 64 + d % 16 + 16 * (r // 4)) * R + nd % R) * 4 + r % 4
    return base + np.where(kv == 0, k_off, v_off)


def token_indices(g: Geometry, layer: int, table_row: np.ndarray, ctx: int):
    """Element indices [ctx, H, D] of K and of V for positions 0..ctx-1 of a
    sequence whose block table row is ``table_row``."""
    p = np.arange(ctx, dtype=np.int64)
    blk = np.asarray(table_row, dtype=np.int64)[p // g.bs]
    if (blk < 0).any() or (blk >= g.N).any():
        raise ValueError("block table references an invalid block id")
    t = p % g.bs
    h = np.arange(g.H, dtype=np.int64)
    d = np.arange(g.D, dtype=np.int64)
    B, T = blk[:, None, None], t[:, None, None]
    Hh, Dd = h[None, :, None], d[None, None, :]
    ik = element_index(g, layer, B, Hh, 0, T, Dd)
    iv = element_index(g, layer, B, Hh, 1, T, Dd)
    return ik, iv


def scatter(pool: np.ndarray, g: Geometry, layer: int, table_row, K: np.ndarray, V: np.ndarray):
    """Write a sequence's logical K/V rows [ctx, H, D] into ``pool`` (flat)."""
    ik, iv = token_indices(g, layer, table_row, K.shape[0])
    pool[ik] = K
    pool[iv] = V


def gather(pool: np.ndarray, g: Geometry, layer: int, table_row, ctx: int):
    """Read a sequence's K/V rows [ctx, H, D] from ``pool`` through its table."""
    if ctx < 1:
        raise ValueError("context length must be at least 1")
    ik, iv = token_indices(g, layer, table_row, ctx)
    return pool[ik], pool[iv]


def slot_of(table_row, block_size: int, p: int) -> int:
    """Global slot number block*bs + offset of logical position p."""
    return int(table_row[p // block_size]) * block_size + p % block_size


def write_token(pool: np.ndarray, g: Geometry, layer: int, block: int, t: int,
                k_row: np.ndarray, v_row: np.ndarray):
    """Store one token's K/V rows [H, D] at slot t of physical block ``block``."""
    h = np.arange(g.H, dtype=np.int64)[:, None]
    d = np.arange(g.D, dtype=np.int64)[None, :]
    pool[element_index(g, layer, block, h, 0, t, d)] = k_row
    pool[element_index(g, layer, block, h, 1, t, d)] = v_row


def copy_block(pool: np.ndarray, g: Geometry, src: int, dst: int):
    """Copy every element (all layers, heads, K and V, all slots) of block src to dst."""
    L, H, kv, t, d = np.meshgrid(np.arange(g.L), np.arange(g.H), np.arange(2), np.arange(g.bs),
                                 np.arange(g.D), indexing="ij")
    pool[element_index(g, L, dst, H, kv, t, d)] = pool[element_index(g, L, src, H, kv, t, d)]
