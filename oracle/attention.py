"""Decode attention over a paged KV cache, float64 (oracle).

What is computed: for one new token per sequence, standard softmax attention
of each query head over that sequence's cached tokens -- paging changes only
where K/V are stored, not the result ("PagedAttention: paging the KV cache like
an OS pages memory", "How it works" and "Worked numbers"; "Paged Attention
Explained", "How Paged Attention Works", Step 4).  For query head g of a
sequence with context length T and kv head h(g):

    s_p = scale * <q_g, K[p, h(g)]>            p = 0 .. T-1
    m   = max_p s_p,   e_p = exp(s_p - m),   l = sum_p e_p
    o_g = sum_p e_p V[p, h(g)] / l

Grouped-query heads: query head g reads kv head g // (Hq / Hkv) (consecutive
grouping; the pages name only the KV head count as its own symbol, in the KV
memory estimate of "Why Does the KV Cache Consume So Much Memory?").

Long contexts are split into partitions whose partial softmax states are merged
by log-sum-exp weighting (``split_decode``); in exact arithmetic this equals the
unsplit result (the pages' FlashAttention comparison names online softmax as
the standard technique; the partition scheme itself is this library's).

Prefill of new tokens (``prefill_one``, ``paged_prefill``): a sequence whose
context of T tokens ends with n new tokens, already written to the cache,
attends from each new token to every cached token up to and including its own
position -- standard causal attention ("PagedAttention: paging the KV cache
like an OS pages memory", "How it works"; the blocks for the new tokens are
allocated first, "Paged Attention Explained", "How Paged Attention Works",
Step 2).  New token k (0-based) sits at position T - n + k.

The scale is taken as the float32 value the device receives.  Inputs arrive in
their storage dtype and are widened to float64 exactly.
"""
from __future__ import annotations

import numpy as np

from . import layout


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of storage values (bf16 given as uint16 bits) to float64."""
    if dtype == "bf16":
        return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype in ("f16", "f32"):
        return np.asarray(x).astype(np.float64)
    raise ValueError(dtype)


def decode_one(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Two-pass softmax attention of query rows q [Hq, D] over K, V [T, Hkv, D]."""
    Hq, D = q.shape
    T, Hkv, D2 = K.shape
    if T < 1:
        raise ValueError("softmax over an empty context is undefined")
    if D2 != D or V.shape != K.shape or Hq % Hkv:
        raise ValueError("shape mismatch")
    G = Hq // Hkv
    sigma = float(np.float32(scale))
    out = np.empty((Hq, D), dtype=np.float64)
    for g in range(Hq):
        h = g // G
        s = sigma * (K[:, h, :] @ q[g])
        m = s.max()
        e = np.exp(s - m)
        out[g] = (e @ V[:, h, :]) / e.sum()
    return out


def partition_state(q, K, V, scale):
    """Softmax state (m, l, o) of one partition: max score, sum of exp(s - m),
    normalised weighted V.  Shapes [Hq], [Hq], [Hq, D]."""
    Hq, D = q.shape
    G = Hq // K.shape[1]
    sigma = float(np.float32(scale))
    m = np.empty(Hq)
    l = np.empty(Hq)
    o = np.empty((Hq, D))
    for g in range(Hq):
        h = g // G
        s = sigma * (K[:, h, :] @ q[g])
        m[g] = s.max()
        e = np.exp(s - m[g])
        l[g] = e.sum()
        o[g] = (e @ V[:, h, :]) / l[g]
    return m, l, o


def lse_merge(ms, ls, os_):
    """Merge partition states: weight w_j = l_j exp(m_j - M), M = max_j m_j;
    out = sum_j w_j o_j / sum_j w_j."""
    ms = np.asarray(ms)
    ls = np.asarray(ls)
    os_ = np.asarray(os_)
    M = ms.max(axis=0)
    w = ls * np.exp(ms - M)
    return (w[..., None] * os_).sum(axis=0) / w.sum(axis=0)[..., None]


def split_decode(q, K, V, scale, partition_tokens: int):
    """Decode with the context cut into partitions of ``partition_tokens``."""
    T = K.shape[0]
    if T < 1 or partition_tokens < 1:
        raise ValueError("bad context or partition size")
    states = [partition_state(q, K[a:a + partition_tokens], V[a:a + partition_tokens], scale)
              for a in range(0, T, partition_tokens)]
    return lse_merge([s[0] for s in states], [s[1] for s in states], [s[2] for s in states])


def paged_decode(pool: np.ndarray, g: layout.Geometry, layer: int, q: np.ndarray,
                 block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
                 seqs=None) -> np.ndarray:
    """Outputs [len(seqs), Hq, D] (float64) for the listed sequences (all by
    default): gather each sequence's K/V through its table, then decode."""
    seqs = range(len(context_lens)) if seqs is None else seqs
    out = []
    for i in seqs:
        K, V = layout.gather(pool, g, layer, block_tables[i], int(context_lens[i]))
        out.append(decode_one(to_f64(q[i], g.dtype), to_f64(K, g.dtype), to_f64(V, g.dtype), scale))
    return np.stack(out)


def prefill_one(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, rows=None) -> np.ndarray:
    """Causal attention of the n newest tokens of a T-token context.

    q [n, Hq, D] are the new tokens' query rows; K, V [T, Hkv, D] hold every
    cached token, the new ones included.  Row k is at position T - n + k and
    attends to positions 0 .. T - n + k.  Returns [len(rows), Hq, D] for the
    listed rows (all by default)."""
    n = q.shape[0]
    T = K.shape[0]
    if n < 1 or n > T:
        raise ValueError("need 1 <= new tokens <= context length")
    rows = range(n) if rows is None else rows
    out = []
    for k in rows:
        pos = T - n + int(k)
        out.append(decode_one(q[k], K[:pos + 1], V[:pos + 1], scale))
    return np.stack(out)


def paged_prefill(pool: np.ndarray, g: layout.Geometry, layer: int, q: np.ndarray,
                  query_start: np.ndarray, block_tables: np.ndarray, context_lens: np.ndarray,
                  scale: float, seqs=None, rows=None) -> list:
    """Per listed sequence (all by default), the [n_i, Hq, D] float64 outputs of
    its new tokens q[query_start[i]:query_start[i+1]]: gather the sequence's
    K/V through its table, then ``prefill_one`` (optionally only ``rows[i]``)."""
    seqs = range(len(context_lens)) if seqs is None else seqs
    out = []
    for i in seqs:
        a, b = int(query_start[i]), int(query_start[i + 1])
        K, V = layout.gather(pool, g, layer, block_tables[i], int(context_lens[i]))
        r = None if rows is None else rows[i]
        out.append(prefill_one(to_f64(q[a:b], g.dtype), to_f64(K, g.dtype), to_f64(V, g.dtype),
                               scale, rows=r))
    return out
