"""Seeded synthetic inputs for paged single-token decode.

This module only draws raw inputs: context lengths, physical block placement,
the query rows and each cached token's key/value rows, rounded to the storage
dtype.  It holds none of the method's arithmetic (no attention, no pool layout,
no slot translation) and is the one module that both the CPU oracle and the
HIP path take their inputs from.

Workloads (shapes from the pages' settings, values synthetic):
  * ``tiny``       4 sequences, lengths {7,16,33,50}, 4 heads, head_dim 64, fp32,
                   block_size 16, a 32-block pool.
  * ``opt13b``     OPT-13B-shaped MHA, fp16: 64 sequences, 40/40 heads, d=128,
                   lengths uniform in [128, 2048], pool exactly full.
  * ``llama3_8b``  Llama-3-8B-shaped GQA, bf16: 256 sequences, 32/8 heads, d=128,
                   lengths lognormal (median 1024, sigma 0.8) clipped to [16, 8192].
  * ``long_ctx``   long-context GQA, bf16: 8 sequences, 64/8 heads, d=128,
                   block_size 32, lengths uniform in [32768, 131072], K/V std 0.5,
                   512-token split-K partitions.
  * ``shared``     16 groups x 4 branches sharing a 2048-token prefix plus 256
                   private tokens per branch, 32/8 heads, bf16.
  * ``shared_cow`` the same with a 2040-token prefix, so the last shared block
                   is partial and the first append of a branch copies it.

Prefill workloads (new tokens appended to a sequence and attended causally):
  * ``prefill_tiny``       fp32, 4/2 heads, d=64: whole prompt, chunks, one token.
  * ``prefill_llama3_8b``  16 whole Llama-3-8B-shaped prompts, bf16, lengths from
                           the decode batch's lognormal.
  * ``chunked_llama3_8b``  64 sequences, lognormal cached context + 256 new tokens.
Their K/V rows are drawn per sequence exactly as for decode (the new tokens'
rows are the last ones); their query rows are drawn after the placement.

The pages' OPT-13B / Alpaca experiments are stood in for by these shapes only
(no trace and no weights are used).

Draw order for a paged workload with seed ``s`` (``rng = default_rng(s)``):
context lengths, then ``perm = rng.permutation(num_blocks)``, then q.  The
key/value rows of sequence ``i`` come from ``default_rng([s, 1, i])`` (K first,
then V), so any one sequence can be regenerated on its own.  Sequence ``i``'s
``j``-th logical block is ``perm[off_i + j]`` with ``off_i`` the running count of
blocks of the sequences before it.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import os

import numpy as np

DTYPES = ("f32", "f16", "bf16")
ITEMSIZE = {"f32": 4, "f16": 2, "bf16": 2}
# Quiet-NaN bit patterns used to poison pool memory that must never be read.
POISON_BITS = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0}


def storage_numpy_dtype(dtype: str):
    """numpy container for a storage dtype (bf16 is kept as its uint16 bits)."""
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 draws to the storage dtype with round-to-nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        b = x.view(np.uint32).astype(np.uint64)
        r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
        nan = np.isnan(x)
        if nan.any():
            r[nan] = POISON_BITS["bf16"]
        return r
    raise ValueError(f"unknown dtype {dtype}")


def _blocks_for(n_tokens: int, block_size: int) -> int:
    # Number of whole blocks a sequence occupies; needed to lay out the input
    # block tables (the same count any paged cache uses).
    return -(-int(n_tokens) // int(block_size))


@dataclass
class PagedWorkload:
    """One decode batch over a paged pool, as raw inputs."""

    name: str
    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    context_lens: np.ndarray  # int32 [S]
    block_tables: np.ndarray  # int32 [S, max_blocks], -1 padded
    q: np.ndarray  # storage dtype [S, Hq, D]
    scale: float
    partition_tokens: int
    kv_std: float
    seed: int
    num_layers: int = 1
    # shared-prefix workloads: description of the fork/append script
    script: dict | None = field(default=None)
    # prefill workloads: new tokens per sequence (the last query_lens[i] of its
    # context); q then holds their query rows, [sum(query_lens), Hq, D]
    query_lens: np.ndarray | None = field(default=None)

    @property
    def query_start(self) -> np.ndarray:
        """Offsets of each sequence's new tokens in q, int32 [S + 1]."""
        qs = np.zeros(self.num_seqs + 1, dtype=np.int32)
        qs[1:] = np.cumsum(self.query_lens)
        return qs

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max())

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max())

    @property
    def total_tokens(self) -> int:
        return int(self.context_lens.astype(np.int64).sum())

    def seq_kv(self, i: int):
        """Logical K and V rows of sequence i, each [ctx_i, Hkv, D], storage dtype."""
        if self.script is not None:
            return _shared_seq_kv(self, i)
        return _draw_kv(self.seed, i, int(self.context_lens[i]), self.num_kv_heads,
                        self.head_dim, self.kv_std, self.dtype)

    def all_kv(self, threads: int | None = None):
        """K and V of every sequence concatenated in sequence order, [sum ctx, Hkv, D]."""
        threads = threads or min(16, os.cpu_count() or 1)
        with ThreadPoolExecutor(threads) as ex:
            parts = list(ex.map(self.seq_kv, range(self.num_seqs)))
        k = np.concatenate([p[0] for p in parts], axis=0)
        v = np.concatenate([p[1] for p in parts], axis=0)
        return k, v


def _draw_kv(seed, i, n, hkv, d, std, dtype):
    rng = np.random.default_rng([int(seed), 1, int(i)])
    k = rng.standard_normal((n, hkv, d), dtype=np.float32)
    v = rng.standard_normal((n, hkv, d), dtype=np.float32)
    if std != 1.0:
        k *= np.float32(std)
        v *= np.float32(std)
    return round_to_storage(k, dtype), round_to_storage(v, dtype)


def _place(ctx: np.ndarray, perm: np.ndarray, block_size: int, width: int | None = None):
    nb = [_blocks_for(c, block_size) for c in ctx]
    width = width or max(nb)
    tables = np.full((len(ctx), width), -1, dtype=np.int32)
    off = 0
    for i, n in enumerate(nb):
        tables[i, :n] = perm[off:off + n]
        off += n
    return tables


def _paged(name, seed, dtype, ctx, hq, hkv, d, bs, num_blocks, kv_std, partition_tokens,
           rng, width=None, scale=None):
    ctx = np.asarray(ctx, dtype=np.int32)
    perm = rng.permutation(num_blocks).astype(np.int32)
    tables = _place(ctx, perm, bs, width)
    q = round_to_storage(rng.standard_normal((len(ctx), hq, d), dtype=np.float32), dtype)
    scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else scale
    return PagedWorkload(name=name, dtype=dtype, num_seqs=len(ctx), num_q_heads=hq,
                         num_kv_heads=hkv, head_dim=d, block_size=bs, num_blocks=num_blocks,
                         context_lens=ctx, block_tables=tables, q=q, scale=scale,
                         partition_tokens=partition_tokens, kv_std=kv_std, seed=seed)


def tiny(seed: int = 1) -> PagedWorkload:
    rng = np.random.default_rng(seed)
    return _paged("tiny", seed, "f32", [7, 16, 33, 50], 4, 4, 64, 16, 32, 1.0, 0, rng)


def opt13b(seed: int = 2) -> PagedWorkload:
    rng = np.random.default_rng(seed)
    ctx = rng.integers(128, 2048, 64, endpoint=True)
    n = sum(_blocks_for(c, 16) for c in ctx)  # pool exactly full
    return _paged("opt13b", seed, "f16", ctx, 40, 40, 128, 16, n, 1.0, 0, rng,
                  width=2048 // 16)


def llama3_8b(seed: int = 3) -> PagedWorkload:
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(256)
    ctx = np.clip(np.rint(np.exp(np.log(1024.0) + 0.8 * z)), 16, 8192).astype(np.int64)
    n = sum(_blocks_for(c, 16) for c in ctx)
    return _paged("llama3_8b", seed, "bf16", ctx, 32, 8, 128, 16, n, 1.0, 0, rng,
                  width=8192 // 16)


def long_ctx(seed: int = 4) -> PagedWorkload:
    rng = np.random.default_rng(seed)
    ctx = rng.integers(32768, 131072, 8, endpoint=True)
    n = sum(_blocks_for(c, 32) for c in ctx)
    return _paged("long_ctx", seed, "bf16", ctx, 64, 8, 128, 32, n, 0.5, 512, rng,
                  width=131072 // 32)


def _shared(name, seed, prefix, private=256, groups=16, branches=4, hq=32, hkv=8, d=128, bs=16):
    """Fork/append script for prefix-sharing branches.

    Per group g: sequence ``4g`` receives the prefix, then ``branches - 1``
    children are forked from it; the ``private`` decode tokens are then appended
    one step at a time, every sequence in ascending id order per step.  The
    allocator hands out blocks in the order ``free_order``.
    """
    rng = np.random.default_rng(seed)
    S = groups * branches
    # pool large enough for the whole script, exactly full for the shared layout
    shared_full = prefix // bs
    per_branch = _blocks_for(prefix + private, bs) - shared_full
    num_blocks = groups * (shared_full + branches * per_branch)
    free_order = rng.permutation(num_blocks).astype(np.int32)
    q = round_to_storage(rng.standard_normal((S, hq, d), dtype=np.float32), "bf16")
    ctx = np.full(S, prefix + private, dtype=np.int32)
    script = dict(groups=groups, branches=branches, prefix=prefix, private=private,
                  free_order=free_order)
    return PagedWorkload(name=name, dtype="bf16", num_seqs=S, num_q_heads=hq, num_kv_heads=hkv,
                         head_dim=d, block_size=bs, num_blocks=num_blocks, context_lens=ctx,
                         block_tables=np.zeros((S, 0), dtype=np.int32), q=q,
                         scale=float(np.float32(1.0 / np.sqrt(d))), partition_tokens=0,
                         kv_std=1.0, seed=seed, script=script)


def shared_prefix_kv(w: PagedWorkload, group: int):
    """Prefix K/V of one group, [prefix, Hkv, D] each."""
    p = w.script["prefix"]
    return _draw_kv(w.seed, 100000 + group, p, w.num_kv_heads, w.head_dim, w.kv_std, w.dtype)


def private_kv(w: PagedWorkload, seq: int):
    """Private (appended) K/V of one branch, [private, Hkv, D] each."""
    n = w.script["private"]
    return _draw_kv(w.seed, 200000 + seq, n, w.num_kv_heads, w.head_dim, w.kv_std, w.dtype)


def _shared_seq_kv(w: PagedWorkload, i: int):
    g = i // w.script["branches"]
    pk, pv = shared_prefix_kv(w, g)
    xk, xv = private_kv(w, i)
    return np.concatenate([pk, xk]), np.concatenate([pv, xv])


def shared(seed: int = 5) -> PagedWorkload:
    return _shared("shared", seed, prefix=2048)


def shared_cow(seed: int = 6) -> PagedWorkload:
    return _shared("shared_cow", seed, prefix=2040)


def _prefill(name, seed, dtype, ctx, qlens, hq, hkv, d, bs, kv_std=1.0, width=None, extra_blocks=0):
    """Prefill batch: sequence i has a context of ctx[i] tokens whose last
    qlens[i] are new.  Draw order: perm, then the new tokens' query rows."""
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx, dtype=np.int32)
    qlens = np.asarray(qlens, dtype=np.int32)
    if ctx.shape != qlens.shape or np.any(qlens < 1) or np.any(qlens > ctx):
        raise ValueError("need 1 <= query_lens <= context_lens")
    n = sum(_blocks_for(c, bs) for c in ctx) + extra_blocks
    perm = rng.permutation(n).astype(np.int32)
    tables = _place(ctx, perm, bs, width)
    q = round_to_storage(rng.standard_normal((int(qlens.sum()), hq, d), dtype=np.float32), dtype)
    return PagedWorkload(name=name, dtype=dtype, num_seqs=len(ctx), num_q_heads=hq,
                         num_kv_heads=hkv, head_dim=d, block_size=bs, num_blocks=n,
                         context_lens=ctx, block_tables=tables, q=q,
                         scale=float(np.float32(1.0 / np.sqrt(d))), partition_tokens=0,
                         kv_std=kv_std, seed=seed, query_lens=qlens)


def _lognormal_lengths(rng, count, median=1024.0, sigma=0.8, lo=16, hi=8192):
    z = rng.standard_normal(count)
    return np.clip(np.rint(np.exp(np.log(median) + sigma * z)), lo, hi).astype(np.int64)


def prefill_tiny(seed: int = 7) -> PagedWorkload:
    """fp32, 4/2 heads, d=64: a whole 7-token prompt, chunks of 5 and 20 new
    tokens after cached ones, and a single new token."""
    return _prefill("prefill_tiny", seed, "f32", [7, 16, 33, 50], [7, 5, 1, 20], 4, 2, 64, 16,
                    extra_blocks=3)


def prefill_llama3_8b(seed: int = 8) -> PagedWorkload:
    """Llama-3-8B-shaped GQA prompts, bf16: 16 whole prompts whose lengths
    follow the decode batch's distribution (lognormal, median 1024, sigma 0.8,
    clipped to [16, 8192])."""
    rng = np.random.default_rng([seed, 0])
    ctx = _lognormal_lengths(rng, 16)
    return _prefill("prefill_llama3_8b", seed, "bf16", ctx, ctx, 32, 8, 128, 16, width=8192 // 16)


def chunked_llama3_8b(seed: int = 9) -> PagedWorkload:
    """Chunked prefill, Llama-3-8B-shaped GQA, bf16: 64 sequences, each with a
    cached context (lognormal, median 1024, sigma 0.8, clipped to [16, 8192])
    followed by a chunk of 256 new tokens."""
    rng = np.random.default_rng([seed, 0])
    ctx = _lognormal_lengths(rng, 64) + 256
    return _prefill("chunked_llama3_8b", seed, "bf16", ctx, np.full(64, 256), 32, 8, 128, 16,
                    width=(8192 + 256) // 16)


def custom_prefill(name: str, seed: int, dtype: str, ctx, qlens, hq: int, hkv: int, d: int,
                   bs: int, kv_std: float = 1.0, extra_blocks: int = 0) -> PagedWorkload:
    """A prefill workload of any shape."""
    return _prefill(name, seed, dtype, ctx, qlens, hq, hkv, d, bs, kv_std=kv_std,
                    extra_blocks=extra_blocks)


@dataclass
class PrefixWorkload:
    """Requests that share a system prompt: request r's tokens are the prompt's
    ids followed by its own question ids.  A token's K/V and query rows are a
    function of the request's tokens up to it, so the prompt's rows are drawn
    once and shared by every request, and each question's rows per request."""

    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    prompt_ids: np.ndarray          # int32 [P]
    question_ids: list              # int32 arrays, one per request
    scale: float
    seed: int
    kv_std: float = 1.0

    @property
    def num_requests(self) -> int:
        return len(self.question_ids)

    def request_ids(self, r: int) -> np.ndarray:
        return np.concatenate([self.prompt_ids, self.question_ids[r]]).astype(np.int32)

    def _rows(self, key, n, heads):
        rng = np.random.default_rng([int(self.seed)] + list(key))
        x = rng.standard_normal((n, heads, self.head_dim), dtype=np.float32)
        return x

    def prompt_kv(self):
        k = self._rows((2, 0), len(self.prompt_ids), self.num_kv_heads) * np.float32(self.kv_std)
        v = self._rows((2, 1), len(self.prompt_ids), self.num_kv_heads) * np.float32(self.kv_std)
        return round_to_storage(k, self.dtype), round_to_storage(v, self.dtype)

    def question_kv(self, r: int):
        n = len(self.question_ids[r])
        k = self._rows((3, r, 0), n, self.num_kv_heads) * np.float32(self.kv_std)
        v = self._rows((3, r, 1), n, self.num_kv_heads) * np.float32(self.kv_std)
        return round_to_storage(k, self.dtype), round_to_storage(v, self.dtype)

    def request_kv(self, r: int):
        pk, pv = self.prompt_kv()
        qk, qv = self.question_kv(r)
        return np.concatenate([pk, qk]), np.concatenate([pv, qv])

    def request_q(self, r: int):
        """Query rows of every token of request r, [P + Q_r, Hq, D]."""
        pq = self._rows((4,), len(self.prompt_ids), self.num_q_heads)
        qq = self._rows((5, r), len(self.question_ids[r]), self.num_q_heads)
        return round_to_storage(np.concatenate([pq, qq]), self.dtype)


def prefix_cache(seed: int = 10, requests: int = 64, prompt: int = 1024, dtype: str = "bf16",
                 hq: int = 32, hkv: int = 8, d: int = 128, bs: int = 16, q_lo: int = 64,
                 q_hi: int = 256) -> PrefixWorkload:
    """Llama-3-8B-shaped requests sharing a 1024-token system prompt, each with
    a question of uniform [64, 256] tokens (ids from a 128k vocabulary)."""
    rng = np.random.default_rng([seed, 0])
    prompt_ids = rng.integers(0, 128000, prompt).astype(np.int32)
    lens = rng.integers(q_lo, q_hi, requests, endpoint=True)
    qids = [rng.integers(0, 128000, int(n)).astype(np.int32) for n in lens]
    return PrefixWorkload(name="prefix_cache", dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                          head_dim=d, block_size=bs, prompt_ids=prompt_ids, question_ids=qids,
                          scale=float(np.float32(1.0 / np.sqrt(d))), seed=seed)


PREFILL_WORKLOADS = {
    "prefill_tiny": prefill_tiny,
    "prefill_llama3_8b": prefill_llama3_8b,
    "chunked_llama3_8b": chunked_llama3_8b,
}


WORKLOADS = {
    "tiny": tiny,
    "opt13b": opt13b,
    "llama3_8b": llama3_8b,
    "long_ctx": long_ctx,
    "shared": shared,
    "shared_cow": shared_cow,
}


def scaled_down(w: PagedWorkload, num_seqs: int, max_ctx: int, seed_offset: int = 1000) -> PagedWorkload:
    """A smaller workload of the same head shape, dtype and block size, for
    parity runs the oracle finishes in seconds.  Lengths are redrawn uniformly in
    [1, max_ctx] and the pool is exactly full."""
    seed = w.seed + seed_offset
    rng = np.random.default_rng(seed)
    ctx = rng.integers(1, max_ctx, num_seqs, endpoint=True)
    n = sum(_blocks_for(c, w.block_size) for c in ctx)
    return _paged(w.name + "_small", seed, w.dtype, ctx, w.num_q_heads, w.num_kv_heads,
                  w.head_dim, w.block_size, n, w.kv_std, w.partition_tokens, rng)


def custom(name: str, seed: int, dtype: str, ctx, hq: int, hkv: int, d: int, bs: int,
           kv_std: float = 1.0, partition_tokens: int = 0, extra_blocks: int = 0) -> PagedWorkload:
    """A paged workload of any shape; the pool holds the used blocks plus
    ``extra_blocks`` that no table references."""
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx, dtype=np.int64)
    n = sum(_blocks_for(c, bs) for c in ctx) + extra_blocks
    return _paged(name, seed, dtype, ctx, hq, hkv, d, bs, n, kv_std, partition_tokens, rng)
