"""Reference model of the refcounted block allocator (oracle).

Mechanism from the pages:
  * blocks are handed out on demand: a sequence takes a new block only when
    its current last block is full ("Paged Attention Explained", "How Paged
    Attention Works", Step 2; "PagedAttention and KV Cache Compression", "Real-
    World Consequences: Zero Fragmentation");
  * finished sequences return their blocks to the pool (Step 5);
  * physical blocks are reference-counted and shared between sequences or
    decode branches; a shared block is copied, block by block, only when it must
    be modified ("PagedAttention: paging the KV cache like an OS pages memory",
    "How it works"; "PagedAttention and KV Cache Compression", glossary entry
    "Copy-on-Write").

Policy details the pages leave open (this library's reading):
  * free blocks form a LIFO stack; its initial pop order is given by the caller
    (``free_order[0]`` is handed out first), default ascending ids;
  * sequence ids are issued 0, 1, 2, ... and never reused;
  * ``fork`` copies the parent's table and length and increments each block's
    count in logical order;
  * ``append(n)`` first copies a shared, partially filled last block (at most
    one copy per call), then takes new blocks as positions cross block
    boundaries; every operation is all-or-nothing;
  * ``release`` walks the table in logical order, decrements, and pushes every
    block whose count reaches zero.
"""
from __future__ import annotations

from dataclasses import dataclass


class AllocError(Exception):
    def __init__(self, code: str, msg: str = ""):
        super().__init__(f"{code}: {msg}")
        self.code = code


INVALID_ARG = "INVALID_ARG"
OUT_OF_BLOCKS = "OUT_OF_BLOCKS"


@dataclass
class _Seq:
    table: list
    length: int


class AllocatorModel:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks < 0 or block_size <= 0:
            raise AllocError(INVALID_ARG, "bad pool geometry")
        self.N = num_blocks
        self.bs = block_size
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise AllocError(INVALID_ARG, "free order must be a permutation of the block ids")
        self.refcount = [0] * num_blocks
        self.stack = order[::-1]  # top of stack = end of list
        self.seqs: dict[int, _Seq] = {}
        self.next_id = 0
        self.cow_copies = 0

    # -- helpers ---------------------------------------------------------
    def _seq(self, sid) -> _Seq:
        if sid not in self.seqs:
            raise AllocError(INVALID_ARG, f"no live sequence {sid}")
        return self.seqs[sid]

    def _nblocks(self, n_tokens):
        return -(-n_tokens // self.bs)

    # -- operations ------------------------------------------------------
    def create(self) -> int:
        sid = self.next_id
        self.next_id += 1
        self.seqs[sid] = _Seq([], 0)
        return sid

    def append(self, sid: int, n_tokens: int):
        """Returns (slots, cow_pairs) for positions length .. length+n-1."""
        s = self._seq(sid)
        if n_tokens < 0:
            raise AllocError(INVALID_ARG, "token count cannot be negative")
        if n_tokens == 0:
            return [], []
        len0, len1 = s.length, s.length + n_tokens
        fresh = self._nblocks(len1) - self._nblocks(len0)
        cow = len0 % self.bs != 0 and self.refcount[s.table[-1]] > 1
        if fresh + int(cow) > len(self.stack):
            raise AllocError(OUT_OF_BLOCKS, "pool exhausted")
        pairs = []
        if cow:
            old = s.table[-1]
            new = self.stack.pop()
            self.refcount[old] -= 1
            self.refcount[new] = 1
            s.table[-1] = new
            pairs.append((old, new))
            self.cow_copies += 1
        for _ in range(fresh):
            b = self.stack.pop()
            self.refcount[b] = 1
            s.table.append(b)
        slots = [s.table[p // self.bs] * self.bs + p % self.bs for p in range(len0, len1)]
        s.length = len1
        return slots, pairs

    def fork(self, parent: int) -> int:
        p = self._seq(parent)
        for b in p.table:
            self.refcount[b] += 1
        cid = self.next_id
        self.next_id += 1
        self.seqs[cid] = _Seq(list(p.table), p.length)
        return cid

    def release(self, sid: int):
        s = self._seq(sid)
        for b in s.table:
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.stack.append(b)
        del self.seqs[sid]

    # -- state -----------------------------------------------------------
    def block_table(self, sid: int):
        return list(self._seq(sid).table)

    def length(self, sid: int) -> int:
        return self._seq(sid).length

    def state(self):
        """(refcounts, free stack bottom->top)."""
        return list(self.refcount), list(self.stack)

    def stats(self):
        live = self.seqs.values()
        return dict(
            num_blocks=self.N,
            free_blocks=len(self.stack),
            used_blocks=self.N - len(self.stack),
            shared_blocks=sum(1 for c in self.refcount if c > 1),
            cow_copies=self.cow_copies,
            live_seqs=len(self.seqs),
            logical_tokens=sum(s.length for s in live),
            tail_slots=sum(len(s.table) * self.bs - s.length for s in live),
        )
