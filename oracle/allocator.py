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

Automatic prefix caching ("PagedAttention and KV Cache Compression", "What
Most People Miss": the engine fingerprints every block of prompt text and
points a request whose block matches to the existing block instead of
processing it again; "Paged Attention Explained", "Support for Prefix
Sharing").  This library's reading, off until enabled:
  * a block's identity is its token ids together with the identity of the
    block before it (its key: the parent's cache serial, 0 for a sequence's
    first block, and the block_size token ids), because a block's K/V depend
    on every earlier token; keys are compared exactly, the hash only finds
    them;
  * ``append_tokens(sid, ids)`` with the sequence at a block boundary looks
    the appended whole blocks up in order and stops at the first miss; every
    hit shares the cached block (count + 1, taken out of the free stack if it
    was free) and its tokens need neither a write nor attention (slot -1);
    hits are applied first, then copy-on-write, then fresh blocks;
  * a block is registered when it becomes full and all its token ids are
    known; if its key is already registered the existing entry stays and the
    sequence continues from that entry's serial;
  * a registered block popped from the free stack for new contents is
    evicted (unregistered); registered blocks released to count 0 go to the
    bottom of the free stack, so uncached free blocks are reused first and
    cached ones least recently freed first;
  * a plain ``append`` (token ids unknown) ends the sequence's chain: no
    further lookups or registrations for it; ``fork`` copies the chain state.

Swap to a host tier ("Paged Attention Explained", "Hybrid Memory Strategies":
cached data may move to another memory tier when GPU memory runs short, at a
transfer cost; "PagedAttention: paging the KV cache like an OS pages memory",
"Why an agent should care", names the swap/preemption policy).  This
library's reading:
  * the host tier is a set of host blocks, each holding one device block of
    every layer; its free blocks form a LIFO stack, initially ascending ids;
  * ``swap_out`` gives every block of the sequence's table, in logical order,
    the top host block, reports (device, host) pairs to copy, then releases
    the device blocks as ``release`` would; the sequence keeps its length and
    prefix-cache chain and becomes swapped (no append or fork until swapped
    in);
  * ``swap_in`` takes fresh device blocks (as an append would) in logical
    order, reports (host, device) pairs, and returns the host blocks to the
    host stack in logical order;
  * both are all-or-nothing; releasing a swapped sequence frees its host
    blocks.
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
    chain: bool = True    # every token id so far is known
    parent: int = 0       # cache serial of the last full block (0: none yet)
    tail: tuple = ()      # token ids of the partially filled last block
    host: list = None     # host blocks while swapped out (None: on the device)


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
        # prefix cache
        self.cache_on = False
        self.cache: dict[tuple, int] = {}   # (parent serial, token ids) -> block
        self.key_of: dict[int, tuple] = {}  # registered block -> key
        self.serial_of: dict[int, int] = {}  # registered block -> serial
        self.next_serial = 1
        self.cache_counts = dict(registered=0, hit_blocks=0, evicted=0, lookups=0)
        # host tier
        self.host_n = 0
        self.host_stack: list = []

    # -- helpers ---------------------------------------------------------
    def _seq(self, sid, swapped_ok=False) -> _Seq:
        if sid not in self.seqs:
            raise AllocError(INVALID_ARG, f"no live sequence {sid}")
        s = self.seqs[sid]
        if s.host is not None and not swapped_ok:
            raise AllocError(INVALID_ARG, f"sequence {sid} is swapped out")
        return s

    def _nblocks(self, n_tokens):
        return -(-n_tokens // self.bs)

    # -- operations ------------------------------------------------------
    def create(self) -> int:
        sid = self.next_id
        self.next_id += 1
        self.seqs[sid] = _Seq([], 0)
        return sid

    def _pop_fresh(self) -> int:
        """Top of the free stack for new contents; a registered block is evicted."""
        b = self.stack.pop()
        if b in self.key_of:
            del self.cache[self.key_of.pop(b)]
            del self.serial_of[b]
            self.cache_counts["evicted"] += 1
        return b

    def append(self, sid: int, n_tokens: int):
        """Returns (slots, cow_pairs) for positions length .. length+n-1."""
        s = self._seq(sid)
        if n_tokens < 0:
            raise AllocError(INVALID_ARG, "token count cannot be negative")
        if n_tokens == 0:
            return [], []
        slots, pairs, _ = self._append(s, n_tokens, None)
        return slots, pairs

    def append_tokens(self, sid: int, token_ids):
        """Append tokens given by id.  Returns (slots, cow_pairs, n_cached):
        slots of tokens served by cached blocks are -1."""
        s = self._seq(sid)
        ids = [int(t) for t in token_ids]
        if not ids:
            return [], [], 0
        return self._append(s, len(ids), ids)

    def _append(self, s: _Seq, n_tokens: int, ids):
        bs = self.bs
        len0, len1 = s.length, s.length + n_tokens
        known = ids is not None and self.cache_on and s.chain
        # lookups: whole blocks from a block boundary, up to the first miss
        hits = []
        lookups = 0
        parent = s.parent
        if known and len0 % bs == 0:
            for j in range(n_tokens // bs):
                key = (parent, tuple(ids[j * bs:(j + 1) * bs]))
                lookups += 1
                b = self.cache.get(key)
                if b is None:
                    break
                hits.append(b)
                parent = self.serial_of[b]
        free_hits = [b for b in hits if self.refcount[b] == 0]
        fresh = self._nblocks(len1) - self._nblocks(len0) - len(hits)
        cow = len0 % bs != 0 and self.refcount[s.table[-1]] > 1
        if fresh + int(cow) > len(self.stack) - len(free_hits):
            raise AllocError(OUT_OF_BLOCKS, "pool exhausted")
        self.cache_counts["lookups"] += lookups
        for b in hits:
            if self.refcount[b] == 0:
                self.stack.remove(b)
            self.refcount[b] += 1
            s.table.append(b)
        self.cache_counts["hit_blocks"] += len(hits)
        pairs = []
        if cow:
            old = s.table[-1]
            new = self._pop_fresh()
            self.refcount[old] -= 1
            self.refcount[new] = 1
            s.table[-1] = new
            pairs.append((old, new))
            self.cow_copies += 1
        for _ in range(fresh):
            b = self._pop_fresh()
            self.refcount[b] = 1
            s.table.append(b)
        n_cached = len(hits) * bs
        slots = [-1] * n_cached + [s.table[p // bs] * bs + p % bs for p in range(len0 + n_cached, len1)]
        s.length = len1
        # chain state and registration of blocks that became full
        if ids is None or not self.cache_on:
            s.chain = False
        if s.chain:
            s.parent = parent
            tail = list(s.tail)
            pos = len0 + n_cached
            for t in ids[n_cached:]:
                tail.append(t)
                pos += 1
                if pos % bs == 0:
                    b = s.table[pos // bs - 1]
                    key = (s.parent, tuple(tail))
                    if key in self.cache:
                        s.parent = self.serial_of[self.cache[key]]
                    else:
                        self.cache[key] = b
                        self.key_of[b] = key
                        self.serial_of[b] = self.next_serial
                        s.parent = self.next_serial
                        self.next_serial += 1
                        self.cache_counts["registered"] += 1
                    tail = []
            s.tail = tuple(tail)
        else:
            s.tail = ()
        return slots, pairs, n_cached

    def fork(self, parent: int) -> int:
        p = self._seq(parent)
        for b in p.table:
            self.refcount[b] += 1
        cid = self.next_id
        self.next_id += 1
        self.seqs[cid] = _Seq(list(p.table), p.length, p.chain, p.parent, p.tail)
        return cid

    def release(self, sid: int):
        s = self._seq(sid, swapped_ok=True)
        if s.host is not None:
            for hb in s.host:
                self.host_stack.append(hb)
            del self.seqs[sid]
            return
        self._free_device(s)
        del self.seqs[sid]

    def _free_device(self, s: _Seq):
        for b in s.table:
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                if self.cache_on and b in self.key_of:
                    self.stack.insert(0, b)  # cached: reused last
                else:
                    self.stack.append(b)

    # -- host tier -------------------------------------------------------
    def host_tier(self, num_host_blocks: int):
        """Set up (or resize, with nothing swapped) the host tier."""
        if num_host_blocks < 0:
            raise AllocError(INVALID_ARG, "negative host block count")
        if any(s.host is not None for s in self.seqs.values()):
            raise AllocError(INVALID_ARG, "sequences are swapped out")
        self.host_n = num_host_blocks
        self.host_stack = list(range(num_host_blocks))[::-1]

    def swap_out(self, sid: int):
        """(device, host) pairs to copy out, in logical order."""
        s = self._seq(sid)
        n = len(s.table)
        if n > len(self.host_stack):
            raise AllocError(OUT_OF_BLOCKS, "host tier exhausted")
        host = [self.host_stack.pop() for _ in range(n)]
        pairs = list(zip(s.table, host))
        self._free_device(s)
        s.table = []
        s.host = host
        return pairs

    def swap_in(self, sid: int):
        """(host, device) pairs to copy in, in logical order."""
        s = self._seq(sid, swapped_ok=True)
        if s.host is None:
            raise AllocError(INVALID_ARG, f"sequence {sid} is not swapped out")
        n = len(s.host)
        if n > len(self.stack):
            raise AllocError(OUT_OF_BLOCKS, "pool exhausted")
        table = []
        for _ in range(n):
            b = self._pop_fresh()
            self.refcount[b] = 1
            table.append(b)
        pairs = list(zip(s.host, table))
        for hb in s.host:
            self.host_stack.append(hb)
        s.table = table
        s.host = None
        return pairs

    def enable_prefix_cache(self, on: bool):
        """Turn prefix caching on or off; turning it off forgets every entry
        and ends every sequence's chain."""
        self.cache_on = bool(on)
        if not on:
            self.cache.clear()
            self.key_of.clear()
            self.serial_of.clear()
            for s in self.seqs.values():
                s.chain = False
                s.tail = ()

    def cache_stats(self):
        return dict(self.cache_counts, cached_blocks=len(self.cache))

    # -- state -----------------------------------------------------------
    def block_table(self, sid: int):
        s = self._seq(sid, swapped_ok=True)
        return list(s.table) if s.host is None else []

    def host_table(self, sid: int):
        s = self._seq(sid, swapped_ok=True)
        return list(s.host or [])

    def length(self, sid: int) -> int:
        return self._seq(sid, swapped_ok=True).length

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
            logical_tokens=sum(s.length for s in live if s.host is None),
            tail_slots=sum(len(s.table) * self.bs - s.length for s in live if s.host is None),
        )

    def host_state(self):
        """(host blocks in use, host free stack bottom->top, swapped sequences)."""
        used = self.host_n - len(self.host_stack)
        return used, list(self.host_stack), sorted(k for k, s in self.seqs.items() if s.host is not None)
