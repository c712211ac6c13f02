"""Pins of the allocator model's host tier (swap out / swap in).

As for prefix caching, correctness is checked by simulation: device and host
slots record the token prefix their K/V would be a function of; swap pairs
copy whole blocks between the tiers; afterwards every resident sequence must
read its own prefixes through its device table and every swapped sequence
through its host table.  Also pinned: all-or-nothing failures, blocks shared
with another sequence staying on the device, released swapped sequences
returning their host blocks, and planted slips."""
import random

import pytest
from hypothesis import given, settings, strategies as st

from oracle.allocator import AllocatorModel, AllocError


class Sim:
    def __init__(self, N, bs, H, cache=False, order=None):
        self.m = AllocatorModel(N, bs, free_order=order)
        self.m.host_tier(H)
        if cache:
            self.m.enable_prefix_cache(True)
        self.bs = bs
        self.dev = {}   # device slot -> prefix
        self.host = {}  # host slot -> prefix
        self.toks = {}

    def new(self, ids):
        s = self.m.create()
        self.toks[s] = []
        self.add(s, ids)
        return s

    def add(self, s, ids):
        slots, pairs, n_cached = self.m.append_tokens(s, ids)
        for a, b in pairs:
            for t in range(self.bs):
                if a * self.bs + t in self.dev:
                    self.dev[b * self.bs + t] = self.dev[a * self.bs + t]
        full = self.toks[s] + list(ids)
        base = len(self.toks[s])
        for x, sl in enumerate(slots):
            if sl >= 0:
                self.dev[sl] = tuple(full[:base + x + 1])
        self.toks[s] = full

    def swap_out(self, s):
        pairs = self.m.swap_out(s)
        for b, hb in pairs:
            for t in range(self.bs):
                self.host[hb * self.bs + t] = self.dev.get(b * self.bs + t)
        return pairs

    def swap_in(self, s):
        pairs = self.m.swap_in(s)
        for hb, b in pairs:
            for t in range(self.bs):
                self.dev[b * self.bs + t] = self.host.get(hb * self.bs + t)
        return pairs

    def check(self):
        bs = self.bs
        used = 0
        for s, ids in self.toks.items():
            host = self.m.host_table(s)
            if host:
                used += len(host)
                assert self.m.block_table(s) == []
                for p in range(len(ids)):
                    assert self.host.get(host[p // bs] * bs + p % bs) == tuple(ids[:p + 1])
            else:
                tbl = self.m.block_table(s)
                for p in range(len(ids)):
                    assert self.dev.get(tbl[p // bs] * bs + p % bs) == tuple(ids[:p + 1])
        h_used, h_stack, _ = self.m.host_state()
        assert h_used == used
        assert sorted(h_stack + [hb for s in self.toks for hb in self.m.host_table(s)]) == list(range(self.m.host_n))
        rc, stack = self.m.state()
        refs = [0] * self.m.N
        for s in self.toks:
            for b in self.m.block_table(s):
                refs[b] += 1
        assert rc == refs


def test_swap_round_trip_moves_contents():
    sim = Sim(10, 4, 8)
    a = sim.new(list(range(10)))
    b = sim.new(list(range(100, 106)))
    pairs = sim.swap_out(a)
    assert [d for d, _ in pairs] == [0, 1, 2] and [h for _, h in pairs] == [0, 1, 2]
    assert sim.m.stats()["free_blocks"] == 10 - 2    # a's three blocks are free again
    c = sim.new(list(range(200, 212)))               # reuses them
    sim.check()
    back = sim.swap_in(a)
    assert [h for h, _ in back] == [0, 1, 2]
    assert sim.m.host_state()[0] == 0
    sim.add(a, [7, 7])                               # resident again: appends work
    sim.check()
    del b, c


def test_swapped_sequences_cannot_grow_or_fork_and_release_frees_host():
    sim = Sim(8, 4, 4)
    a = sim.new(list(range(6)))
    sim.swap_out(a)
    with pytest.raises(AllocError):
        sim.m.append(a, 1)
    with pytest.raises(AllocError):
        sim.m.fork(a)
    with pytest.raises(AllocError):
        sim.m.swap_out(a)
    sim.m.release(a)
    del sim.toks[a]
    assert sim.m.host_state() == (0, [3, 2, 0, 1], [])    # pushed back in logical order
    sim.check()


def test_shared_blocks_stay_on_the_device():
    sim = Sim(8, 4, 8)
    a = sim.new(list(range(8)))
    b_ = sim.m.fork(a)
    sim.toks[b_] = list(sim.toks[a])
    sim.swap_out(a)
    assert sim.m.state()[0][:2] == [1, 1]             # b still holds both blocks
    sim.check()
    sim.swap_in(a)
    sim.check()


def test_failures_change_nothing():
    sim = Sim(4, 4, 2)
    a = sim.new(list(range(12)))                      # 3 blocks, host has 2
    before = (sim.m.state(), sim.m.host_state(), sim.m.block_table(a))
    with pytest.raises(AllocError):
        sim.m.swap_out(a)
    assert (sim.m.state(), sim.m.host_state(), sim.m.block_table(a)) == before
    sim2 = Sim(3, 4, 4)
    x = sim2.new(list(range(8)))
    sim2.swap_out(x)
    y = sim2.new(list(range(50, 58)))                 # takes two of the three device blocks
    before = (sim2.m.state(), sim2.m.host_state())
    with pytest.raises(AllocError):
        sim2.m.swap_in(x)                             # needs two, one is free
    assert (sim2.m.state(), sim2.m.host_state()) == before
    del y


@settings(max_examples=60, deadline=None)
@given(st.integers(0, 10 ** 6), st.sampled_from([2, 4, 16]), st.integers(8, 40), st.booleans())
def test_random_scripts_keep_contents(seed, bs, N, cache):
    rng = random.Random(seed)
    sim = Sim(N, bs, N // 2 + 1, cache=cache, order=rng.sample(range(N), N))
    prompts = [[rng.randrange(3) for _ in range(rng.randint(bs, 4 * bs))] for _ in range(3)]
    live = []
    for _ in range(50):
        op = rng.random()
        try:
            if op < 0.3 or not live:
                p = rng.choice(prompts)
                live.append(sim.new(p[:rng.randint(1, len(p))]))
            elif op < 0.5:
                s = rng.choice(live)
                if not sim.m.host_table(s):
                    sim.add(s, [rng.randrange(3) for _ in range(rng.randint(1, bs + 2))])
            elif op < 0.65:
                s = rng.choice(live)
                if not sim.m.host_table(s):
                    sim.swap_out(s)
            elif op < 0.8:
                s = rng.choice(live)
                if sim.m.host_table(s):
                    sim.swap_in(s)
            elif op < 0.87:
                s = rng.choice(live)
                if not sim.m.host_table(s):
                    c = sim.m.fork(s)
                    sim.toks[c] = list(sim.toks[s])
                    live.append(c)
            else:
                s = live.pop(rng.randrange(len(live)))
                sim.m.release(s)
                del sim.toks[s]
        except AllocError as e:
            assert e.code == "OUT_OF_BLOCKS"
        sim.check()


def test_planted_slips_are_caught():
    # swap-in that forgets to copy one block
    caught = 0
    for slip in ("skip_copy", "free_shared"):
        sim = Sim(8, 4, 8)
        a = sim.new(list(range(8)))
        if slip == "skip_copy":
            pairs = sim.m.swap_out(a)
            for b, hb in pairs[:-1]:
                for t in range(4):
                    sim.host[hb * 4 + t] = sim.dev.get(b * 4 + t)
        else:
            b_ = sim.m.fork(a)
            sim.toks[b_] = list(sim.toks[a])
            sim.swap_out(a)
            sim.m.refcount[sim.m.block_table(b_)[0]] -= 1   # as if the shared block were freed
        try:
            sim.check()
        except AssertionError:
            caught += 1
    assert caught == 2
