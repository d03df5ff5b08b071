"""Pins for the oracle's prefix caching.

  * tests/golden/prefix_cache.json: the pages' block life cycle under prefix
    caching applied by hand to a small FIFO pool: hits by reference, the
    num_tokens - 1 cap, touch out of the free queue, cached-free blocks kept
    on release, atomic failure, eviction of the queue head's identity and a
    lookup that stops at the first missing block of the chain;
  * properties of the hash chain: equal prefixes give equal hashes, a change
    anywhere changes every later block's hash and none before, extra keys
    change all of them, a partial block has none, 32-byte SHA-256 digests
    (checked through hashlib on one block);
  * a content simulation over random admissions, cachings and releases:
    every hit returns blocks whose written tokens are exactly the requested
    prefix, blocks in use are never evicted or handed out twice, the free
    queue holds exactly the unreferenced blocks, and the map and the blocks'
    identities agree.
"""
import hashlib

import numpy as np
import pytest

from oracle.prefix_cache import NO_PARENT, CachedBlockPool, block_hashes


def test_prefix_cache_timeline(golden):
    g = golden("prefix_cache.json")
    pool = CachedBlockPool(g["num_blocks"], g["block_size"])
    tables, toks = {}, {}
    for st in g["steps"]:
        op = st["op"]
        if op == "admit":
            table, cached = pool.admit(st["tokens"])
            tables[st["rid"]], toks[st["rid"]] = table, st["tokens"]
            assert table == st["table"] and cached == st["cached_tokens"], st
            if "evicted_hash_of_block" in st:
                assert pool.hash_of[st["evicted_hash_of_block"]] is None
        elif op == "cache":
            pool.cache_full_blocks(tables[st["rid"]], toks[st["rid"]])
            for k, b in st["cached"].items():
                assert pool.block_of[block_hashes(toks[st["rid"]], 4)[int(k)]] == b
        elif op == "release":
            pool.release(tables.pop(st["rid"]))
        elif op == "admit_fails":
            before = (list(pool.free), list(pool.ref), dict(pool.block_of))
            with pytest.raises(MemoryError):
                pool.admit(list(range(1000, 1000 + st["tokens_count"])))
            assert before == (list(pool.free), list(pool.ref), dict(pool.block_of))
        elif op == "lookup":
            assert pool.longest_hit(block_hashes(st["tokens"], 4)) == st["hit"]
        if "free" in st:
            assert list(pool.free) == st["free"], st
        if "refs" in st:
            assert pool.ref == st["refs"], st


def test_hash_chain_properties():
    rng = np.random.default_rng(3)
    a = [int(x) for x in rng.integers(-2**31, 2**31, size=37)]
    h = block_hashes(a, 8)
    assert len(h) == 4 and all(len(x) == 32 for x in h)       # 37 // 8 full blocks
    assert h == block_hashes(a[:32], 8) == block_hashes(a + [5, 6], 8)[:4]
    # the first block is SHA-256 of (no parent, its tokens, no extra)
    first = NO_PARENT + b"".join(t.to_bytes(4, "little", signed=True) for t in a[:8])
    assert h[0] == hashlib.sha256(first).digest()
    for pos in (0, 9, 31):
        b = list(a)
        b[pos] ^= 1
        hb = block_hashes(b, 8)
        k = pos // 8
        assert hb[:k] == h[:k]                                # earlier blocks unchanged
        assert all(x != y for x, y in zip(hb[k:], h[k:]))     # this and every later one change
    he = block_hashes(a, 8, extra=b"lora-7")
    assert all(x != y for x, y in zip(he, h))
    # the same block content after different prefixes is a different block
    c = [1] * 8 + a[8:16]
    d = [2] * 8 + a[8:16]
    assert block_hashes(c, 8)[1] != block_hashes(d, 8)[1]
    assert block_hashes(a[:7], 8) == []


def _simulate(seed, pool_cls=CachedBlockPool):
    rng = np.random.default_rng(seed)
    B = int(rng.choice([1, 2, 4]))
    N = 24
    pool = pool_cls(N, B, rng.permutation(N).tolist())
    content = {}                      # block -> tokens written into it
    live = {}
    prompts = [[int(x) for x in rng.integers(0, 3, size=int(rng.integers(1, 6 * B)))]
               for _ in range(6)]
    for step in range(150):
        op = rng.choice(["admit", "admit", "release"])
        if op == "release" and live:
            rid = list(live)[int(rng.integers(len(live)))]
            pool.release(live.pop(rid)[0])
        else:
            base = prompts[int(rng.integers(len(prompts)))]
            toks = base[:int(rng.integers(1, len(base) + 1))] + \
                [int(x) for x in rng.integers(0, 3, size=int(rng.integers(0, 2 * B)))]
            try:
                table, cached = pool.admit(toks)
            except MemoryError:
                continue
            nb = cached // B
            for i, b in enumerate(table[:nb]):         # hits hold exactly these tokens
                assert content[b] == toks[i * B:(i + 1) * B], (step, b)
            for i, b in enumerate(table[nb:], start=nb):   # fresh blocks get new data
                content[b] = toks[i * B:(i + 1) * B]
            pool.cache_full_blocks(table, toks)
            live[step] = (table, toks)
        held = [0] * N
        for table, _ in live.values():
            for b in table:
                held[b] += 1
        assert held == pool.ref
        assert sorted(pool.free) == [b for b in range(N) if pool.ref[b] == 0]
        for h, b in pool.block_of.items():
            assert pool.hash_of[b] == h
        assert sum(h is not None for h in pool.hash_of) == len(pool.block_of)


@pytest.mark.parametrize("seed", range(20))
def test_prefix_cache_simulation(seed):
    _simulate(seed)


class _NoEviction(CachedBlockPool):
    def allocate(self, n):
        if n > len(self.free):
            raise MemoryError
        out = []
        for _ in range(n):
            b = self.free.popleft()
            self.ref[b] = 1
            out.append(b)
        return out


class _NoTouch(CachedBlockPool):
    def touch(self, blocks):
        for b in blocks:
            self.ref[b] += 1


def test_planted_mistakes_fail_the_simulation():
    for cls in (_NoEviction, _NoTouch):
        fails = 0
        for seed in range(10):
            try:
                _simulate(seed, cls)
            except (AssertionError, ValueError):
                fails += 1
        assert fails >= 3, cls
