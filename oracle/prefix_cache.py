"""Prefix caching on the block pool: the oracle's plain model.

TEST INFRASTRUCTURE ONLY: imported by tests/ and the CPU baseline leg of
bench.py, never by the library.

Sources (page titles as printed at the head of each page):
  * "vLLM PagedAttention: from fragmentation to slot mapping", block
    metadata and life cycle under prefix caching: a block carries a
    reference count and an optional cache identity (its hash). ref > 0: in
    use, never overwritten. ref = 0 with a hash: in the free queue, can be
    hit and can be evicted. ref = 0 without a hash: plainly free. A hit on a
    ref-0 cached block takes it out of the free queue (touch) and counts a
    reference; releasing to 0 appends it to the queue, hash kept; taking a
    block for new data evicts its identity (removed from the map, cleared).
    The free queue's head is the first reuse / eviction candidate.
  * "vLLM source walkthrough: PagedAttention and continuous batching",
    section 1.9: the block hash is SHA-256 over the block's token ids and
    extra keys (32 bytes); a new request looks its blocks up one by one and
    reuses the hits; the longest hit is capped at num_tokens - 1 (the last
    token is recomputed to get its logits); section 1.5: full blocks are
    added to the cache after allocation.

Reading taken where the pages are silent: a block's identity must cover its
whole prefix (the glossary-adjacent remark that an equal-looking string is
not enough to share blocks safely), so each block's hash message starts with
the previous block's hash (32 zero bytes before the first block), followed by
its token ids as little-endian int32 and the extra keys. A hash already
mapped to another block keeps that mapping (the first block cached with it).
"""
from __future__ import annotations

import hashlib
from collections import deque

HASH_BYTES = 32
NO_PARENT = bytes(HASH_BYTES)


def block_hashes(tokens, block_size: int, extra: bytes = b"") -> list:
    """Hashes of the full blocks of ``tokens`` (a trailing partial block has
    none)."""
    out = []
    parent = NO_PARENT
    for b in range(len(tokens) // block_size):
        chunk = tokens[b * block_size:(b + 1) * block_size]
        msg = parent + b"".join(int(t).to_bytes(4, "little", signed=True) for t in chunk) + extra
        parent = hashlib.sha256(msg).digest()
        out.append(parent)
    return out


class CachedBlockPool:
    """Blocks 0..N-1 with reference counts, a FIFO free queue (take from the
    head, return to the tail) and a hash -> block map."""

    def __init__(self, num_blocks: int, block_size: int, initial_free=None):
        self.block_size = block_size
        self.num_blocks = num_blocks
        order = list(range(num_blocks)) if initial_free is None else [int(b) for b in initial_free]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("initial_free must be a permutation of range(num_blocks)")
        self.free = deque(order)
        self.ref = [0] * num_blocks
        self.hash_of = [None] * num_blocks
        self.block_of = {}

    # -- queries -------------------------------------------------------------
    def longest_hit(self, hashes) -> list:
        """Blocks of the leading hashes that are cached, stopping at the
        first miss. No state changes."""
        out = []
        for h in hashes:
            b = self.block_of.get(bytes(h))
            if b is None:
                break
            out.append(b)
        return out

    def num_free(self) -> int:
        return len(self.free)

    # -- changes ---------------------------------------------------------------
    def touch(self, blocks) -> None:
        """One more reference on each block; a ref-0 block leaves the queue."""
        for b in blocks:
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1

    def allocate(self, n: int) -> list:
        """n blocks from the head of the free queue for new data; a cached
        one loses its identity. Atomic: too few free blocks -> MemoryError."""
        if n > len(self.free):
            raise MemoryError(f"need {n}, free {len(self.free)}")
        out = []
        for _ in range(n):
            b = self.free.popleft()
            h = self.hash_of[b]
            if h is not None:
                del self.block_of[h]
                self.hash_of[b] = None
            self.ref[b] = 1
            out.append(b)
        return out

    def cache(self, block: int, h: bytes) -> bool:
        """Give an in-use full block the identity h. False (no change) when
        h already names a block or the block already has an identity."""
        h = bytes(h)
        assert self.ref[block] > 0, "only blocks in use get an identity"
        if h in self.block_of or self.hash_of[block] is not None:
            return False
        self.block_of[h] = block
        self.hash_of[block] = h
        return True

    def release(self, blocks) -> None:
        """One reference less on each block, in order; at 0 a block goes to
        the tail of the queue and keeps its identity."""
        for b in blocks:
            assert self.ref[b] > 0, f"refcount underflow on block {b}"
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)

    # -- a request's admission, as the walkthrough page describes it -------------
    def admit(self, tokens, extra: bytes = b""):
        """Blocks for a request: the longest cached prefix (capped so that
        the last token is recomputed) by reference, the rest fresh. Returns
        (table, number of cached tokens)."""
        hashes = block_hashes(tokens, self.block_size, extra)
        cap = max(0, (len(tokens) - 1) // self.block_size)
        hit = self.longest_hit(hashes[:cap])
        need = -(-len(tokens) // self.block_size) - len(hit)
        revived = sum(1 for b in hit if self.ref[b] == 0)
        if need > len(self.free) - revived:
            raise MemoryError(f"need {need}, free {len(self.free) - revived}")
        self.touch(hit)
        table = hit + self.allocate(need)
        return table, len(hit) * self.block_size

    def cache_full_blocks(self, table, tokens, extra: bytes = b"") -> None:
        """After the request's K/V are written: its full blocks get their
        identities (first come keeps a shared hash)."""
        for b, h in zip(table, block_hashes(tokens, self.block_size, extra)):
            if self.hash_of[b] is None:
                self.cache(b, h)
